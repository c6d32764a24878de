// Fused backward of MiniMax Sparse Attention: main-branch gradients
// dQ, dK, dV and the index-branch KL-alignment gradients dq_idx, dk_idx.
//
// Pages: "How FlashAttention cuts GPU memory traffic without approximation",
// 'Training and the backward pass' (probabilities rebuilt from the stored
// row log-sum-exp; dV += P^T dO and dP = dO V^T per tile); "How Flash-MSA
// cuts million-token training cost with sparse-k", 'Kernel design and
// execution' (backward of the proxy and main attention fused in one pass,
// since the proxy's signal needs both distributions; the inverted block map
// schedules the queries of each KV block so the block is reused on chip) and
// 'Removing the KL-divergence bottleneck' (the gradient with respect to a
// proxy score is the proxy probability minus the main probability, so no KL
// distribution is materialised); "How to solve the memory problem with
// MiniMax Sparse Attention", 'Training sparse attention' (the teacher is the
// main softmax averaged over the group's heads; no KL gradient reaches the
// backbone).
//
// Passes:
//   bwd_rowdot_kernel    D[b,t,h] = sum_c dO * O
//   idx_lse_kernel       per (KV block, selecting queries): log-sum-exp of
//                        the index logits over the block (KV-outer, MFMA)
//   idx_lse_merge_kernel lse_idx[b,t,g] over the selected support
//   bwd_main16_kernel    per query chunk and work item (KV block j of group g,
//                        its own queries and up to 1024-4096 list entries,
//                        chosen per launch): 8 waves
//                        of 16 keys keep dK, dV, dk_idx in registers; per 32
//                        (query, head) rows they rebuild S and P, dP, dS, the
//                        index logits, p_px, the head-averaged teacher pbar and
//                        dz = lam (p_px - pbar); dS and dz go through LDS to
//                        form dQ = dS K (stored as a bf16 partial per selected
//                        block) and dq_idx = dz K_idx (fp32 atomics); the
//                        block's dK, dV, dk_idx are added once per item.
//   dq_merge_kernel      dq = sum of a row's partials over its valid slots
//   f32_to_bf16_kernel   fp32 accumulators -> bf16 dk, dv.
#include "msa_internal.h"

#include <type_traits>

namespace msa {
namespace {

// List entries per work item of the index log-sum-exp pass (its diagonal
// items hold the block's own 128 queries).
constexpr int kLseItem = 512;

// ---------------------------------------------------------------------------
// D = rowsum(dO * O)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const bf16* __restrict__ dO, const bf16* __restrict__ O,
                                                         float* __restrict__ Dv, size_t rows) {
  constexpr int LPR = D / 8;
  const size_t row = (size_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(dO + row * D + part * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(O + row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += (float)a[i] * (float)b[i];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) Dv[row] = acc;
}

// ---------------------------------------------------------------------------
// Work-item decode shared by the KV-outer kernels of this file.
// ---------------------------------------------------------------------------
struct Item {
  int b, g, j, nq;
  bool diag;
  const int32_t* ent;
};

__device__ inline bool decode_item(const int32_t* __restrict__ tiles, const int32_t* __restrict__ pos,
                                   const int32_t* __restrict__ offs, const int32_t* __restrict__ rows,
                                   int n_lists, int N, int H_kv, int topk, int nblk, int nsb, Item* it) {
  const int w = xcd_item(tiles[n_lists]);
  if (w < 0) return false;
  int lo = 0, hi = n_lists - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tiles[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int local = w - tiles[lo];
  it->j = lo % nblk;
  const int bg = lo / nblk;
  it->g = bg % H_kv;
  it->b = bg / H_kv;
  it->diag = local == 0;   // the whole sequence is one range: every list has its diagonal item
  it->nq = kBlock;
  it->ent = nullptr;
  if (!it->diag) {
    const int32_t* pb = pos + (size_t)bg * (nsb + 1) * nblk + it->j;
    const int seg1 = pb[(size_t)nsb * nblk];
    const int e0 = (local - 1) * kLseItem;
    it->nq = min(kLseItem, seg1 - e0);
    it->ent = rows + (size_t)bg * N * topk + offs[(size_t)bg * (nblk + 1) + it->j] + e0;
  }
  return true;
}

// The item's queries, staged in LDS once per item: (t << 6) | slot, or -1
// for an entry outside the sequence (a well-formed map never has one; it is
// dropped rather than trusted).  The diagonal item looks up each own query's
// slot in its selection here.
__device__ inline void stage_item_queries(const Item& it, const int32_t* __restrict__ block_idx, int N, int H_kv,
                                          int topk, int* qent) {
  for (int i = threadIdx.x; i < it.nq; i += blockDim.x) {
    int t, slot = 0;
    if (it.diag) {
      t = it.j * kBlock + i;
      const int32_t* brow = block_idx + (((size_t)it.b * N + t) * H_kv + it.g) * topk;
      for (int e = 0; e < topk; ++e)
        if (brow[e] == it.j) slot = e;
    } else {
      const int e = it.ent[i];
      t = e >> 6;
      slot = e & 63;
    }
    qent[i] = (t < 0 || t >= N || slot >= topk) ? -1 : ((t << 6) | slot);
  }
}

// ---------------------------------------------------------------------------
// Index log-sum-exp over the selected support, per (b, t, g): KV-outer
// partials (max, sum) per slot, then a merge.
// ---------------------------------------------------------------------------
template <int DIDX>
__global__ __launch_bounds__(256, 4) void idx_lse_kernel(
    const bf16* __restrict__ q_idx, const bf16* __restrict__ k_idx, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ offs, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ tiles, float2* __restrict__ part, int N, int H_kv, int topk, int causal,
    int nblk, int nsb, int n_lists, float scale_idx) {
  constexpr int PK = DIDX + 8;
  constexpr int KSTEPS = DIDX / 16;
  __shared__ __align__(16) bf16 Ks[kBlock * PK];
  __shared__ int qent[kLseItem > kBlock ? kLseItem : kBlock];
  Item it;
  if (!decode_item(tiles, pos, offs, rows, n_lists, N, H_kv, topk, nblk, nsb, &it)) return;
  stage_item_queries(it, block_idx, N, H_kv, topk, qent);
  {
    const bf16* src = k_idx + ((size_t)it.b * N + (size_t)it.j * kBlock) * DIDX;
    constexpr int CPR = DIDX / 8;
    for (int c = threadIdx.x; c < kBlock * CPR; c += 256) {
      const int key = c / CPR, col = c % CPR;
      *reinterpret_cast<uint4*>(Ks + key * PK + col * 8) =
          *reinterpret_cast<const uint4*>(src + (size_t)key * DIDX + col * 8);
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Query tiles of 32: wave w takes tiles w, w + 4, ...; a tile's query ids
  // (from LDS) and q_idx rows are fetched while the previous tile computes.
  int tile = wave;
  if (tile * 32 >= it.nq) return;
  int t, slot;
  bool valid;
  bf16x8 qn[KSTEPS];
  auto fetch = [&](int tl) {
    const int qi = tl * 32 + (lane & 31);
    const int e = qent[min(qi, it.nq - 1)];
    valid = qi < it.nq && e >= 0;
    t = e >= 0 ? (e >> 6) : 0;          // dropped entries are clamped for the loads
    slot = e >= 0 ? (e & 63) : 0;
    const bf16* qrow = q_idx + (((size_t)it.b * N + t) * H_kv + it.g) * DIDX + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qn[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  };
  fetch(tile);
  const float c = scale_idx * kLog2e;
#pragma unroll 1
  while (true) {
    const int tc = t, sc = slot;
    const bool vc = valid;
    bf16x8 qf[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = qn[ks];
    const int next = tile + 4;
    const bool more = next * 32 < it.nq;
    if (more) fetch(next);
    // The block's 128 keys in two halves of 64 (32 accumulator registers at a
    // time), combined as an online log-sum-exp.  Only the diagonal item
    // masks (keys after the query); the scale c > 0 goes inside the
    // exponent: max(c s) = c max(s).
    float m = -INFINITY, l = 0.f;
#pragma unroll 1
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 s[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int mt = 2 * hf + h;
        s[h] = zero16();
        const bf16* kp = Ks + (mt * 32 + (lane & 31)) * PK + 8 * (lane >> 5);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks)
          s[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kp + ks * 16), qf[ks],
                                                         s[h], 0, 0, 0);
      }
      if (it.diag && causal) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (it.j * kBlock + (2 * hf + h) * 32 + c_row(v, lane) > tc) s[h][v] = -INFINITY;
      }
      float mh = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) mh = fmaxf(mh, s[h][v]);
      mh = fmaxf(mh, swap_half(mh)) * c;       // the same in both lanes of the query
      const float off = mh == -INFINITY ? 0.f : mh;   // a fully masked half adds 0
      float lh = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v = 0; v < 16; ++v) lh += __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][v], c, -off));
      if (hf == 0) {
        m = mh;
        l = lh;
      } else {
        // Finite: half 0 holds key 128 j <= t, or is unmasked.  A masked half
        // (mh = -inf) contributes exp2(-inf) * 0 = 0.
        const float mn = fmaxf(m, mh);
        l = l * __builtin_amdgcn_exp2f(m - mn) + lh * __builtin_amdgcn_exp2f(mh - mn);
        m = mn;
      }
    }
    l += swap_half(l);
    if (vc && lane < 32) part[(((size_t)it.b * N + tc) * H_kv + it.g) * topk + sc] = make_float2(m, l);
    if (!more) break;
    tile = next;
  }
}

// lse_idx (natural log) from the per-slot partials (log2-domain max, sum).
// Four lanes per row, KM / 4 slots each (KM >= topk, a compile-time bound):
// every load of the row is issued at once (slot indices past topk clamped to
// the last slot and skipped), then a max and a sum over the four lanes.
template <int KM>
__global__ __launch_bounds__(256) void idx_lse_merge_kernel(const float2* __restrict__ part,
                                                            const int32_t* __restrict__ block_idx,
                                                            float* __restrict__ lse_idx, int rows, int topk) {
  constexpr int SPL = KM / 4;
  const int r = (blockIdx.x * 256 + threadIdx.x) >> 2;
  const int e0 = (threadIdx.x & 3) * SPL;
  const bool live = r < rows;
  const int rc = live ? r : rows - 1;
  const int32_t* brow = block_idx + (size_t)rc * topk;
  const float2* p = part + (size_t)rc * topk;
  float2 pv[SPL];
  bool ok[SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int e = e0 + i, ec = min(e, topk - 1);
    pv[i] = p[ec];
    ok[i] = e < topk && brow[ec] >= 0;
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < SPL; ++i) m = ok[i] ? fmaxf(m, pv[i].x) : m;
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));   // finite: the own block is always valid
  float l = 0.f;
#pragma unroll
  for (int i = 0; i < SPL; ++i) l += ok[i] ? pv[i].y * __builtin_amdgcn_exp2f(pv[i].x - m) : 0.f;
  l += __shfl_xor(l, 1);
  l += __shfl_xor(l, 2);
  if (live && (threadIdx.x & 3) == 0) lse_idx[r] = (m + __builtin_amdgcn_logf(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Main fused backward: work items, step tables and LDS tile layouts.
// ---------------------------------------------------------------------------
// Work items of the main kernel: the queries of KV block j (its own 128, with
// the causal mask) together with the first item_q entries of its inverted
// list, or a later run of item_q list entries.  Long items keep the per-item
// flush of dK, dV and dk_idx rare; item_q (at most kBigItem) is chosen per
// launch so that the items still outnumber the CUs many times over.
constexpr int kBigItem = 4096;

// Per-step tables (32 entries each) in LDS, double buffered: the row tables
// by step, the query tables (index rows) by index group.
enum : int {
  kRowT = 0,     // t of the row, -1 past the item's end
  kRowCut,       // key u is visible to the row iff u <= cut (-1: none)
  kRowLse,       // LSE * log2(e)
  kRowD,         // rowsum(dO * O)
  kRowId,        // dQ partial row ((b CQ + t - c0) topk + slot) H_q + h, or -1
  kQryT,         // per index row (query) of the step or index group: t or -1
  kQrySlot,      // position of block j in the query's selection
  kQryCut,       // visibility cut-off of the query (-1: none)
  kQryLse,       // index LSE * log2(e)
  kQryKl,        // KL partial (optional output)
  kQryId,        // (b N + t) H_kv + g, or -1
  kNumTabs
};

// Row-major bf16 tiles in LDS.  Pad<P>: rows of P elements.
template <int P>
struct Pad {
  static constexpr int pitch = P;
  __device__ static int off(int r, int c) { return r * P + c; }
};
// A work item of the main kernel and the queries it covers: item-local query
// qi < n_own is t = 128 j + qi (diagonal, causal mask); otherwise it is list
// entry e0 + qi - n_own of block j's inverted list.
struct BigItem {
  int b, g, j, n_own, ne, e0;
  const int32_t* ent;
};

__device__ inline bool decode_big_item(const int32_t* __restrict__ tiles, const int32_t* __restrict__ pos,
                                       const int32_t* __restrict__ offs, const int32_t* __restrict__ rows,
                                       int n_lists, int N, int H_kv, int topk, int nblk, int nsb, int s_lo,
                                       int s_hi, int jb_lo, int jb_hi, int item_q, BigItem* it) {
  const int w = xcd_item(tiles[n_lists]);
  if (w < 0) return false;
  int lo = 0, hi = n_lists - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tiles[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int li = w - tiles[lo];
  it->j = lo % nblk;
  const int bg = lo / nblk;
  it->g = bg % H_kv;
  it->b = bg / H_kv;
  // The list entries of the query chunk: super-blocks [s_lo, s_hi) of list j.
  const int32_t* pb = pos + (size_t)bg * (nsb + 1) * nblk + it->j;
  const int seg0 = pb[(size_t)s_lo * nblk], seg1 = pb[(size_t)s_hi * nblk];
  const bool diag = it->j >= jb_lo && it->j < jb_hi;
  it->n_own = (li == 0 && diag) ? kBlock : 0;
  it->e0 = seg0 + li * item_q;
  it->ne = max(0, min(item_q, seg1 - it->e0));
  it->ent = rows + (size_t)bg * N * topk + offs[(size_t)bg * (nblk + 1) + it->j];
  return true;
}

// t (-1 when qi is past the item) and the slot of block j in the query's row.
__device__ inline int big_query(const BigItem& it, int qi, const int32_t* __restrict__ block_idx, int N, int H_kv,
                                int topk, int* slot) {
  *slot = 0;
  if (qi < it.n_own) {
    const int t = it.j * kBlock + qi;
    const int32_t* brow = block_idx + (((size_t)it.b * N + t) * H_kv + it.g) * topk;
    for (int e = 0; e < topk; ++e)
      if (brow[e] == it.j) *slot = e;
    return t;
  }
  const int ei = qi - it.n_own;
  if (ei >= it.ne) return -1;
  const int e = it.ent[it.e0 + ei];
  const int t = e >> 6;
  if (t < 0 || t >= N || (e & 63) >= topk) return -1;   // malformed map: drop the entry
  *slot = e & 63;
  return t;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

__device__ inline bf16x4 pack4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (bf16)a; r[1] = (bf16)b; r[2] = (bf16)c; r[3] = (bf16)d;
  return r;
}

// ---------------------------------------------------------------------------
// Main fused backward, 16x16x32 formulation.  8 waves; wave w owns keys
// 16w..16w+15 of the block, which keeps its dK, dV and dk_idx accumulators
// small enough for two waves per SIMD.  16x16x32 MFMA layouts (lane l,
// q = l / 16, c = l % 16): A: row c, k = 8q + i; B: column c, k = 8q + i;
// C: column c, rows 4q + v in slot v.
// A step covers 32 (query, head) rows in two 16-row tiles.  Row 16 tile + 4q + v
// of a step holds R = 8q + 4 tile + v, i.e. query R / G and head R % G, so
// that the lanes of group q hold whole queries (for G <= 8) and the teacher
// mean over a query's heads is a sum inside the lane.  The index logits use
// "query rows" m' = 16 t + 4q + v whose query is ri_query<G>(t, q, v), or,
// for G >= 8, the query rows of an index group of G / 2 steps (idx_group).
// ---------------------------------------------------------------------------
constexpr int kW16 = 8;                        // waves of the 16x16 kernel
constexpr int kT16 = kW16 * kWave;             // its threads

__device__ inline f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Operand of a 16x16x32 MFMA read with the gfx950 transpose read from a
// row-major tile of layout L: lane (q, c) gets column m0 + c and the K values
// of rows ra .. ra+3 (slots 0..3) and rb .. rb+3 (slots 4..7), where ra and rb
// are the lane group's row bases.
template <class L>
__device__ inline bf16x8 tr16(const bf16* base, int m0, int ra, int rb, int lane) {
  const int jj = lane & 15;
  const int col = m0 + 4 * (jj & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + L::off(ra + (jj >> 2), col)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + L::off(rb + (jj >> 2), col)));
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
  bf16x8 r;
  r[0] = l4[0]; r[1] = l4[1]; r[2] = l4[2]; r[3] = l4[3];
  r[4] = h4[0]; r[5] = h4[1]; r[6] = h4[2]; r[7] = h4[3];
  return r;
}
// B operand whose K slots are rows 4q..4q+3 of tile 0 and of tile 1 of a
// C-layout pair: the two tiles' registers as they are.
__device__ inline bf16x8 cpair(const f32x4& a, const f32x4& b) {
  bf16x8 r;
  r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)a[2]; r[3] = (bf16)a[3];
  r[4] = (bf16)b[0]; r[5] = (bf16)b[1]; r[6] = (bf16)b[2]; r[7] = (bf16)b[3];
  return r;
}
// Step row of tile t, lane group q, slot v -> R (query R / G, head R % G).
__device__ inline int row_r(int t, int q, int v) { return 8 * q + 4 * t + v; }
// Query (within the step) of query row m' = 16 t + 4 q + v, or -1.
template <int G>
__device__ inline int ri_query(int t, int q, int v) {
  if constexpr (G == 1) return 8 * q + 4 * t + v;
  else if constexpr (G <= 8) return (t == 0 && v < 8 / G) ? q * (8 / G) + v : -1;
  else return (t == 0 && v == 0 && (q & 1) == 0) ? q / 2 : -1;
}
// Index-logit groups.  With G >= 8 a step holds TQ = 32 / G <= 4 queries and
// fills at most a quarter of a 16-row index-logit tile.  The index work
// (logits, dz, dk_idx and dq_idx) then runs once per F = 16 / TQ = G / 2
// consecutive steps, on one tile whose row 4q + v holds query idx_local of
// group step idx_step.  That query's teacher mean is in lane group q of the
// step (slot 0 of head_mean16), so each lane keeps the four means of its
// rows until the group's last step.  With G <= 4 (F = 1) the tile rows are
// the ri_query rows of every step: at G = 4, groups of two steps measured
// slower than the half-empty tiles (B = 4, N = 8K: 5.04 -> 5.2 ms).
template <int G>
constexpr int idx_group() { return G >= 8 ? G / 2 : 1; }
template <int G>
__device__ inline int idx_step(int q, int v) { return G == 8 ? v : 4 * (q & 1) + v; }
template <int G>
__device__ inline int idx_local(int q, int v) { return G == 8 ? q : q >> 1; }
// What step st of a group (s = st mod F) stores in index row r (0..31): the
// local query >= 0 to load, -1 to clear the row (no query), -2 to keep it.
// A group's first step clears every row that a later step of the group
// fills, so that rows a short item never reaches hold no query.
template <int G>
__device__ inline int idx_row_query(int r, int s) {
  if constexpr (idx_group<G>() == 1) {
    return ri_query<G>(r >> 4, (r >> 2) & 3, r & 3);
  } else {
    if (r < 16 && idx_step<G>(r >> 2, r & 3) == s) return idx_local<G>(r >> 2, r & 3);
    return s == 0 ? -1 : -2;
  }
}
// Whether index row 16 t + 4 q + v can hold a query.
template <int G>
__device__ inline bool idx_row_used(int t, int q, int v) {
  if constexpr (idx_group<G>() == 1) return ri_query<G>(t, q, v) >= 0;
  else return t == 0;
}
// Teacher: mean of P over each query's heads, at the query rows' C layout.
template <int G>
__device__ inline void head_mean16(const f32x4* p, f32x4* pb) {
  constexpr float inv = 1.0f / G;
  if constexpr (G == 1) {
    pb[0] = p[0];
    pb[1] = p[1];
  } else if constexpr (G == 2) {
#pragma unroll
    for (int v = 0; v < 4; ++v) pb[0][v] = (p[v >> 1][2 * (v & 1)] + p[v >> 1][2 * (v & 1) + 1]) * inv;
  } else if constexpr (G == 4) {
    pb[0] = zero4();
#pragma unroll
    for (int v = 0; v < 2; ++v) pb[0][v] = (p[v][0] + p[v][1] + p[v][2] + p[v][3]) * inv;
  } else {
    float s = p[0][0] + p[0][1] + p[0][2] + p[0][3] + p[1][0] + p[1][1] + p[1][2] + p[1][3];
    if constexpr (G == 16) s += __shfl_xor(s, 16);
    pb[0] = zero4();
    pb[0][0] = s * inv;
  }
}

// LDS tiles of the main kernel.  The gfx950 LDS serves the reads of 32 lanes
// together, from 128 four-byte banks for 16-byte reads and from 64 banks for
// 8-byte and transpose reads; writes use 32 banks.  Under that rule the padded
// pitches below leave the kernel's per-step accesses free of bank conflicts:
// the 16-byte A-operand reads of one chunk from 16 consecutive rows of Q, dO
// and q_idx, the transpose reads of Q, dO and q_idx, and the 8-byte dS^T / dz^T
// writes (whose transpose reads keep a 2-way conflict in one of four passes).
// Padding folds into instruction offsets, where an XOR swizzle would hold one
// address register per access.
template <int D, int DIDX>
struct Bwd16Cfg {
  using TQ = Pad<D + 16>;                  // Q, dO tiles (step rows)
  using TI = Pad<DIDX + 16>;               // q_idx, K_idx tiles
  using TS = Pad<32 + 4>;                  // dS^T, dz^T: one row of 32 step rows per key (+8 B)
  using TT = Pad<kBlock + 16>;             // K^T, K_idx^T: one row of the 128 keys per column
  static constexpr int PQ = TQ::pitch, PQI = TI::pitch, PST = TS::pitch, PKT = TT::pitch;
  static constexpr size_t OFF_QS = 0;                                    // Q        [32][PQ]
  static constexpr size_t OFF_DOS = OFF_QS + (size_t)32 * PQ * 2;        // dO       [32][PQ]
  static constexpr size_t OFF_QIS = OFF_DOS + (size_t)32 * PQ * 2;       // q_idx    [32][PQI]
  static constexpr size_t OFF_DST = OFF_QIS + (size_t)32 * PQI * 2;      // dS^T     [128][PST]
  static constexpr size_t OFF_DZT = OFF_DST + (size_t)kBlock * PST * 2;  // dz^T     2 x [128][PST]
  static constexpr size_t OFF_TAB = OFF_DZT + (size_t)2 * kBlock * PST * 2;   // 2 x kNumTabs x [32]
  static constexpr size_t OFF_KT = OFF_TAB + (size_t)2 * kNumTabs * 32 * 4;   // K^T    [D][PKT]
  static constexpr size_t OFF_KIS = OFF_KT + (size_t)D * PKT * 2;        // K_idx  [128][PQI]
  static constexpr size_t OFF_KIT = OFF_KIS + (size_t)kBlock * PQI * 2;  // K_idx^T [DIDX][PKT]
  static constexpr size_t OFF_QL = OFF_KIT + (size_t)DIDX * PKT * 2;     // item queries: (t << 6) | slot
  static constexpr int KPQ = kW16 / (D / 16);                             // key parts of the dQ product
  static constexpr int PDQ = D + 4;                                       // dQ tile row pitch (fp32)
  // dQ [KPQ][32][PDQ] fp32, only when the dQ product is split over key parts
  // (d = 64); at d = 128 each wave's product covers all keys and is stored
  // from registers.
  // The list is followed by kQlPad entries of -1, so that the step loop's
  // look-ahead past the item's end reads them instead of testing its index.
  static constexpr int kQlPad = 128;
  static constexpr size_t OFF_DQ = OFF_QL + (size_t)(kBlock + kBigItem + kQlPad) * 4;
  static constexpr size_t LDS = OFF_DQ + (KPQ > 1 ? (size_t)KPQ * 32 * PDQ * 4 : 0);
  // The flush at the end of an item reuses [0, OFF_QL) as 8 x [16][D + 4] fp32.
  static_assert(OFF_QL >= (size_t)kW16 * 16 * (D + 4) * 4, "flush scratch");
  static_assert(LDS <= 160 * 1024, "LDS of one CU");
  static_assert(PQ % 8 == 0 && PQI % 8 == 0 && PST % 4 == 0 && PKT % 8 == 0,
                "16-byte rows for 16-byte accesses, 8-byte for dS^T");
};
// Position of key kk in a row of the K^T and K_idx^T tiles.  The 16-byte
// read at position 32 a + 8 q of a row gives lane group q the keys
// 32 a + 4 q .. +3 and 32 a + 16 + 4 q .. +3, the K order in which the
// transpose reads of dS^T and dz^T hand their rows to the same lanes.
__device__ inline int kt_pos(int kk) {
  return (kk & ~31) + 8 * ((kk >> 2) & 3) + 4 * ((kk >> 4) & 1) + (kk & 3);
}

template <int D, int DIDX, int G, bool EXTRA>
__global__ __launch_bounds__(kT16, 2) void bwd_main16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dv,
    const bf16* __restrict__ q_idx, const bf16* __restrict__ k_idx, const float* __restrict__ lse_idx,
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ pos, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ tiles, bf16* __restrict__ dq_part,
    float* __restrict__ dk_acc, float* __restrict__ dv_acc, float* __restrict__ dq_idx,
    float* __restrict__ dk_idx, float* __restrict__ dscore, float* __restrict__ kl, int N, int H_kv, int topk,
    int causal, int nblk, int nsb, int n_lists, float scale, float scale_idx, float lam, int n_prow,
    int n_grows, int c0, int CQ, int s_lo, int s_hi, int item_q) {
  using C = Bwd16Cfg<D, DIDX>;
  constexpr int KS = D / 32;        // 32-wide k-steps over d
  constexpr int KSI = DIDX / 32;    // 32-wide k-steps over d_idx
  constexpr int DT = D / 16;        // 16-wide d tiles
  constexpr int DTI = DIDX / 16;    // 16-wide d_idx tiles
  constexpr int TQ = 32 / G;        // queries per 32-row step
  constexpr int NTQ = G == 1 ? 2 : 1;                       // query-row tiles
  constexpr int F = idx_group<G>();                         // steps per index group
  constexpr int CPR = D / 8;        // 16-byte chunks per Q / dO row
  constexpr int CPRI = DIDX / 8;    // 16-byte chunks per q_idx row
  constexpr int NT = kNumTabs * 32;
  // dQ: column tile w % DT over the key part w / DT (of KPQ parts); dq_idx likewise.
  constexpr int KPQ = kW16 / DT;    // 1 (d = 128) or 2 (d = 64) parts of the 128 keys
  static_assert(kW16 % DT == 0 && kW16 % DTI == 0, "wave split");
  static_assert(32 * CPR <= kT16 && 32 * CPRI <= kT16, "one tile chunk per thread");
  extern __shared__ __align__(16) char smem[];
  bf16* Qs = reinterpret_cast<bf16*>(smem + C::OFF_QS);
  bf16* dOs = reinterpret_cast<bf16*>(smem + C::OFF_DOS);
  bf16* QIs = reinterpret_cast<bf16*>(smem + C::OFF_QIS);
  bf16* dSt = reinterpret_cast<bf16*>(smem + C::OFF_DST);
  bf16* dZt2 = reinterpret_cast<bf16*>(smem + C::OFF_DZT);  // dz^T of steps of either parity
  int* tabs = reinterpret_cast<int*>(smem + C::OFF_TAB);
  bf16* Kt = reinterpret_cast<bf16*>(smem + C::OFF_KT);
  bf16* KIs = reinterpret_cast<bf16*>(smem + C::OFF_KIS);
  bf16* KIt = reinterpret_cast<bf16*>(smem + C::OFF_KIT);
  int* qlist = reinterpret_cast<int*>(smem + C::OFF_QL);   // (t << 6) | slot, or -1
  float* dQt = reinterpret_cast<float*>(smem + C::OFF_DQ);  // a step's dQ tile, one slice per key part

  BigItem it;
  if (!decode_big_item(tiles, pos, offs, rows, n_lists, N, H_kv, topk, nblk, nsb, s_lo, s_hi, c0 / kBlock,
                       (c0 + CQ + kBlock - 1) / kBlock, item_q, &it))
    return;
  int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int c = lane & 15, lq = lane >> 4;                  // C layout: column c, rows 4 lq + v
  const int H_q = H_kv * G;
  const int b = it.b, g = it.g, j = it.j;
  const int key = 16 * wave + c;                      // this lane's key inside the block
  const int u = j * kBlock + key;
  const size_t blk_row0 = ((size_t)b * N + (size_t)j * kBlock) * H_kv + g;   // key 0 of the block
  const int nq = it.n_own + it.ne;   // >= 1: an item holds its diagonal queries or list entries

  for (int qi = threadIdx.x; qi < nq + C::kQlPad; qi += kT16) {
    int slot;
    const int t = big_query(it, qi, block_idx, N, H_kv, topk, &slot);
    qlist[qi] = (qi >= nq || t < 0) ? -1 : ((t << 6) | slot);
  }
  // K and K_idx transposed (keys in kt_pos order) for the B operands of the
  // dQ and dq_idx products; K_idx also row-major for the index logits.
  for (int cc = threadIdx.x; cc < kBlock * CPR; cc += kT16) {
    const int kk = cc / CPR, col = (cc % CPR) * 8;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(k + (blk_row0 + (size_t)kk * H_kv) * D + col);
#pragma unroll
    for (int i = 0; i < 8; ++i) Kt[(col + i) * C::PKT + kt_pos(kk)] = x[i];
  }
  for (int cc = threadIdx.x; cc < kBlock * CPRI; cc += kT16) {
    const int kk = cc / CPRI, col = (cc % CPRI) * 8;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(k_idx + ((size_t)b * N + j * kBlock + kk) * DIDX + col);
    *reinterpret_cast<bf16x8*>(KIs + C::TI::off(kk, col)) = x;
#pragma unroll
    for (int i = 0; i < 8; ++i) KIt[(col + i) * C::PKT + kt_pos(kk)] = x[i];
  }
  int qct = wave % DT, qkp = wave / DT;         // dQ column tile and key part
  // The B operands of S and dP (this lane's key row of K and of V), constant
  // over the item: held in registers, which takes a third of the step's LDS
  // operand traffic off the S / dP products.
  bf16x8 kfr[KS], vfr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {   // straight from memory: K and V rows are read only here
    kfr[ks] = *reinterpret_cast<const bf16x8*>(k + (blk_row0 + (size_t)key * H_kv) * D + 32 * ks + 8 * lq);
    vfr[ks] = *reinterpret_cast<const bf16x8*>(v + (blk_row0 + (size_t)key * H_kv) * D + 32 * ks + 8 * lq);
  }
  int ict = wave % DTI, ikp = wave / DTI;       // dq_idx column tile; ikp = 0: the wave that computes it

  f32x4 acc_dv[DT], acc_dk[DT], acc_dki[DTI];
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    acc_dv[i] = zero4();
    acc_dk[i] = zero4();
  }
#pragma unroll
  for (int i = 0; i < DTI; ++i) acc_dki[i] = zero4();
  __syncthreads();   // item query list and the K^T, K_idx, K_idx^T tiles ready

  // Per-thread share of a step, loaded one step ahead: one 16-byte chunk of
  // Q and of dO (thread < 32 CPR) with the row's statistics when the chunk is
  // the row's first, one chunk of q_idx (thread < 32 CPRI), and the query-row
  // table entry (thread < 32).
  const int tx = threadIdx.x;
  const bool ld_row = tx < 32 * CPR;
  const int ld_m = (tx / CPR) & 31, ld_col = (tx % CPR) * 8;
  const int ld_rr = row_r(ld_m >> 4, (ld_m >> 2) & 3, ld_m & 3);   // R of the thread's row
  const bool ld_qi = tx < 32 * CPRI;
  const int ld_mi = (tx / CPRI) & 31, ld_qcol = (tx % CPRI) * 8;
  const int mq = tx & 31;
  struct Pre {
    bf16x8 q, d, qi;
    float lse, rd, qlse;
    int t, cut, id, qt, qslot, qcut, qid;
  };
  Pre pre;
  int pk_e = -1, pk_qi = -1, pk_qt = -1;
  // Look-ahead indices stay below nq + 3 * TQ <= nq + 96 (two steps ahead
  // of the last, each of at most 32 queries), inside the padding.
  auto entry = [&](int qi) { return qlist[qi]; };
  auto cutoff = [&](int qi, int t) { return t < 0 ? -1 : ((qi < it.n_own && causal) ? t : 0x7fffffff); };
  auto peek = [&](int st) {
    pk_e = ld_row ? entry(st * TQ + ld_rr / G) : -1;
    const int lqi = idx_row_query<G>(ld_mi, st & (F - 1)), lqt = idx_row_query<G>(mq, st & (F - 1));
    pk_qi = (ld_qi && lqi >= 0) ? entry(st * TQ + lqi) : -1;
    pk_qt = (tx < 32 && lqt >= 0) ? entry(st * TQ + lqt) : -1;
  };
  // Unconditional loads (clamped to a valid row): the compiler counts them.
  // Row indices are 32-bit (B N H_q < 2^31, checked by the host), with the
  // thread's constant column and head folded into base pointers, so a step's
  // addresses cost a 32-bit multiply-add and a shift each.
  const int hq_ld = g * G + ld_rr % G;                       // head of the thread's Q / dO row
  const int bN = b * N;
  const bf16* q_ld = q + (size_t)hq_ld * D + ld_col;
  const bf16* dO_ld = dO + (size_t)hq_ld * D + ld_col;
  const float* lse_ld = lse + hq_ld;
  const float* Dv_ld = Dv + hq_ld;
  const bf16* qi_ld = q_idx + (size_t)g * DIDX + ld_qcol;
  const int id_base = b * CQ - c0;                            // chunk-local query of t: id_base + t
  auto load_step = [&](int st) {
    {
      const int t = pk_e < 0 ? -1 : (pk_e >> 6);
      pre.t = t;
      pre.cut = cutoff(st * TQ + ld_rr / G, t);
      const int qrow = (bN + max(t, 0)) * H_q;                // row of (b, t, head 0)
      // dQ partial row of (t, head, slot) within the query chunk.
      const bool in_chunk = t >= c0 && t < c0 + CQ;
      pre.id = in_chunk ? (((id_base + t) * topk + (pk_e & 63)) * H_q + hq_ld) : -1;
      pre.q = *reinterpret_cast<const bf16x8*>(q_ld + (size_t)qrow * D);
      pre.d = *reinterpret_cast<const bf16x8*>(dO_ld + (size_t)qrow * D);
      pre.lse = lse_ld[qrow];
      pre.rd = Dv_ld[qrow];
    }
    {
      const int tq = pk_qi < 0 ? -1 : (pk_qi >> 6);
      pre.qi = *reinterpret_cast<const bf16x8*>(qi_ld + (size_t)((bN + max(tq, 0)) * H_kv) * DIDX);
      if (tq < 0) pre.qi = bf16x8{};
    }
    {
      pre.qt = pk_qt < 0 ? -1 : (pk_qt >> 6);
      pre.qslot = pk_qt < 0 ? 0 : (pk_qt & 63);
      pre.qcut = cutoff(st * TQ + max(idx_row_query<G>(mq, st & (F - 1)), 0), pre.qt);
      const int qrow = (bN + max(pre.qt, 0)) * H_kv + g;
      pre.qid = pre.qt < 0 ? -1 : qrow;
      pre.qlse = lse_idx[qrow];
    }
  };
  auto store_step = [&](int st) {
    int* tb = tabs + (st & 1) * NT;
    float* tf = reinterpret_cast<float*>(tb);
    if (ld_row) {
      *reinterpret_cast<bf16x8*>(Qs + C::TQ::off(ld_m, ld_col)) = pre.q;
      *reinterpret_cast<bf16x8*>(dOs + C::TQ::off(ld_m, ld_col)) = pre.d;
      if (ld_col == 0) {
        tb[kRowT * 32 + ld_m] = pre.t;
        tb[kRowCut * 32 + ld_m] = pre.cut;
        tf[kRowLse * 32 + ld_m] = pre.t < 0 ? INFINITY : pre.lse * kLog2e;   // no query: P = 0
        tf[kRowD * 32 + ld_m] = pre.rd;
        tb[kRowId * 32 + ld_m] = pre.id;
      }
    }
    if (ld_qi && idx_row_query<G>(ld_mi, st & (F - 1)) != -2)
      *reinterpret_cast<bf16x8*>(QIs + C::TI::off(ld_mi, ld_qcol)) = pre.qi;
    int* tg = tabs + ((st / F) & 1) * NT;   // the query tables of the step's index group
    float* tgf = reinterpret_cast<float*>(tg);
    if (tx < 32 && idx_row_query<G>(mq, st & (F - 1)) != -2) {
      tg[kQryT * 32 + tx] = pre.qt;
      tg[kQrySlot * 32 + tx] = pre.qslot;
      tg[kQryCut * 32 + tx] = pre.qcut;
      tgf[kQryLse * 32 + tx] = pre.qlse * kLog2e;
      tgf[kQryKl * 32 + tx] = 0.f;
      tg[kQryId * 32 + tx] = pre.qid;
    }
  };

  const float c_s = scale * kLog2e;
  const float c_i = scale_idx * kLog2e;
  const int n_steps = (nq * G + 31) / 32;
  // dq_idx[query rows, column tile ict] = dz K_idx over the block's keys, for
  // the index group that ends at step st.  It runs at the top of step st + 1,
  // before that step's loads are issued: its atomics are conditional, so the
  // compiler cannot count them, and there they sit behind no load that has to
  // be waited for (dz^T is double buffered for it, by group).
  auto dq_idx_step = [&](int st) {
    // The waves of key part 0 take all 128 keys of their column tile and the
    // others skip, so each dq_idx value gets one atomic per index group
    // rather than one per key part (at d_idx = 64 a skipping wave shares its
    // SIMD with a working one).
    if (ikp != 0) return;
    const int* tb = tabs + ((st / F) & 1) * NT;
    const bf16* dZt = dZt2 + ((st / F) & 1) * kBlock * C::PST;
    f32x4 o[NTQ];
#pragma unroll
    for (int t = 0; t < NTQ; ++t) {
      o[t] = zero4();
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int k0 = 32 * ks + 4 * lq;
        o[t] = mma16(tr16<typename C::TS>(dZt, 16 * t, k0, k0 + 16, lane),
                     *reinterpret_cast<const bf16x8*>(KIt + (16 * ict + c) * C::PKT + 32 * ks + 8 * lq), o[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < NTQ; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (idx_row_used<G>(t, lq, e)) {
          const int id = tb[kQryId * 32 + 16 * t + 4 * lq + e];
          if ((unsigned)id < (unsigned)n_grows) atomicAdd(dq_idx + (size_t)id * DIDX + 16 * ict + c, o[t][e]);
        }
  };
  // Store step st's dQ rows from its tile in LDS as bf16 partials (one row of
  // d values per (query, head, slot)): wave w takes rows 4w .. 4w+3, 16 bytes
  // per lane, whole rows per instruction.  A row without a query goes to the
  // spare row n_prow, so the stores are unconditional; every row index is
  // checked against the partial rows before it becomes an address.
  auto dq_store = [&](int st) {
    constexpr int LPR = D / 8;                          // lanes per row
    const int* tb = tabs + (st & 1) * NT;
    const int row = 4 * wave + (lane / LPR) % 4;
    const int col = (lane % LPR) * 8;
    if (lane < 4 * LPR) {
      float x[8];
#pragma unroll
      for (int kp = 0; kp < C::KPQ; ++kp) {
        const float4 a0 = *reinterpret_cast<const float4*>(dQt + (kp * 32 + row) * C::PDQ + col);
        const float4 a1 = *reinterpret_cast<const float4*>(dQt + (kp * 32 + row) * C::PDQ + col + 4);
        const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = kp == 0 ? a[i] : x[i] + a[i];   // no 0 + a for the first part
      }
      bf16x8 y;
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = (bf16)x[i];
      const int id = tb[kRowId * 32 + row];
      const int dst = (unsigned)id < (unsigned)n_prow ? id : n_prow;
      // Streaming store: the partials are read once, by dq_merge_kernel.
      __builtin_nontemporal_store(y, reinterpret_cast<bf16x8*>(dq_part + (size_t)dst * D + col));
    }
  };
  f32x4 pbh = zero4();   // teacher means of the lane's index rows (F > 1)
  peek(0);
  load_step(0);
  store_step(0);
  peek(1);
#pragma unroll 1
  for (int st = 0; st < n_steps; ++st) {
    asm volatile("" ::: "memory");
    const int* tb = tabs + (st & 1) * NT;
    const float* tf = reinterpret_cast<const float*>(tb);
    __syncthreads();   // step st's tiles and tables in LDS; step st-1's dS^T / dz^T complete
    if (st > 0 && ((st - 1) & (F - 1)) == F - 1) dq_idx_step(st - 1);   // a group ended at step st - 1
    // Index work in this step: every step with F = 1, else a group's last
    // step and the item's last step (which may end a group early).
    const bool idx_now = F == 1 || (st & (F - 1)) == F - 1 || st == n_steps - 1;
    const int* tg = tabs + ((st / F) & 1) * NT;   // the index group's query tables
    const float* tgf = reinterpret_cast<const float*>(tg);
    load_step(st + 1);
    peek(st + 2);
    if constexpr (C::KPQ > 1)
      if (st > 0) dq_store(st - 1);   // after the loads: the wait for them at the step's end skips it

    // Index work on the query rows (NTQ tiles; lane = key, slots = rows):
    // the logits, p_px and dz (with dz^T to LDS), and dk_idx^T += q_idx^T dz.
    auto idx_logits = [&](f32x4* ri) {
#pragma unroll
      for (int t = 0; t < NTQ; ++t) {
        ri[t] = zero4();
#pragma unroll
        for (int ks = 0; ks < KSI; ++ks) {
          const int col = 32 * ks + 8 * lq;
          ri[t] = mma16(*reinterpret_cast<const bf16x8*>(QIs + C::TI::off(16 * t + c, col)),
                        *reinterpret_cast<const bf16x8*>(KIs + C::TI::off(key, col)), ri[t]);
        }
      }
    };
    auto idx_dz = [&](const f32x4* ri, const f32x4* pb, f32x4* dz) {
#pragma unroll
      for (int t = 0; t < NTQ; ++t) {
        const int r4 = 16 * t + 4 * lq;
        const int4 qc = *reinterpret_cast<const int4*>(tg + kQryCut * 32 + r4);
        const f32x4 ql = *(const volatile lds_f32x4*)(tgf + kQryLse * 32 + r4);
        const int qcs[4] = {qc.x, qc.y, qc.z, qc.w};
        const float qls[4] = {ql[0], ql[1], ql[2], ql[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lz = ri[t][e] * c_i - qls[e];     // log2 p_px
          const bool vis = u <= qcs[e];                  // -1 for rows that hold no query
          const float ez = __builtin_amdgcn_exp2f(vis ? lz : -INFINITY);
          dz[t][e] = vis ? lam * (ez - pb[t][e]) : 0.f;
          if (EXTRA && dscore != nullptr && vis) {
            const int tq = tg[kQryT * 32 + r4 + e], sl = tg[kQrySlot * 32 + r4 + e];
            if ((unsigned)tq < (unsigned)N && (unsigned)sl < (unsigned)topk)
              dscore[((((size_t)b * N + tq) * H_kv + g) * topk + sl) * kBlock + key] = dz[t][e];
          }
          if (EXTRA && kl != nullptr) {
            float klv = (vis && pb[t][e] > 0.f) ? pb[t][e] * (logf(pb[t][e]) - lz * kLn2) : 0.f;
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) klv += __shfl_xor(klv, off);   // over the lane group's 16 keys
            if (c == 0 && qcs[e] >= 0)
              atomicAdd(reinterpret_cast<float*>(tabs + ((st / F) & 1) * NT) + kQryKl * 32 + r4 + e, klv);
          }
        }
        *reinterpret_cast<bf16x4*>(dZt2 + ((st / F) & 1) * kBlock * C::PST + key * C::PST + r4) =
            pack4(dz[t][0] * scale_idx, dz[t][1] * scale_idx, dz[t][2] * scale_idx, dz[t][3] * scale_idx);
      }
    };
    auto idx_dki = [&](const f32x4* dz) {
      const bf16x8 zb = cpair(dz[0] * scale_idx, NTQ == 2 ? dz[NTQ - 1] * scale_idx : zero4());
#pragma unroll
      for (int dt = 0; dt < DTI; ++dt)
        acc_dki[dt] = mma16(tr16<typename C::TI>(QIs, 16 * dt, 4 * lq, 16 + 4 * lq, lane), zb, acc_dki[dt]);
    };

    // The product stretches of the step run at raised wave priority: of two
    // waves of a SIMD in the same stretch, one then runs ahead and reaches
    // its vector work while the other still issues products.
    // S, dP (two row tiles; lane = key, slots = rows), with the index logits
    // when every step runs the index work (F = 1).
    __builtin_amdgcn_s_setprio(1);
    f32x4 s[2], dp[2], ri[NTQ], dz[NTQ];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = zero4();
      dp[t] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int col = 32 * ks + 8 * lq;
        s[t] = mma16(*reinterpret_cast<const bf16x8*>(Qs + C::TQ::off(16 * t + c, col)), kfr[ks], s[t]);
        dp[t] = mma16(*reinterpret_cast<const bf16x8*>(dOs + C::TQ::off(16 * t + c, col)), vfr[ks], dp[t]);
      }
    }
    if constexpr (F == 1) idx_logits(ri);
    __builtin_amdgcn_s_setprio(0);
    // P, dS; dS^T to LDS (rows 16 t + 4 lq .. +3 of this lane's key).  Only
    // the steps holding the block's own queries (causal) test each key
    // against the row's cut-off; a row without a query has LSE = +inf, so
    // its P is exp2(-inf) = 0 either way.
    f32x4 p[2], ds[2];
    auto p_ds = [&](auto masked_c) {
      constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r4 = 16 * t + 4 * lq;
        int cuts[4] = {0, 0, 0, 0};
        if constexpr (MASKED) {
          const int4 cut = *reinterpret_cast<const int4*>(tb + kRowCut * 32 + r4);
          cuts[0] = cut.x; cuts[1] = cut.y; cuts[2] = cut.z; cuts[3] = cut.w;
        }
        // Volatile: read whole and up front, never sunk into the masked use.
        const f32x4 l2 = *(const volatile lds_f32x4*)(tf + kRowLse * 32 + r4);
        const float4 dd = *reinterpret_cast<const float4*>(tf + kRowD * 32 + r4);
        const float l2s[4] = {l2[0], l2[1], l2[2], l2[3]};
        const float dds[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // Masked by the exponent (exp2(-inf) = 0), so no branch is formed.
          const float x = s[t][e] * c_s - l2s[e];
          const float pv = __builtin_amdgcn_exp2f(MASKED ? (u <= cuts[e] ? x : -INFINITY) : x);
          p[t][e] = pv;
          ds[t][e] = pv * (dp[t][e] - dds[e]) * scale;
        }
        *reinterpret_cast<bf16x4*>(dSt + key * C::PST + r4) = pack4(ds[t][0], ds[t][1], ds[t][2], ds[t][3]);
      }
    };
    // (At G = 16, and in the instances with per-score outputs, the two
    // versions of this code cost spilled registers, so those keep the masked
    // one for every step.)
    if (EXTRA || G > 8 || (causal && st * TQ < it.n_own)) p_ds(std::true_type{});
    else p_ds(std::false_type{});
    // Teacher p̄ on the query rows; with F > 1 each lane keeps the means of
    // its index rows until the group's last step.
    f32x4 pb[NTQ];
    head_mean16<G>(p, pb);
    if constexpr (F == 1) {
      idx_dz(ri, pb, dz);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (idx_step<G>(lq, v) == (st & (F - 1))) pbh[v] = pb[0][0];
    }
    // dV^T += dO^T P, dK^T += Q^T dS (K = the 32 rows, in the order of the
    // two tiles' slots), dk_idx^T += q_idx^T dz.
    {
      __builtin_amdgcn_s_setprio(1);
      const bf16x8 pbf = cpair(p[0], p[1]), sbf = cpair(ds[0], ds[1]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        acc_dv[dt] = mma16(tr16<typename C::TQ>(dOs, 16 * dt, 4 * lq, 16 + 4 * lq, lane), pbf, acc_dv[dt]);
        acc_dk[dt] = mma16(tr16<typename C::TQ>(Qs, 16 * dt, 4 * lq, 16 + 4 * lq, lane), sbf, acc_dk[dt]);
      }
      if constexpr (F == 1) idx_dki(dz);
      __builtin_amdgcn_s_setprio(0);
    }
    // With F > 1 the group's index work, once, on its last step.
    if constexpr (F > 1) {
      if (idx_now) {
        const f32x4 pbg[1] = {pbh};
        idx_logits(ri);
        idx_dz(ri, pbg, dz);
        idx_dki(dz);
      }
    }
    __syncthreads();   // dS^T, dz^T and the KL partials complete

    // dQ[rows, column tile qct] = dS K over key part qkp.  With one key part
    // (d = 128) it is computed transposed, dQ^T = K^T dS^T, so that a lane
    // holds 4 consecutive columns of one row and stores them as the row's
    // bf16 partial at once.  With two (d = 64) the parts meet in the step's
    // dQ tile in LDS (lane = column, slots = rows), which leaves as bf16
    // partials at the top of the next step, whose barrier completes it;
    // nothing reads the tile between the barrier above and this write.
    {
      // The K operands are read once for both row tiles, and the tile is
      // written after all products (an LDS write between them would make the
      // compiler read K again for the second tile).
      bf16x8 kq[4 / KPQ];
#pragma unroll
      for (int ks = 0; ks < 4 / KPQ; ++ks)   // keys k0 .. k0+3, k0+16 .. k0+19 of the dS^T reads below
        kq[ks] = *reinterpret_cast<const bf16x8*>(Kt + (16 * qct + c) * C::PKT + 32 * (qkp * (4 / KPQ) + ks) + 8 * lq);
      f32x4 o[2];
      if constexpr (C::KPQ == 1) {
        __builtin_amdgcn_s_setprio(1);   // as for the other product stretches
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          o[t] = zero4();
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const int k0 = 32 * ks + 4 * lq;
            o[t] = mma16(kq[ks], tr16<typename C::TS>(dSt, 16 * t, k0, k0 + 16, lane), o[t]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
        // Row 16 t + c, columns 16 qct + 4 lq .. +3.  A row without a query
        // goes to the spare row n_prow, so the stores are unconditional; every
        // row index is checked against the partial rows before it becomes an
        // address.  Ordinary (not streaming) stores: the 8 waves' 32-byte
        // pieces of a row meet in L2 as whole lines (streaming stores of these
        // pieces made the kernel 10% slower at N = 128K).
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int id = tb[kRowId * 32 + 16 * t + c];
          const int dst = (unsigned)id < (unsigned)n_prow ? id : n_prow;
          *reinterpret_cast<bf16x4*>(dq_part + (size_t)dst * D + 16 * qct + 4 * lq) =
              pack4(o[t][0], o[t][1], o[t][2], o[t][3]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          o[t] = zero4();
#pragma unroll
          for (int ks = 0; ks < 4 / KPQ; ++ks) {
            const int k0 = 32 * (qkp * (4 / KPQ) + ks) + 4 * lq;
            o[t] = mma16(tr16<typename C::TS>(dSt, 16 * t, k0, k0 + 16, lane), kq[ks], o[t]);
          }
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) dQt[(qkp * 32 + 16 * t + 4 * lq + e) * C::PDQ + 16 * qct + c] = o[t][e];
      }
    }
    if (EXTRA && kl != nullptr && idx_now && threadIdx.x < 32) {
      const int id = tg[kQryId * 32 + threadIdx.x];
      if ((unsigned)id < (unsigned)n_grows) atomicAdd(&kl[id], tgf[kQryKl * 32 + threadIdx.x]);
    }
    store_step(st + 1);
  }
  // The lane's LDS offsets for the last step and the flush are recomputed
  // past the loop rather than kept in registers through it, where the plain
  // instances would spill them (the instances with per-score outputs spill
  // less without this).
  if constexpr (!EXTRA)
    asm volatile("" : "+v"(lane), "+v"(c), "+v"(lq), "+v"(wave), "+v"(qct), "+v"(qkp), "+v"(ict), "+v"(ikp));
  dq_idx_step(n_steps - 1);   // its dz^T was completed by the loop's last barrier
  if constexpr (C::KPQ > 1) {
    __syncthreads();          // the last step's dQ tile complete
    dq_store(n_steps - 1);
  }

  // Flush the wave's dK, dV (group g) and dk_idx (shared by the groups):
  // C layout [d rows][16 keys] -> LDS [16 keys][d] -> atomics of whole key rows.
  float* scr = reinterpret_cast<float*>(smem) + wave * 16 * (D + 4);
  auto flush = [&](const f32x4* acc, int ntile, int width, float* dst_row0, size_t row_stride) {
    __syncthreads();
    for (int dt = 0; dt < ntile; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) scr[c * (D + 4) + 16 * dt + 4 * lq + e] = acc[dt][e];
    __syncthreads();
    for (int i = lane; i < 16 * width; i += 64) {
      const int kr = i / width, col = i % width;
      atomicAdd(dst_row0 + (size_t)kr * row_stride + col, scr[kr * (D + 4) + col]);
    }
  };
  const size_t kv0 = ((size_t)b * N + (size_t)j * kBlock + 16 * wave) * H_kv + g;   // wave's first key row
  flush(acc_dk, DT, D, dk_acc + kv0 * D, (size_t)H_kv * D);
  flush(acc_dv, DT, D, dv_acc + kv0 * D, (size_t)H_kv * D);
  flush(acc_dki, DTI, DIDX, dk_idx + ((size_t)b * N + (size_t)j * kBlock + 16 * wave) * DIDX, (size_t)DIDX);
}

// dq of every (query, head) of a query chunk: the sum, in fp32, of its bf16
// partials over the valid slots of its selection (one partial per selected
// block, written by the main kernel; layout [b, query, slot, head, d], so the
// heads of one query and slot are contiguous on both sides).  D / 8 lanes per
// row, 16 bytes each.  KM >= topk is the compile-time slot count: all partial
// loads of the row are issued at once (slot indices past topk clamped to the
// last slot and skipped), so a row costs one memory round trip (two at
// KM = 64, whose loads go in chunks of 32).  Padded slots
// hold unwritten memory and are excluded by selection.  Row indices fit in 32
// bits (checked by the host).
template <int D, int KM>
__global__ __launch_bounds__(256) void dq_merge_kernel(const bf16* __restrict__ part,
                                                       const int32_t* __restrict__ block_idx, bf16* __restrict__ dq,
                                                       int B, int N, int H_kv, int G, int topk, int c0, int CQ) {
  constexpr int LPR = D / 8;
  const int H_q = H_kv * G;
  const int row = blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  if (row >= B * CQ * H_q) return;
  const int col = (threadIdx.x % LPR) * 8;
  const int h = row % H_q;
  const int bt = row / H_q;
  const int tl = bt % CQ, b = bt / CQ;
  const int t = c0 + tl, g = h / G;
  const int32_t* brow = block_idx + (((size_t)b * N + t) * H_kv + g) * topk;
  const bf16* prow = part + ((size_t)bt * topk * H_q + h) * D + col;   // slot e at + e H_q D
  // Partial loads in flight: all of the row's (KM <= 32), else chunks of 32.
  constexpr int KC = KM > 32 ? 32 : KM;
  bf16x8 raw[KC];
  auto load_chunk = [&](int e0) {
#pragma unroll
    for (int e = 0; e < KC; ++e)   // streaming loads: each partial is read once
      raw[e] = __builtin_nontemporal_load(
          reinterpret_cast<const bf16x8*>(prow + (size_t)min(e0 + e, topk - 1) * H_q * D));
  };
  load_chunk(0);
  bool ok[KM];
  if (topk == KM) {
#pragma unroll
    for (int e = 0; e < KM; e += 4) {
      const int4 bi = *reinterpret_cast<const int4*>(brow + e);
      ok[e] = bi.x >= 0; ok[e + 1] = bi.y >= 0; ok[e + 2] = bi.z >= 0; ok[e + 3] = bi.w >= 0;
    }
  } else {
#pragma unroll
    for (int e = 0; e < KM; ++e) ok[e] = e < topk && brow[min(e, topk - 1)] >= 0;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int e0 = 0; e0 < KM; e0 += KC) {
    if (e0 > 0) load_chunk(e0);
#pragma unroll
    for (int e = 0; e < KC; ++e)
      if (ok[e0 + e])
#pragma unroll
        for (int k2 = 0; k2 < 8; ++k2) acc[k2] += (float)raw[e][k2];
  }
  bf16x8 y;
#pragma unroll
  for (int k2 = 0; k2 < 8; ++k2) y[k2] = (bf16)acc[k2];
  *reinterpret_cast<bf16x8*>(dq + (((size_t)b * N + t) * H_q + h) * D + col) = y;
}

template <int D>
hipError_t launch_dq_merge(const Problem& P, const bf16* part, const int32_t* block_idx, bf16* dq, int c0, int CQ,
                           hipStream_t s) {
  const size_t rows = (size_t)P.B * CQ * P.H_q;
  if (rows > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int rpb = 256 / (D / 8);
  const unsigned blocks = (unsigned)((rows + rpb - 1) / rpb);
  auto kern = P.topk <= 4 ? dq_merge_kernel<D, 4>
            : P.topk <= 8 ? dq_merge_kernel<D, 8>
            : P.topk <= 16 ? dq_merge_kernel<D, 16>
            : P.topk <= 32 ? dq_merge_kernel<D, 32> : dq_merge_kernel<D, 64>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, part, block_idx, dq, P.B, P.N, P.H_kv, P.G, P.topk, c0,
                     CQ);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float* __restrict__ src, bf16* __restrict__ dst,
                                                          size_t n) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 x = *reinterpret_cast<const float4*>(src + i);
    bf16x4 y;
    y[0] = (bf16)x.x; y[1] = (bf16)x.y; y[2] = (bf16)x.z; y[3] = (bf16)x.w;
    *reinterpret_cast<bf16x4*>(dst + i) = y;
  } else {
    for (size_t k2 = i; k2 < n; ++k2) dst[k2] = (bf16)src[k2];
  }
}

hipError_t to_bf16(const float* src, void* dst, size_t n, hipStream_t s) {
  const size_t blocks = (n / 4 + 255) / 256 + 1;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, src, static_cast<bf16*>(dst), n);
  return hipGetLastError();
}

template <int D, int DIDX, int G>
hipError_t run_main(const Problem& P, const BwdArgs& a, const BlockMap& m, const BwdScratch& w, int grid,
                    int c0, int CQ, int s_lo, int s_hi, int item_q, hipStream_t s) {
  using C = Bwd16Cfg<D, DIDX>;
  // The optional per-score outputs get their own instantiation so that the
  // plain training path carries none of their registers.
  auto kern = (a.dscore != nullptr || a.kl != nullptr) ? bwd_main16_kernel<D, DIDX, G, true>
                                                       : bwd_main16_kernel<D, DIDX, G, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kT16), C::LDS, s, static_cast<const bf16*>(a.q),
                     static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dO),
                     a.lse, w.D, static_cast<const bf16*>(a.q_idx), static_cast<const bf16*>(a.k_idx), w.lse_idx,
                     a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.dq_part, w.dk_acc, w.dv_acc, a.dq_idx,
                     a.dk_idx, a.dscore, a.kl, P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb,
                     P.B * P.H_kv * P.nblk, P.scale, P.scale_idx, a.kl_weight, P.B * CQ * P.H_q * P.topk,
                     P.B * P.N * P.H_kv, c0, CQ, s_lo, s_hi, item_q);
  return hipGetLastError();
}

template <int D, int DIDX>
hipError_t run_main_g(const Problem& P, const BwdArgs& a, const BlockMap& m, const BwdScratch& w, int grid, int c0,
                      int CQ, int s_lo, int s_hi, int item_q, hipStream_t s) {
  switch (P.G) {
    case 1: return run_main<D, DIDX, 1>(P, a, m, w, grid, c0, CQ, s_lo, s_hi, item_q, s);
    case 2: return run_main<D, DIDX, 2>(P, a, m, w, grid, c0, CQ, s_lo, s_hi, item_q, s);
    case 4: return run_main<D, DIDX, 4>(P, a, m, w, grid, c0, CQ, s_lo, s_hi, item_q, s);
    case 8: return run_main<D, DIDX, 8>(P, a, m, w, grid, c0, CQ, s_lo, s_hi, item_q, s);
    case 16: return run_main<D, DIDX, 16>(P, a, m, w, grid, c0, CQ, s_lo, s_hi, item_q, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// List entries per backward work item for a query chunk of CQ queries: the
// largest of 4096, 2048, 1024 that still gives at least 24 items per CU for
// lists of the average length (a chunk's lists hold about (topk - 1) entries
// per query and group).  Longer items flush dK, dV and dk_idx less often;
// enough of them keep the CUs evenly loaded (measured: 4096 is 1% faster at
// N = 128K, and 9% slower than 1024 at B = 4, N = 8K, where it leaves 8
// items per CU).
static int bwd_item_queries(const Problem& P, int CQ) {
  const double lists = (double)P.B * P.H_kv * P.nblk;
  const double avg_len = (double)P.B * P.H_kv * CQ * (P.topk - 1) / lists;
  for (int q = kBigItem; q > 1024; q /= 2)
    if (lists * std::ceil(avg_len / q) >= 24.0 * 256) return q;
  return 1024;
}

int bwd_chunk_queries(const Problem& P) {
  // Queries per chunk of the main kernel: their dQ partials (bf16, one row per
  // (query, slot, head)) must fit in 40 GiB (one chunk at N = 128K with 64
  // heads); a multiple of the block map's super-block span, since chunks select
  // list entries by super-block.
  const size_t per_query = (size_t)P.B * P.H_q * P.topk * P.d * 2;
  const size_t cap = size_t(40) << 30;
  const size_t span = (size_t)block_map_super_span(P);
  size_t q = cap / per_query;
  q -= q % span;
  if (q < span) q = span;
  if (q >= (size_t)P.N) q = P.N;
  return (int)q;
}

size_t sparse_bwd_scratch_bytes(const Problem& P) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows_q = (size_t)P.B * P.N * P.H_q;
  const size_t rows_g = (size_t)P.B * P.N * P.H_kv;
  const size_t part_rows = (size_t)P.B * bwd_chunk_queries(P) * P.H_q * P.topk + 1;   // + the spare row
  return al(rows_q * 4) + al(rows_g * P.topk * 8) + al(rows_g * 4) + al(part_rows * P.d * 2) +
         2 * al(rows_g * P.d * 4);
}

void sparse_bwd_scratch_carve(const Problem& P, void* ws, BwdScratch* w) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows_q = (size_t)P.B * P.N * P.H_q;
  const size_t rows_g = (size_t)P.B * P.N * P.H_kv;
  const size_t part_rows = (size_t)P.B * bwd_chunk_queries(P) * P.H_q * P.topk + 1;
  char* p = static_cast<char*>(ws);
  w->D = reinterpret_cast<float*>(p);
  p += al(rows_q * 4);
  w->idx_part = reinterpret_cast<float2*>(p);
  p += al(rows_g * P.topk * 8);
  w->lse_idx = reinterpret_cast<float*>(p);
  p += al(rows_g * 4);
  w->dq_part = reinterpret_cast<bf16*>(p);
  p += al(part_rows * P.d * 2);
  w->dk_acc = reinterpret_cast<float*>(p);
  p += al(rows_g * P.d * 4);
  w->dv_acc = reinterpret_cast<float*>(p);
}

hipError_t launch_sparse_bwd(const Problem& P, const BwdArgs& a, const BlockMap& m, const BwdScratch& w,
                             hipStream_t s) {
  hipError_t e;
  const size_t rows_q = (size_t)P.B * P.N * P.H_q;
  const size_t rows_g = (size_t)P.B * P.N * P.H_kv;
  // Zero every accumulator (fill kernels: safe inside captured graphs).
  {
  ProfScope prof("bwd_prep", s);
  if ((e = launch_fill_f32(w.dk_acc, rows_g * P.d, 0.f, s)) != hipSuccess) return e;
  if ((e = launch_fill_f32(w.dv_acc, rows_g * P.d, 0.f, s)) != hipSuccess) return e;
  if ((e = launch_fill_f32(a.dq_idx, rows_g * P.d_idx, 0.f, s)) != hipSuccess) return e;
  if ((e = launch_fill_f32(a.dk_idx, (size_t)P.B * P.N * P.d_idx, 0.f, s)) != hipSuccess) return e;
  if (a.dscore && (e = launch_fill_f32(a.dscore, rows_g * P.topk * kBlock, 0.f, s)) != hipSuccess) return e;
  if (a.kl && (e = launch_fill_f32(a.kl, rows_g, 0.f, s)) != hipSuccess) return e;
  // D = rowsum(dO * O).
  {
    const int lpr = P.d / 8;
    const size_t blocks = (rows_q + (256 / lpr) - 1) / (256 / lpr);
    if (P.d == 128)
      hipLaunchKernelGGL(bwd_rowdot_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, s,
                         static_cast<const bf16*>(a.dO), static_cast<const bf16*>(a.o), w.D, rows_q);
    else
      hipLaunchKernelGGL(bwd_rowdot_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, s,
                         static_cast<const bf16*>(a.dO), static_cast<const bf16*>(a.o), w.D, rows_q);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  }
  // Index log-sum-exp over the selected support (items of <= kLseItem queries).
  if ((e = launch_block_items(P, m, 0, P.N, kLseItem, s)) != hipSuccess) return e;
  size_t grid = block_items_upper_bound(P, 0, P.N, kLseItem);
  grid = (grid + 7) & ~size_t(7);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int n_lists = P.B * P.H_kv * P.nblk;
  {
  ProfScope prof("bwd_idx_lse", s);
  if (P.d_idx == 64)
    hipLaunchKernelGGL(idx_lse_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16*>(a.q_idx),
                       static_cast<const bf16*>(a.k_idx), a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.idx_part,
                       P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb, n_lists, P.scale_idx);
  else
    hipLaunchKernelGGL(idx_lse_kernel<32>, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16*>(a.q_idx),
                       static_cast<const bf16*>(a.k_idx), a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.idx_part,
                       P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb, n_lists, P.scale_idx);
  {
    if (rows_g > 0x1fffffff) return hipErrorInvalidConfiguration;
    auto mk = P.topk <= 4 ? idx_lse_merge_kernel<4>
            : P.topk <= 8 ? idx_lse_merge_kernel<8>
            : P.topk <= 16 ? idx_lse_merge_kernel<16>
            : P.topk <= 32 ? idx_lse_merge_kernel<32> : idx_lse_merge_kernel<64>;
    hipLaunchKernelGGL(mk, dim3((unsigned)((rows_g * 4 + 255) / 256)), dim3(256), 0, s, w.idx_part, a.block_idx,
                       w.lse_idx, (int)rows_g, P.topk);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // Main kernel per query chunk (long items: own queries + up to item_q
  // list entries), then the chunk's dq from its partials.
  const int chunk = bwd_chunk_queries(P);
  const int span = block_map_super_span(P);
  for (int c0 = 0; c0 < P.N; c0 += chunk) {
    const int c1 = c0 + chunk < P.N ? c0 + chunk : P.N;
    const int CQ = c1 - c0;
    const int item_q = bwd_item_queries(P, CQ);
    if ((e = launch_block_items(P, m, c0, c1, item_q, s, 1)) != hipSuccess) return e;
    size_t g2 = block_items_upper_bound(P, c0, c1, item_q);
    g2 = (g2 + 7) & ~size_t(7);
    if (g2 > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int s_lo = c0 / span;
    const int s_hi = (c1 == P.N) ? m.nsb : c1 / span;
    {
      ProfScope prof("bwd_main", s);
      if (P.d == 128 && P.d_idx == 64) e = run_main_g<128, 64>(P, a, m, w, (int)g2, c0, CQ, s_lo, s_hi, item_q, s);
      else if (P.d == 128) e = run_main_g<128, 32>(P, a, m, w, (int)g2, c0, CQ, s_lo, s_hi, item_q, s);
      else if (P.d_idx == 64) e = run_main_g<64, 64>(P, a, m, w, (int)g2, c0, CQ, s_lo, s_hi, item_q, s);
      else e = run_main_g<64, 32>(P, a, m, w, (int)g2, c0, CQ, s_lo, s_hi, item_q, s);
      if (e != hipSuccess) return e;
    }
    {
      ProfScope prof("bwd_dq_merge", s);
      e = P.d == 128 ? launch_dq_merge<128>(P, w.dq_part, a.block_idx, static_cast<bf16*>(a.dq), c0, CQ, s)
                     : launch_dq_merge<64>(P, w.dq_part, a.block_idx, static_cast<bf16*>(a.dq), c0, CQ, s);
      if (e != hipSuccess) return e;
    }
  }
  // fp32 accumulators to bf16 outputs.
  ProfScope prof("bwd_finalize", s);
  if ((e = to_bf16(w.dk_acc, a.dk, rows_g * P.d, s)) != hipSuccess) return e;
  return to_bf16(w.dv_acc, a.dv, rows_g * P.d, s);
}

}  // namespace msa
