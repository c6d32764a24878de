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
//   bwd_main_kernel      per work item (KV block j of group g, <= 1024 + 128
//                        queries that selected it): 4 waves, wave w owns keys
//                        32w..32w+31 and keeps dK, dV, dk_idx of those keys in
//                        registers; per 32 (query, head) rows it rebuilds
//                        S = Q K^T and P, dP = dO V^T, dS = P (dP - D), the
//                        index logits, p_px and the head-averaged teacher
//                        pbar, dz = lam (p_px - pbar); dS and dz go through LDS
//                        to form dQ = dS K and dq_idx = dz K_idx (fp32
//                        atomics); the block's dK, dV, dk_idx are added once
//                        per item.
//   bwd_finalize_kernel  fp32 accumulators -> bf16 dq, dk, dv.
#include "msa_internal.h"

#include <type_traits>

namespace msa {
namespace {

constexpr int kItemQueries = 128;

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
    const int e0 = (local - 1) * kItemQueries;
    it->nq = min(kItemQueries, seg1 - e0);
    it->ent = rows + (size_t)bg * N * topk + offs[(size_t)bg * (nblk + 1) + it->j] + e0;
  }
  return true;
}

// Query t and slot of item-local query qi (clamped, with a validity flag).
__device__ inline void item_query(const Item& it, int qi, const int32_t* __restrict__ block_idx, int N, int H_kv,
                                  int topk, int* t, int* slot, bool* valid) {
  *valid = qi < it.nq;
  const int qc = min(qi, it.nq - 1);
  if (it.diag) {
    *t = it.j * kBlock + qc;
    const int32_t* brow = block_idx + (((size_t)it.b * N + *t) * H_kv + it.g) * topk;
    int s = 0;
    for (int e = 0; e < topk; ++e)
      if (brow[e] == it.j) s = e;
    *slot = s;
  } else {
    const int e = it.ent[qc];
    *t = e >> 6;
    *slot = e & 63;
    if (*t < 0 || *t >= N || *slot >= topk) {
      *valid = false;
      *t = 0;
      *slot = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// Index log-sum-exp over the selected support, per (b, t, g): KV-outer
// partials (max, sum) per slot, then a merge.
// ---------------------------------------------------------------------------
template <int DIDX>
__global__ __launch_bounds__(256) void idx_lse_kernel(
    const bf16* __restrict__ q_idx, const bf16* __restrict__ k_idx, const int32_t* __restrict__ block_idx,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ offs, const int32_t* __restrict__ rows,
    const int32_t* __restrict__ tiles, float2* __restrict__ part, int N, int H_kv, int topk, int causal,
    int nblk, int nsb, int n_lists, float scale_idx) {
  constexpr int PK = DIDX + 8;
  constexpr int KSTEPS = DIDX / 16;
  __shared__ __align__(16) bf16 Ks[kBlock * PK];
  Item it;
  if (!decode_item(tiles, pos, offs, rows, n_lists, N, H_kv, topk, nblk, nsb, &it)) return;
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
  const int qi = wave * 32 + (lane & 31);
  if (wave * 32 >= it.nq) return;
  int t, slot;
  bool valid;
  item_query(it, qi, block_idx, N, H_kv, topk, &t, &slot, &valid);
  bf16x8 qf[KSTEPS];
  const bf16* qrow = q_idx + (((size_t)it.b * N + t) * H_kv + it.g) * DIDX + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 16);
  f32x16 s[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    s[mt] = zero16();
    const bf16* kp = Ks + (mt * 32 + (lane & 31)) * PK + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kp + ks * 16), qf[ks],
                                                       s[mt], 0, 0, 0);
  }
  const float c = scale_idx * kLog2e;
  float m = -INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const bool vis = !(it.diag && causal && it.j * kBlock + mt * 32 + c_row(v, lane) > t);
      s[mt][v] = vis ? s[mt][v] * c : -INFINITY;
      m = fmaxf(m, s[mt][v]);
    }
  m = fmaxf(m, swap_half(m));
  float l = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v = 0; v < 16; ++v) l += exp2f(s[mt][v] - m);
  l += swap_half(l);
  if (valid && lane < 32) part[(((size_t)it.b * N + t) * H_kv + it.g) * topk + slot] = make_float2(m, l);
}

// lse_idx (natural log) from the per-slot partials (log2-domain max, sum).
__global__ __launch_bounds__(256) void idx_lse_merge_kernel(const float2* __restrict__ part,
                                                            const int32_t* __restrict__ block_idx,
                                                            float* __restrict__ lse_idx, size_t rows, int topk) {
  const size_t r = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int32_t* brow = block_idx + r * topk;
  const float2* p = part + r * topk;
  float m = -INFINITY;
  for (int e = 0; e < topk; ++e)
    if (brow[e] >= 0) m = fmaxf(m, p[e].x);
  float l = 0.f;
  for (int e = 0; e < topk; ++e)
    if (brow[e] >= 0) l += p[e].y * exp2f(p[e].x - m);
  lse_idx[r] = (m + log2f(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Main fused backward.  4 waves; wave w owns keys 32w..32w+31 of the block.
// 32x32x16 MFMA tiles (C-layout: lane l holds column l % 32, rows
// 8*(v/4) + 4*(l/32) + v%4 in slot v; A/B operands: lane l holds row/column
// l % 32 and k = 8*(l/32) + i).  Per step of 32 (query, head) rows:
//   S = Q K_w^T, dP = dO V_w^T          (A from LDS tiles, B in registers)
//   P, dS                               (lane = key, slots = rows)
//   dV_w^T += dO^T P, dK_w^T += Q^T dS  (A from transposed LDS tiles, B = the
//                                        P / dS registers as they are)
//   index logits, p_px, teacher, dz, dk_idx_w^T += q_idx^T dz
//   dQ[:, 32w..32w+31] = dS K, dq_idx = dz K_idx  (K^T / K_idx^T operands of
//                                        the wave's output columns in registers)
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 4;
constexpr int kMainThreads = kBwdWaves * kWave;

// Work items of the main kernel: the queries of KV block j (its own 128, with
// the causal mask) together with the first kBigItem entries of its inverted
// list, or a later run of kBigItem list entries.  Long items keep the
// per-item flush of dK, dV and dk_idx rare.
constexpr int kBigItem = 1024;

// Per-step tables (32 entries each) in LDS, double buffered.
enum : int {
  kRowT = 0,     // t of the row, -1 past the item's end
  kRowCut,       // key u is visible to the row iff u <= cut (-1: none)
  kRowLse,       // LSE * log2(e)
  kRowD,         // rowsum(dO * O)
  kRowId,        // (b N + t) H_q + h, or -1
  kQryT,         // per query of the step: t or -1
  kQrySlot,      // position of block j in the query's selection
  kQryCut,       // visibility cut-off of the query (-1: none)
  kQryLse,       // index LSE * log2(e)
  kQryKl,        // KL partial (optional output)
  kQryId,        // (b N + t) H_kv + g, or -1
  kNumTabs
};

// Row-major bf16 tiles in LDS.  Pad<P>: rows of P elements.  Swz128: rows of
// 128 elements (256 B, no padding) whose 16-byte chunk c of row r is stored at
// chunk c ^ (4 (r & 3) + ((r >> 2) & 3)); a read of one chunk from each of 16
// consecutive rows and a transpose read of 4 consecutive rows x 2 chunks then
// both touch 16 distinct chunks, so neither has an LDS bank conflict.
template <int P>
struct Pad {
  static constexpr int pitch = P;
  __device__ static int off(int r, int c) { return r * P + c; }
};
struct Swz128 {
  static constexpr int pitch = 128;
  __device__ static int off(int r, int c) {   // c: a multiple of 4
    return r * 128 + (((c >> 3) ^ (4 * (r & 3) + ((r >> 2) & 3))) << 3) + (c & 7);
  }
};
template <int W>
using TileOf = typename std::conditional<W == 128, Swz128, Pad<W + 8>>::type;

template <int D, int DIDX>
struct BwdCfg {
  using TQ = TileOf<D>;                    // Q, dO, K, V tiles
  using TI = Pad<DIDX + 8>;                // q_idx, K_idx tiles
  using TS = Pad<32 + 4>;                  // dS^T, dz^T: one row of 32 step rows per key
  static constexpr int PQ = TQ::pitch;
  static constexpr int PQI = TI::pitch;
  static constexpr int PST = TS::pitch;
  static constexpr size_t OFF_QS = 0;                                    // Q        [32][PQ]
  static constexpr size_t OFF_DOS = OFF_QS + (size_t)32 * PQ * 2;        // dO       [32][PQ]
  static constexpr size_t OFF_QIS = OFF_DOS + (size_t)32 * PQ * 2;       // q_idx    [32][PQI]
  static constexpr size_t OFF_DST = OFF_QIS + (size_t)32 * PQI * 2;      // dS^T     [128][PST]
  static constexpr size_t OFF_DZT = OFF_DST + (size_t)kBlock * PST * 2;  // dz^T     2 x [128][PST]
  static constexpr size_t OFF_TAB = OFF_DZT + (size_t)2 * kBlock * PST * 2;   // 2 x kNumTabs x [32]
  static constexpr size_t OFF_KS = OFF_TAB + (size_t)2 * kNumTabs * 32 * 4;   // K of the block  [128][PQ]
  static constexpr size_t OFF_VS = OFF_KS + (size_t)kBlock * PQ * 2;     // V of the block     [128][PQ]
  static constexpr size_t OFF_KIS = OFF_VS + (size_t)kBlock * PQ * 2;    // K_idx of the block [128][PQI]
  static constexpr size_t OFF_QL = OFF_KIS + (size_t)kBlock * PQI * 2;   // item queries: (t << 6) | slot
  static constexpr size_t LDS = OFF_QL + (size_t)(kBlock + kBigItem) * 4;
  // The flush at the end of an item reuses [OFF_QS, OFF_TAB) as 4 x [32][33] fp32.
  static_assert(OFF_TAB - OFF_QS >= 4 * 32 * 33 * 4, "flush scratch");
  static_assert(LDS <= 160 * 1024, "LDS of one CU");
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
                                       int n_lists, int N, int H_kv, int topk, int nblk, int nsb, BigItem* it) {
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
  const int len = pos[((size_t)bg * (nsb + 1) + nsb) * nblk + it->j];
  it->n_own = li == 0 ? kBlock : 0;
  it->e0 = li * kBigItem;
  it->ne = max(0, min(kBigItem, len - it->e0));
  it->ent = rows + (size_t)bg * N * topk + offs[(size_t)bg * (nblk + 1) + it->j];
  return true;
}

// t (-1 when qi is past the item) and, when asked, the slot of block j in the
// query's row.
__device__ inline int big_query(const BigItem& it, int qi, const int32_t* __restrict__ block_idx, int N, int H_kv,
                                int topk, bool want_slot, int* slot) {
  *slot = 0;
  if (qi < it.n_own) {
    const int t = it.j * kBlock + qi;
    if (want_slot) {
      const int32_t* brow = block_idx + (((size_t)it.b * N + t) * H_kv + it.g) * topk;
      for (int e = 0; e < topk; ++e)
        if (brow[e] == it.j) *slot = e;
    }
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

// A operand X^T of a 32x32x16 MFMA read straight from a row-major [rows][cols]
// bf16 LDS tile of layout L with the gfx950 transpose read (within each group of 16
// lanes, lane i receives element i % 4 of the vectors addressed by lanes
// 4k + i / 4, k = 0..3; checked on hardware): lane l gets column m0 + l % 32
// and the K values of rows r0 .. r0+3 (slots 0..3) and r0+8 .. r0+11
// (slots 4..7), with r0 = 16 kc + 4 (l / 32) - the row order of a C-layout
// tile's slots 8 kc .. 8 kc + 7.
template <class L>
__device__ inline bf16x8 trfrag(const bf16* base, int m0, int kc, int lane) {
  const int jj = lane & 15;
  const int r0 = 16 * kc + 4 * (lane >> 5) + (jj >> 2);
  const int col = m0 + 16 * ((lane >> 4) & 1) + 4 * (jj & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + L::off(r0, col)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + L::off(r0 + 8, col)));
  const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
  bf16x8 r;
  r[0] = l4[0]; r[1] = l4[1]; r[2] = l4[2]; r[3] = l4[3];
  r[4] = h4[0]; r[5] = h4[1]; r[6] = h4[2]; r[7] = h4[3];
  return r;
}
// Matching B operand: slots 8kc .. 8kc+7 of a C-layout tile.
__device__ inline bf16x8 cfrag(const f32x16& x, int kc) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)x[8 * kc + i];
  return r;
}
__device__ inline f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline bf16x4 pack4(float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (bf16)a; r[1] = (bf16)b; r[2] = (bf16)c; r[3] = (bf16)d;
  return r;
}
// x of lane l % 32 (lo) and of lane l % 32 + 32 (hi), in every lane.
__device__ inline void halves(float x, float* lo, float* hi) {
  const auto v = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  *lo = __uint_as_float(v[0]);
  *hi = __uint_as_float(v[1]);
}

// Mean over the G heads of each query of a 32-row C-layout tile whose row
// q G + e is head e of query q, returned in the C layout of a tile whose rows
// are the queries (slot v of half hf holds query c_row(v, hf)); slots that hold
// no query of the step are left 0.
template <int G>
__device__ inline f32x16 head_mean(const f32x16& p, int hf) {
  f32x16 r = zero16();
  constexpr float inv = 1.0f / G;
  if constexpr (G == 1) {
    r = p;
  } else if constexpr (G >= 8) {
    // rows qG .. qG+G-1: slots [q G/2, (q+1) G/2) of both halves
    constexpr int H2 = G / 2;
#pragma unroll
    for (int q = 0; q < 32 / G; ++q) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < H2; ++e) s += p[q * H2 + e];
      float lo, hi;
      halves(s, &lo, &hi);
      r[q] = (lo + hi) * inv;
    }
  } else if constexpr (G == 4) {
    // slots 4gi .. 4gi+3 of half h: query 2gi + h
    float x0[4], x1[4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) halves(p[4 * gi] + p[4 * gi + 1] + p[4 * gi + 2] + p[4 * gi + 3], &x0[gi], &x1[gi]);
#pragma unroll
    for (int v = 0; v < 4; ++v) {   // query 4 hf + v
      const float* x = (v & 1) ? x1 : x0;
      r[v] = (hf ? x[2 + (v >> 1)] : x[v >> 1]) * inv;
    }
  } else {
    static_assert(G == 2, "group size");
    // slots 4gi + 2k, 4gi + 2k + 1 of half h: query 4gi + 2h + k
    float y0[4][2], y1[4][2];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        halves(p[4 * gi + 2 * k2] + p[4 * gi + 2 * k2 + 1], &y0[gi][k2], &y1[gi][k2]);
#pragma unroll
    for (int v = 0; v < 8; ++v) {   // query 8 (v / 4) + 4 hf + v % 4
      const int g0 = 2 * (v >> 2);
      const float a = ((v >> 1) & 1) ? y1[g0][v & 1] : y0[g0][v & 1];
      const float c = ((v >> 1) & 1) ? y1[g0 + 1][v & 1] : y0[g0 + 1][v & 1];
      r[v] = (hf ? c : a) * inv;
    }
  }
  return r;
}

// ---------------------------------------------------------------------------
// Main fused backward.  4 waves; wave w owns keys 32w..32w+31 of the block.
// 32x32x16 MFMA tiles (C-layout: lane l holds column l % 32, rows
// 8*(v/4) + 4*(l/32) + v%4 in slot v; A/B operands: lane l holds row/column
// l % 32 and k = 8*(l/32) + i).  Per step of 32 (query, head) rows:
//   S = Q K_w^T, dP = dO V_w^T, r = q_idx K_idx,w^T  (A and B from LDS tiles)
//   P, dS; the head-mean teacher pbar, p_px and dz    (lane = key, all in registers)
//   dV_w^T += dO^T P, dK_w^T += Q^T dS, dk_idx_w^T += q_idx^T dz
//   dS^T, dz^T -> LDS; barrier
//   dQ[:, 32w..32w+31] = dS K and dq_idx = dz K_idx  (A and B by transpose reads of
//                                        dS^T / dz^T and of the K / K_idx tiles)
// The block's K, V and K_idx stay in LDS for the whole item and every MFMA
// operand is read from LDS, which leaves the registers to the accumulators
// and to operands fetched ahead of their MFMAs.
// ---------------------------------------------------------------------------
template <int D, int DIDX, int G, bool EXTRA>
__global__ __launch_bounds__(kMainThreads, 1) void bwd_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dv,
    const bf16* __restrict__ q_idx, const bf16* __restrict__ k_idx, const float* __restrict__ lse_idx,
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ pos, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ tiles, float* __restrict__ dq_acc,
    float* __restrict__ dk_acc, float* __restrict__ dv_acc, float* __restrict__ dq_idx,
    float* __restrict__ dk_idx, float* __restrict__ dscore, float* __restrict__ kl, int N, int H_kv, int topk,
    int causal, int nblk, int nsb, int n_lists, float scale, float scale_idx, float lam) {
  using C = BwdCfg<D, DIDX>;
  constexpr int KS = D / 16;        // 16-wide k-steps over d
  constexpr int KSI = DIDX / 16;    // 16-wide k-steps over d_idx
  constexpr int DT = D / 32;        // 32-wide d tiles
  constexpr int DTI = DIDX / 32;    // 32-wide d_idx tiles
  constexpr int TQ = 32 / G;        // queries per 32-row step
  constexpr int KCQ = TQ > 16 ? 2 : 1;                     // 16-query chunks holding real queries
  constexpr int NVQ = TQ <= 8 ? 4 : (TQ <= 16 ? 8 : 16);   // slots that can hold a query < TQ
  constexpr int CPR = D / 8;        // 16-byte chunks per Q / dO row
  constexpr int CPRI = DIDX / 8;    // 16-byte chunks per q_idx row
  constexpr int LDM = 32 * CPR / kMainThreads;              // Q (and dO) chunks per thread
  constexpr int NT = kNumTabs * 32;
  static_assert(32 * CPR % kMainThreads == 0, "tile split");
  static_assert(32 * CPRI <= kMainThreads, "q_idx tile split");
  static_assert(DT <= kBwdWaves, "one dQ column tile per wave");
  extern __shared__ __align__(16) char smem[];
  bf16* Qs = reinterpret_cast<bf16*>(smem + C::OFF_QS);
  bf16* dOs = reinterpret_cast<bf16*>(smem + C::OFF_DOS);
  bf16* QIs = reinterpret_cast<bf16*>(smem + C::OFF_QIS);
  bf16* dSt = reinterpret_cast<bf16*>(smem + C::OFF_DST);
  bf16* dZt2 = reinterpret_cast<bf16*>(smem + C::OFF_DZT);   // dz^T of steps of either parity
  int* tabs = reinterpret_cast<int*>(smem + C::OFF_TAB);
  bf16* Ks = reinterpret_cast<bf16*>(smem + C::OFF_KS);
  bf16* Vs = reinterpret_cast<bf16*>(smem + C::OFF_VS);
  bf16* KIs = reinterpret_cast<bf16*>(smem + C::OFF_KIS);
  int* qlist = reinterpret_cast<int*>(smem + C::OFF_QL);   // (t << 6) | slot, or -1

  BigItem it;
  if (!decode_big_item(tiles, pos, offs, rows, n_lists, N, H_kv, topk, nblk, nsb, &it)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, hf = lane >> 5;
  const int H_q = H_kv * G;
  const int b = it.b, g = it.g, j = it.j;
  const int key = 32 * wave + n;                      // this lane's key inside the block
  const int u = j * kBlock + key;
  const size_t blk_row0 = ((size_t)b * N + (size_t)j * kBlock) * H_kv + g;   // key 0 of the block
  const int nq = it.n_own + it.ne;
  const bool want_slot = EXTRA && dscore != nullptr;

  // The item's queries in LDS, so that the step loop needs no dependent
  // global load (the vector-memory counter is in order: a wait on a
  // dependent load would also wait for the previous step's atomics).
  for (int qi = threadIdx.x; qi < nq; qi += kMainThreads) {
    int slot;
    const int t = big_query(it, qi, block_idx, N, H_kv, topk, want_slot, &slot);
    qlist[qi] = t < 0 ? -1 : ((t << 6) | slot);
  }
  // K, V and K_idx of the block in LDS, row-major (one row per key).
  for (int c = threadIdx.x; c < kBlock * CPR; c += kMainThreads) {
    const int kk = c / CPR, col = (c % CPR) * 8;
    const size_t row = blk_row0 + (size_t)kk * H_kv;
    *reinterpret_cast<bf16x8*>(Ks + C::TQ::off(kk, col)) = *reinterpret_cast<const bf16x8*>(k + row * D + col);
    *reinterpret_cast<bf16x8*>(Vs + C::TQ::off(kk, col)) = *reinterpret_cast<const bf16x8*>(v + row * D + col);
  }
  for (int c = threadIdx.x; c < kBlock * CPRI; c += kMainThreads) {
    const int kk = c / CPRI, col = (c % CPRI) * 8;
    *reinterpret_cast<bf16x8*>(KIs + C::TI::off(kk, col)) =
        *reinterpret_cast<const bf16x8*>(k_idx + ((size_t)b * N + j * kBlock + kk) * DIDX + col);
  }
  const bool has_q = DT == kBwdWaves || wave < DT;   // the wave owns dQ columns 32w..32w+31
  // dq_idx: output tile wave % DTI, over the 16-key chunks
  // [kpart * KCW, (kpart + 1) * KCW), so every wave issues the same atomics.
  constexpr int KPARTS = kBwdWaves / DTI;
  constexpr int KCW = 8 / KPARTS;
  const int itile = wave % DTI, kpart = wave / DTI;
  const int qcol = 32 * wave + n;                     // dQ column (wave < DT)

  f32x16 acc_dv[DT], acc_dk[DT], acc_dki[DTI];
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    acc_dv[i] = zero16();
    acc_dk[i] = zero16();
  }
#pragma unroll
  for (int i = 0; i < DTI; ++i) acc_dki[i] = zero16();
  __syncthreads();   // item query list and the K, V, K_idx tiles ready

  // Per-thread share of a step, loaded into registers one step ahead: LDM
  // 16-byte chunks of Q and dO (with LSE, D, cut-off and id of the rows whose
  // first chunk it holds), one chunk of q_idx, and - for threads < TQ - the
  // step's query table entry.  The loads of step st + 1 are issued at the top
  // of step st, before its atomics; the vector-memory counter completes in
  // order, so the wait for them at the end of the step covers nothing issued
  // later, as long as every memory operation in between is unconditional and
  // can be counted.  The query-list entries the loads need are read from LDS
  // one step before they are issued (pk_*).
  struct Pre {
    bf16x8 q[LDM], d[LDM], qi;
    float lse[LDM], rd[LDM], qlse;
    int t[LDM], cut[LDM], id[LDM], qt, qslot, qcut, qid;
  };
  Pre pre;
  int pk_e[LDM], pk_qi = -1, pk_qt = -1;
  const int ld_col = (threadIdx.x % CPR) * 8;
  const int ld_qr = threadIdx.x / CPRI, ld_qcol = (threadIdx.x % CPRI) * 8;
  const bool ld_idx = threadIdx.x < 32 * CPRI;
  const int tx = threadIdx.x & 31;
  auto entry = [&](int qi) { return qi < nq ? qlist[qi] : -1; };
  auto cutoff = [&](int qi, int t) { return t < 0 ? -1 : ((qi < it.n_own && causal) ? t : 0x7fffffff); };
  auto peek = [&](int st) {
#pragma unroll
    for (int c = 0; c < LDM; ++c) pk_e[c] = entry((32 * st + (threadIdx.x + c * kMainThreads) / CPR) / G);
    pk_qi = ld_qr < TQ ? entry(st * TQ + ld_qr) : -1;
    pk_qt = tx < TQ ? entry(st * TQ + tx) : -1;
  };
  // Every load below is unconditional (clamped to a valid row; past the end
  // of the item it re-reads valid rows, unused) so that the compiler can count
  // the memory operations exactly.
  auto load_step = [&](int st, Pre& x) {
#pragma unroll
    for (int c = 0; c < LDM; ++c) {
      const int r = (threadIdx.x + c * kMainThreads) / CPR;
      const int t = pk_e[c] < 0 ? -1 : (pk_e[c] >> 6);
      x.t[c] = t;
      x.cut[c] = cutoff((32 * st + r) / G, t);
      const size_t qrow = ((size_t)b * N + (t < 0 ? 0 : t)) * H_q + g * G + r % G;
      x.id[c] = t < 0 ? -1 : (int)qrow;
      x.q[c] = *reinterpret_cast<const bf16x8*>(q + qrow * D + ld_col);
      x.d[c] = *reinterpret_cast<const bf16x8*>(dO + qrow * D + ld_col);
      x.lse[c] = lse[qrow];
      x.rd[c] = Dv[qrow];
    }
    {
      const int tq = pk_qi < 0 ? -1 : (pk_qi >> 6);
      x.qi = *reinterpret_cast<const bf16x8*>(q_idx + (((size_t)b * N + (tq < 0 ? 0 : tq)) * H_kv + g) * DIDX +
                                              ld_qcol);
      if (tq < 0) x.qi = bf16x8{};
    }
    {
      x.qt = pk_qt < 0 ? -1 : (pk_qt >> 6);
      x.qslot = pk_qt < 0 ? 0 : (pk_qt & 63);
      x.qcut = cutoff(st * TQ + tx, x.qt);
      const size_t qrow = ((size_t)b * N + (x.qt < 0 ? 0 : x.qt)) * H_kv + g;
      x.qid = x.qt < 0 ? -1 : (int)qrow;
      x.qlse = lse_idx[qrow];
    }
  };
  // Store a step's prefetched registers into its LDS tiles and tables.
  auto store_step = [&](int st, const Pre& x) {
    int* tb = tabs + (st & 1) * NT;
    float* tf = reinterpret_cast<float*>(tb);
#pragma unroll
    for (int c = 0; c < LDM; ++c) {
      const int r = (threadIdx.x + c * kMainThreads) / CPR;
      *reinterpret_cast<bf16x8*>(Qs + C::TQ::off(r, ld_col)) = x.q[c];
      *reinterpret_cast<bf16x8*>(dOs + C::TQ::off(r, ld_col)) = x.d[c];
      if (ld_col == 0) {
        tb[kRowT * 32 + r] = x.t[c];
        tb[kRowCut * 32 + r] = x.cut[c];
        tf[kRowLse * 32 + r] = x.lse[c] * kLog2e;
        tf[kRowD * 32 + r] = x.rd[c];
        tb[kRowId * 32 + r] = x.id[c];
      }
    }
    if (ld_idx) *reinterpret_cast<bf16x8*>(QIs + C::TI::off(ld_qr, ld_qcol)) = x.qi;
    if (threadIdx.x < 32) {
      tb[kQryT * 32 + tx] = x.qt;
      tb[kQrySlot * 32 + tx] = x.qslot;
      tb[kQryCut * 32 + tx] = x.qcut;
      tf[kQryLse * 32 + tx] = x.qlse * kLog2e;
      tf[kQryKl * 32 + tx] = 0.f;
      tb[kQryId * 32 + tx] = x.qid;
    }
  };

  const float c_s = scale * kLog2e;
  const float c_i = scale_idx * kLog2e;
  const int n_steps = (nq * G + 31) / 32;

  // dq_idx[queries, tile] = dz K_idx over this wave's share of the keys
  // (lane = d_idx column, slots = queries), for step st.  It runs at the top
  // of step st + 1, before that step's loads are issued: its atomics are
  // conditional, so the compiler cannot count them, and there they sit
  // behind no load that has to be waited for.  dz^T is double buffered for it.
  auto dq_idx_step = [&](int st) {
    const int* tb = tabs + (st & 1) * NT;
    const bf16* dZt = dZt2 + (st & 1) * kBlock * C::PST;
    f32x16 o = zero16();
#pragma unroll
    for (int kc = 0; kc < KCW; ++kc) {
      const int kq = kpart * KCW + kc;
      o = mma32(trfrag<typename C::TS>(dZt, 0, kq, lane), trfrag<typename C::TI>(KIs, 32 * itile, kq, lane), o);
    }
    const int qid0 = max(tb[kQryId * 32], 0);
#pragma unroll
    for (int vv = 0; vv < NVQ; ++vv) {
      const int qr = c_row(vv, lane);
      if (qr < TQ) {
        const int id = tb[kQryId * 32 + qr];
        atomicAdd(dq_idx + (size_t)(id >= 0 ? id : qid0) * DIDX + 32 * itile + n, id >= 0 ? o[vv] : 0.f);
      }
    }
  };

  peek(0);
  load_step(0, pre);
  store_step(0, pre);
  peek(1);
#pragma unroll 1
  for (int st = 0; st < n_steps; ++st) {
    asm volatile("" ::: "memory");
    const int* tb = tabs + (st & 1) * NT;
    const float* tf = reinterpret_cast<const float*>(tb);
    __syncthreads();   // step st's tiles and tables in LDS; step st-1's dS^T consumed
    if (st > 0) dq_idx_step(st - 1);
    load_step(st + 1, pre);
    peek(st + 2);

    // S, dP, index logits (lane = key, slots = rows / queries).
    f32x16 s = zero16(), dp = zero16(), ri = zero16();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // S: A = Q rows (lane = row n), B = K rows (lane = key); dP likewise.
      s = mma32(*reinterpret_cast<const bf16x8*>(Qs + C::TQ::off(n, 16 * ks + 8 * hf)),
                *reinterpret_cast<const bf16x8*>(Ks + C::TQ::off(key, 16 * ks + 8 * hf)), s);
      dp = mma32(*reinterpret_cast<const bf16x8*>(dOs + C::TQ::off(n, 16 * ks + 8 * hf)),
                 *reinterpret_cast<const bf16x8*>(Vs + C::TQ::off(key, 16 * ks + 8 * hf)), dp);
    }
#pragma unroll
    for (int ks = 0; ks < KSI; ++ks)
      ri = mma32(*reinterpret_cast<const bf16x8*>(QIs + C::TI::off(n, 16 * ks + 8 * hf)),
                 *reinterpret_cast<const bf16x8*>(KIs + C::TI::off(key, 16 * ks + 8 * hf)), ri);
    // P, dS; dS^T to LDS.
    f32x16 p, ds;
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      const int r4 = 8 * grp + 4 * hf;                 // rows r4 .. r4+3 = slots 4grp .. 4grp+3
      const int4 cut = *reinterpret_cast<const int4*>(tb + kRowCut * 32 + r4);
      const float4 l2 = *reinterpret_cast<const float4*>(tf + kRowLse * 32 + r4);
      const float4 dd = *reinterpret_cast<const float4*>(tf + kRowD * 32 + r4);
      const int cuts[4] = {cut.x, cut.y, cut.z, cut.w};
      const float l2s[4] = {l2.x, l2.y, l2.z, l2.w};
      const float dds[4] = {dd.x, dd.y, dd.z, dd.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int vv = 4 * grp + e;
        const float pv = u <= cuts[e] ? __builtin_amdgcn_exp2f(s[vv] * c_s - l2s[e]) : 0.f;
        p[vv] = pv;
        ds[vv] = pv * (dp[vv] - dds[e]) * scale;
      }
      *reinterpret_cast<bf16x4*>(dSt + key * C::PST + r4) =
          pack4(ds[4 * grp], ds[4 * grp + 1], ds[4 * grp + 2], ds[4 * grp + 3]);
    }
    // Index branch on the query slots: teacher pbar (mean of P over the
    // query's heads), p_px, dz = lam (p_px - pbar); dz^T to LDS.
    const f32x16 pb = head_mean<G>(p, hf);
    f32x16 dz = zero16();
#pragma unroll
    for (int gq = 0; gq < NVQ / 4; ++gq) {
      const int r4 = 8 * gq + 4 * hf;                  // queries r4 .. r4+3 = slots 4gq .. 4gq+3
      const int4 qc = *reinterpret_cast<const int4*>(tb + kQryCut * 32 + r4);
      const float4 ql = *reinterpret_cast<const float4*>(tf + kQryLse * 32 + r4);
      const int qcs[4] = {qc.x, qc.y, qc.z, qc.w};
      const float qls[4] = {ql.x, ql.y, ql.z, ql.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int vv = 4 * gq + e;
        const float lz = ri[vv] * c_i - qls[e];       // log2 p_px
        const bool vis = u <= qcs[e];                  // -1 for rows that hold no query
        dz[vv] = vis ? lam * (__builtin_amdgcn_exp2f(lz) - pb[vv]) : 0.f;
        if (EXTRA && dscore != nullptr && vis) {
          const int qr = r4 + e;
          dscore[((((size_t)b * N + tb[kQryT * 32 + qr]) * H_kv + g) * topk + tb[kQrySlot * 32 + qr]) * kBlock +
                 key] = dz[vv];
        }
        if (EXTRA && kl != nullptr) {
          float klv = (vis && pb[vv] > 0.f) ? pb[vv] * (logf(pb[vv]) - lz * kLn2) : 0.f;
#pragma unroll
          for (int off = 16; off > 0; off >>= 1) klv += __shfl_xor(klv, off);   // over the half-wave's 32 keys
          if (n == 0 && r4 + e < TQ) atomicAdd(reinterpret_cast<float*>(tabs + (st & 1) * NT) + kQryKl * 32 + r4 + e, klv);
        }
      }
      if (r4 < TQ)
        *reinterpret_cast<bf16x4*>(dZt2 + (st & 1) * kBlock * C::PST + key * C::PST + r4) =
            pack4(dz[4 * gq] * scale_idx, dz[4 * gq + 1] * scale_idx, dz[4 * gq + 2] * scale_idx,
                  dz[4 * gq + 3] * scale_idx);
    }
    // dV^T += dO^T P, dK^T += Q^T dS, dk_idx^T += q_idx^T dz.
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const bf16x8 pbf = cfrag(p, kc), sbf = cfrag(ds, kc);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        acc_dv[dt] = mma32(trfrag<typename C::TQ>(dOs, 32 * dt, kc, lane), pbf, acc_dv[dt]);
        acc_dk[dt] = mma32(trfrag<typename C::TQ>(Qs, 32 * dt, kc, lane), sbf, acc_dk[dt]);
      }
    }
    {
      f32x16 zs;
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) zs[vv] = dz[vv] * scale_idx;
#pragma unroll
      for (int kc = 0; kc < KCQ; ++kc) {
        const bf16x8 zb = cfrag(zs, kc);
#pragma unroll
        for (int dt = 0; dt < DTI; ++dt)
          acc_dki[dt] = mma32(trfrag<typename C::TI>(QIs, 32 * dt, kc, lane), zb, acc_dki[dt]);
      }
    }
    __syncthreads();   // dS^T, dz^T and the KL partials complete

    // dQ[rows, wave's 32 columns] = dS K (this wave's share of the keys): lane
    // = output column, slots = rows, so each atomic instruction covers 32
    // consecutive floats of one row per half-wave.  A row without a query adds
    // 0 at the step's first row (always a real one) instead of branching, so
    // the number of memory operations after the loads is fixed and the wait
    // for them at the end of the step covers none of these atomics.
    if (has_q) {
      f32x16 o = zero16();
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
        o = mma32(trfrag<typename C::TS>(dSt, 0, kc, lane), trfrag<typename C::TQ>(Ks, 32 * wave, kc, lane), o);
      const int id0 = max(tb[kRowId * 32], 0);
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int4 id4 = *reinterpret_cast<const int4*>(tb + kRowId * 32 + 8 * grp + 4 * hf);
        const int ids[4] = {id4.x, id4.y, id4.z, id4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int vv = 4 * grp + e;
          atomicAdd(dq_acc + (size_t)(ids[e] >= 0 ? ids[e] : id0) * D + qcol, ids[e] >= 0 ? o[vv] : 0.f);
        }
      }
    }
    if (EXTRA && kl != nullptr && threadIdx.x < TQ && tb[kQryId * 32 + threadIdx.x] >= 0)
      atomicAdd(&kl[tb[kQryId * 32 + threadIdx.x]], tf[kQryKl * 32 + threadIdx.x]);
    // Step st + 1's tiles: nothing reads Qs / dOs / QIs or the other table set
    // after the barrier above, so this can overlap the atomics.
    store_step(st + 1, pre);
  }
  dq_idx_step(n_steps - 1);   // dz^T of the last step is complete (barrier before its dQ)

  // Flush the block's dK, dV (group g) and dk_idx (shared by the groups)
  // through LDS, so that each atomic instruction covers two 32-float runs of
  // one key row instead of 32 rows.
  float* scr = reinterpret_cast<float*>(smem + C::OFF_QS) + wave * 32 * 33;
  auto flush = [&](const f32x16& acc, float* dst_row0, size_t row_stride) {
    __syncthreads();
#pragma unroll
    for (int vv = 0; vv < 16; ++vv) scr[n * 33 + c_row(vv, lane)] = acc[vv];
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int kr = 2 * kk + hf;                      // key row of the wave
      atomicAdd(dst_row0 + (size_t)kr * row_stride + n, scr[kr * 33 + n]);
    }
  };
  const size_t kv0 = ((size_t)b * N + (size_t)j * kBlock + 32 * wave) * H_kv + g;   // wave's first key row
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    flush(acc_dk[dt], dk_acc + kv0 * D + 32 * dt, (size_t)H_kv * D);
    flush(acc_dv[dt], dv_acc + kv0 * D + 32 * dt, (size_t)H_kv * D);
  }
#pragma unroll
  for (int dt = 0; dt < DTI; ++dt)
    flush(acc_dki[dt], dk_idx + ((size_t)b * N + (size_t)j * kBlock + 32 * wave) * DIDX + 32 * dt, (size_t)DIDX);
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
                    hipStream_t s) {
  using C = BwdCfg<D, DIDX>;
  // The optional per-score outputs get their own instantiation so that the
  // plain training path carries none of their registers.
  auto kern = (a.dscore != nullptr || a.kl != nullptr) ? bwd_main_kernel<D, DIDX, G, true>
                                                       : bwd_main_kernel<D, DIDX, G, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kMainThreads), C::LDS, s, static_cast<const bf16*>(a.q),
                     static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dO),
                     a.lse, w.D, static_cast<const bf16*>(a.q_idx), static_cast<const bf16*>(a.k_idx), w.lse_idx,
                     a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.dq_acc, w.dk_acc, w.dv_acc, a.dq_idx,
                     a.dk_idx, a.dscore, a.kl, P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb,
                     P.B * P.H_kv * P.nblk, P.scale, P.scale_idx, a.kl_weight);
  return hipGetLastError();
}

template <int D, int DIDX>
hipError_t run_main_g(const Problem& P, const BwdArgs& a, const BlockMap& m, const BwdScratch& w, int grid,
                      hipStream_t s) {
  switch (P.G) {
    case 1: return run_main<D, DIDX, 1>(P, a, m, w, grid, s);
    case 2: return run_main<D, DIDX, 2>(P, a, m, w, grid, s);
    case 4: return run_main<D, DIDX, 4>(P, a, m, w, grid, s);
    case 8: return run_main<D, DIDX, 8>(P, a, m, w, grid, s);
    case 16: return run_main<D, DIDX, 16>(P, a, m, w, grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t sparse_bwd_scratch_bytes(const Problem& P) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows_q = (size_t)P.B * P.N * P.H_q;
  const size_t rows_g = (size_t)P.B * P.N * P.H_kv;
  return al(rows_q * 4) + al(rows_g * P.topk * 8) + al(rows_g * 4) + al(rows_q * P.d * 4) +
         2 * al(rows_g * P.d * 4);
}

void sparse_bwd_scratch_carve(const Problem& P, void* ws, BwdScratch* w) {
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t rows_q = (size_t)P.B * P.N * P.H_q;
  const size_t rows_g = (size_t)P.B * P.N * P.H_kv;
  char* p = static_cast<char*>(ws);
  w->D = reinterpret_cast<float*>(p);
  p += al(rows_q * 4);
  w->idx_part = reinterpret_cast<float2*>(p);
  p += al(rows_g * P.topk * 8);
  w->lse_idx = reinterpret_cast<float*>(p);
  p += al(rows_g * 4);
  w->dq_acc = reinterpret_cast<float*>(p);
  p += al(rows_q * P.d * 4);
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
  prof_begin("bwd_prep", s);
  if ((e = launch_fill_f32(w.dq_acc, rows_q * P.d, 0.f, s)) != hipSuccess) return e;
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
  prof_end(s);
  // Index log-sum-exp over the selected support (items of <= 128 queries).
  if ((e = launch_block_items(P, m, 0, P.N, kItemQueries, s)) != hipSuccess) return e;
  size_t grid = block_items_upper_bound(P, 0, P.N, kItemQueries);
  grid = (grid + 7) & ~size_t(7);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int n_lists = P.B * P.H_kv * P.nblk;
  prof_begin("bwd_idx_lse", s);
  if (P.d_idx == 64)
    hipLaunchKernelGGL(idx_lse_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16*>(a.q_idx),
                       static_cast<const bf16*>(a.k_idx), a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.idx_part,
                       P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb, n_lists, P.scale_idx);
  else
    hipLaunchKernelGGL(idx_lse_kernel<32>, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16*>(a.q_idx),
                       static_cast<const bf16*>(a.k_idx), a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.idx_part,
                       P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb, n_lists, P.scale_idx);
  hipLaunchKernelGGL(idx_lse_merge_kernel, dim3((unsigned)((rows_g + 255) / 256)), dim3(256), 0, s, w.idx_part,
                     a.block_idx, w.lse_idx, rows_g, P.topk);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // Long items (own queries + up to kBigItem list entries) for the main kernel.
  if ((e = launch_block_items(P, m, 0, P.N, kBigItem, s, 1)) != hipSuccess) return e;
  grid = block_items_upper_bound(P, 0, P.N, kBigItem);
  grid = (grid + 7) & ~size_t(7);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  // Fused main + index backward.
  prof_begin("bwd_main", s);
  if (P.d == 128 && P.d_idx == 64) e = run_main_g<128, 64>(P, a, m, w, (int)grid, s);
  else if (P.d == 128) e = run_main_g<128, 32>(P, a, m, w, (int)grid, s);
  else if (P.d_idx == 64) e = run_main_g<64, 64>(P, a, m, w, (int)grid, s);
  else e = run_main_g<64, 32>(P, a, m, w, (int)grid, s);
  prof_end(s);
  if (e != hipSuccess) return e;
  // fp32 accumulators to bf16 outputs.
  prof_begin("bwd_finalize", s);
  if ((e = to_bf16(w.dq_acc, a.dq, rows_q * P.d, s)) != hipSuccess) return e;
  if ((e = to_bf16(w.dk_acc, a.dk, rows_g * P.d, s)) != hipSuccess) return e;
  e = to_bf16(w.dv_acc, a.dv, rows_g * P.d, s);
  prof_end(s);
  return e;
}

}  // namespace msa
