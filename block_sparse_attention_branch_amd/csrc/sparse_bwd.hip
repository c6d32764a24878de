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
//   bwd_main_kernel      per work item (KV block j of group g, <= 128 queries
//                        that selected it): 4 waves, wave w owns keys
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
                                   int n_lists, int per_xcd, int N, int H_kv, int topk, int nblk, int nsb,
                                   Item* it) {
  const int w = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (w >= tiles[n_lists]) return false;
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
    int nblk, int nsb, int n_lists, float scale_idx, int per_xcd) {
  constexpr int PK = DIDX + 8;
  constexpr int KSTEPS = DIDX / 16;
  __shared__ __align__(16) bf16 Ks[kBlock * PK];
  Item it;
  if (!decode_item(tiles, pos, offs, rows, n_lists, per_xcd, N, H_kv, topk, nblk, nsb, &it)) return;
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
// Main fused backward.  16x16x32 MFMA tiles: a 16x16 output D[m][n] lives in
// 4 fp32 slots per lane, lane l holding column n = l % 16 and rows
// m = 4*(l/16) + v (checked on gfx950 hardware); A-operand lane l holds row
// l % 16, B-operand lane l column l % 16, both with k = 8*(l/16) + i.
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 8;
constexpr int kMainThreads = kBwdWaves * kWave;

template <int D, int DIDX>
struct BwdCfg {
  static constexpr int PKT = kBlock + 8;   // rows of 128 keys (+16 B)
  static constexpr int PQ = D + 8;         // Q / dO rows (+16 B)
  static constexpr int PQI = DIDX + 8;     // q_idx rows (+16 B)
  static constexpr int PR = 32 + 8;        // transposed tiles: rows of 32 (+16 B)
  static constexpr size_t OFF_KT = 0;                                   // K^T      [D][PKT]
  static constexpr size_t OFF_KIT = OFF_KT + (size_t)D * PKT * 2;       // K_idx^T  [DIDX][PKT]
  static constexpr size_t OFF_QS = OFF_KIT + (size_t)DIDX * PKT * 2;    // Q        [32][PQ]
  static constexpr size_t OFF_DOS = OFF_QS + (size_t)32 * PQ * 2;       // dO       [32][PQ]
  static constexpr size_t OFF_QT = OFF_DOS + (size_t)32 * PQ * 2;       // Q^T      [D][PR]
  static constexpr size_t OFF_DOT = OFF_QT + (size_t)D * PR * 2;        // dO^T     [D][PR]
  static constexpr size_t OFF_QIS = OFF_DOT + (size_t)D * PR * 2;       // q_idx    [32][PQI]
  static constexpr size_t OFF_QIT = OFF_QIS + (size_t)32 * PQI * 2;     // q_idx^T  [DIDX][PR]
  static constexpr size_t OFF_DS = OFF_QIT + (size_t)DIDX * PR * 2;     // dS       [32][PKT]
  static constexpr size_t OFF_DZ = OFF_DS + (size_t)32 * PKT * 2;       // dz       [32][PKT]
  static constexpr size_t OFF_PB = OFF_DZ + (size_t)32 * PKT * 2;       // P        [32][128] fp32
  static constexpr size_t OFF_TAB = OFF_PB + (size_t)32 * kBlock * 4;   // 2 x row/query tables
  static constexpr int TAB_WORDS = 10 * 32;
  static constexpr size_t LDS = OFF_TAB + 2 * TAB_WORDS * 4;
};

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4;

__device__ inline f4 mma16(bf16x8 a, bf16x8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// A operand from a transposed [m][32 rows] LDS tile whose K (rows) follow
// the C-layout of two stacked 16-row tiles: lane l, slot i <-> row
// 4*(l/16) + i for i < 4 and 16 + 4*(l/16) + i - 4 otherwise.
__device__ inline bf16x8 tfrag16(const bf16* base, int pitch, int m, int lane) {
  const bf16* p = base + m * pitch + 4 * (lane >> 4);
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}
// Matching B operand from two stacked 16-row C-layout tiles.
__device__ inline bf16x8 cfrag16(const f4& x0, const f4& x1) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (bf16)x0[i];
    r[i + 4] = (bf16)x1[i];
  }
  return r;
}

template <int D, int DIDX, int G>
__global__ __launch_bounds__(kMainThreads, 1) void bwd_main_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Dv,
    const bf16* __restrict__ q_idx, const bf16* __restrict__ k_idx, const float* __restrict__ lse_idx,
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ pos, const int32_t* __restrict__ offs,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ tiles, float* __restrict__ dq_acc,
    float* __restrict__ dk_acc, float* __restrict__ dv_acc, float* __restrict__ dq_idx,
    float* __restrict__ dk_idx, float* __restrict__ dscore, float* __restrict__ kl, int N, int H_kv, int topk,
    int causal, int nblk, int nsb, int n_lists, float scale, float scale_idx, float lam, int per_xcd) {
  using C = BwdCfg<D, DIDX>;
  constexpr int KS = D / 32;        // k-steps over d
  constexpr int KSI = DIDX / 32;    // k-steps over d_idx
  constexpr int DT = D / 16;        // 16-wide d tiles
  constexpr int DTI = DIDX / 16;    // 16-wide d_idx tiles
  constexpr int TQ = 32 / G;        // queries per 32-row step
  constexpr int MQ = TQ > 16 ? 2 : 1;
  constexpr int NT_Q = 2 * DT;      // dQ output tiles per step
  constexpr int NT = NT_Q + MQ * DTI;
  extern __shared__ __align__(16) char smem[];
  bf16* Kt = reinterpret_cast<bf16*>(smem + C::OFF_KT);
  bf16* KIt = reinterpret_cast<bf16*>(smem + C::OFF_KIT);
  bf16* Qs = reinterpret_cast<bf16*>(smem + C::OFF_QS);
  bf16* dOs = reinterpret_cast<bf16*>(smem + C::OFF_DOS);
  bf16* Qt = reinterpret_cast<bf16*>(smem + C::OFF_QT);
  bf16* dOt = reinterpret_cast<bf16*>(smem + C::OFF_DOT);
  bf16* QIs = reinterpret_cast<bf16*>(smem + C::OFF_QIS);
  bf16* QIt = reinterpret_cast<bf16*>(smem + C::OFF_QIT);
  bf16* dSs = reinterpret_cast<bf16*>(smem + C::OFF_DS);
  bf16* dZs = reinterpret_cast<bf16*>(smem + C::OFF_DZ);
  float* Pb = reinterpret_cast<float*>(smem + C::OFF_PB);
  int* tab0 = reinterpret_cast<int*>(smem + C::OFF_TAB);

  Item it;
  if (!decode_item(tiles, pos, offs, rows, n_lists, per_xcd, N, H_kv, topk, nblk, nsb, &it)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nn = lane & 15, qg = lane >> 4;
  const int H_q = H_kv * G;
  const int b = it.b, g = it.g, j = it.j;
  const int key = 16 * wave + nn;                     // this lane's key inside the block
  const int u = j * kBlock + key;
  const size_t kv_row = ((size_t)b * N + u) * H_kv + g;

  // K^T and K_idx^T of the block (B operands of dQ and dq_idx).
  for (int c = threadIdx.x; c < kBlock * (D / 8); c += kMainThreads) {
    const int kk = c / (D / 8), col = (c % (D / 8)) * 8;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(k + (((size_t)b * N + j * kBlock + kk) * H_kv + g) * D + col);
#pragma unroll
    for (int i = 0; i < 8; ++i) Kt[(col + i) * C::PKT + kk] = x[i];
  }
  for (int c = threadIdx.x; c < kBlock * (DIDX / 8); c += kMainThreads) {
    const int kk = c / (DIDX / 8), col = (c % (DIDX / 8)) * 8;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(k_idx + ((size_t)b * N + j * kBlock + kk) * DIDX + col);
#pragma unroll
    for (int i = 0; i < 8; ++i) KIt[(col + i) * C::PKT + kk] = x[i];
  }
  // This wave's 16 keys as B operands (lane = key, K = d), in registers.
  bf16x8 kf[KS], vf[KS], kif[KSI];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = *reinterpret_cast<const bf16x8*>(k + kv_row * D + 32 * ks + 8 * qg);
    vf[ks] = *reinterpret_cast<const bf16x8*>(v + kv_row * D + 32 * ks + 8 * qg);
  }
#pragma unroll
  for (int ks = 0; ks < KSI; ++ks)
    kif[ks] = *reinterpret_cast<const bf16x8*>(k_idx + ((size_t)b * N + u) * DIDX + 32 * ks + 8 * qg);

  f4 acc_dv[DT], acc_dk[DT], acc_dki[DTI];
#pragma unroll
  for (int i = 0; i < DT; ++i) {
    acc_dv[i] = zero4();
    acc_dk[i] = zero4();
  }
#pragma unroll
  for (int i = 0; i < DTI; ++i) acc_dki[i] = zero4();

  const float c_s = scale * kLog2e;
  const float c_i = scale_idx * kLog2e;
  const int n_steps = (it.nq * G + 31) / 32;
#pragma unroll 1
  for (int st = 0; st < n_steps; ++st) {
    asm volatile("" ::: "memory");
    int* tab = tab0 + (st & 1) * C::TAB_WORDS;
    int* row_t = tab;                                        // t of row, -1 if invalid
    int* row_h = tab + 32;                                   // head of row
    float* row_lse = reinterpret_cast<float*>(tab + 64);     // LSE * log2(e)
    float* row_d = reinterpret_cast<float*>(tab + 96);       // D
    int* qry_t = tab + 128;                                  // t of query, -1 if invalid
    int* qry_slot = tab + 160;
    float* qry_lse = reinterpret_cast<float*>(tab + 192);    // lse_idx * log2(e)
    float* qry_kl = reinterpret_cast<float*>(tab + 224);

    // (a) row and query tables.
    if (wave == 0) {
      const int x = lane & 31;
      if (lane < 32) {
        const int r = 32 * st + x;
        int t, slot;
        bool valid;
        item_query(it, r / G, block_idx, N, H_kv, topk, &t, &slot, &valid);
        const int h = g * G + x % G;
        const size_t qrow = ((size_t)b * N + t) * H_q + h;
        row_t[x] = valid ? t : -1;
        row_h[x] = h;
        row_lse[x] = lse[qrow] * kLog2e;
        row_d[x] = Dv[qrow];
      } else {
        int t = 0, slot = 0;
        bool valid = false;
        if (x < TQ) item_query(it, st * TQ + x, block_idx, N, H_kv, topk, &t, &slot, &valid);
        qry_t[x] = valid ? t : -1;
        qry_slot[x] = slot;
        qry_lse[x] = lse_idx[((size_t)b * N + t) * H_kv + g] * kLog2e;
        qry_kl[x] = 0.f;
      }
    }
    __syncthreads();
    // (b) Q, dO (32 rows) and q_idx (TQ rows) into LDS, row-major and transposed.
    for (int c = threadIdx.x; c < 32 * (D / 8); c += kMainThreads) {
      const int r = c / (D / 8), col = (c % (D / 8)) * 8;
      const int tr = row_t[r];
      const size_t qrow = ((size_t)b * N + (tr < 0 ? 0 : tr)) * H_q + row_h[r];
      const bf16x8 xq = *reinterpret_cast<const bf16x8*>(q + qrow * D + col);
      const bf16x8 xd = *reinterpret_cast<const bf16x8*>(dO + qrow * D + col);
      *reinterpret_cast<bf16x8*>(Qs + r * C::PQ + col) = xq;
      *reinterpret_cast<bf16x8*>(dOs + r * C::PQ + col) = xd;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        Qt[(col + i) * C::PR + r] = xq[i];
        dOt[(col + i) * C::PR + r] = xd[i];
      }
    }
    for (int c = threadIdx.x; c < 32 * (DIDX / 8); c += kMainThreads) {
      const int r = c / (DIDX / 8), col = (c % (DIDX / 8)) * 8;
      const int tq = qry_t[r];
      bf16x8 x = bf16x8{};
      if (tq >= 0) x = *reinterpret_cast<const bf16x8*>(q_idx + (((size_t)b * N + tq) * H_kv + g) * DIDX + col);
      *reinterpret_cast<bf16x8*>(QIs + r * C::PQI + col) = x;
#pragma unroll
      for (int i = 0; i < 8; ++i) QIt[(col + i) * C::PR + r] = x[i];
    }
    __syncthreads();

    // (c) S = Q K_w^T, dP = dO V_w^T (lane = key, slots = rows 16 mt + 4 qg + v),
    // P, dS, then dV^T += dO^T P and dK^T += Q^T dS for this wave's 16 keys.
    f4 s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = zero4();
      dp[mt] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + (16 * mt + nn) * C::PQ + 32 * ks + 8 * qg);
        const bf16x8 ad = *reinterpret_cast<const bf16x8*>(dOs + (16 * mt + nn) * C::PQ + 32 * ks + 8 * qg);
        s[mt] = mma16(aq, kf[ks], s[mt]);
        dp[mt] = mma16(ad, vf[ks], dp[mt]);
      }
    }
    f4 ri[MQ];
#pragma unroll
    for (int mt = 0; mt < MQ; ++mt) {
      ri[mt] = zero4();
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks)
        ri[mt] = mma16(*reinterpret_cast<const bf16x8*>(QIs + (16 * mt + nn) * C::PQI + 32 * ks + 8 * qg), kif[ks],
                       ri[mt]);
    }
    f4 p[2], ds[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int r = 16 * mt + 4 * qg + vv;
        const int tr = row_t[r];
        const bool vis = tr >= 0 && !(it.diag && causal && u > tr);
        const float pv = vis ? exp2f(s[mt][vv] * c_s - row_lse[r]) : 0.f;
        p[mt][vv] = pv;
        ds[mt][vv] = pv * (dp[mt][vv] - row_d[r]) * scale;
        Pb[r * kBlock + key] = pv;
        dSs[r * C::PKT + key] = (bf16)ds[mt][vv];
      }
    {
      const bf16x8 pb = cfrag16(p[0], p[1]), sb = cfrag16(ds[0], ds[1]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        acc_dv[dt] = mma16(tfrag16(dOt, C::PR, 16 * dt + nn, lane), pb, acc_dv[dt]);
        acc_dk[dt] = mma16(tfrag16(Qt, C::PR, 16 * dt + nn, lane), sb, acc_dk[dt]);
      }
    }
    __syncthreads();   // P of every head of a query visible to the teacher; dS complete

    // (d) Index branch on the query slots: p_px, teacher pbar, dz.
    f4 dz[2];
    dz[0] = zero4();
    dz[1] = zero4();
    float klv[MQ][4];
#pragma unroll
    for (int mt = 0; mt < MQ; ++mt)
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int qr = 16 * mt + 4 * qg + vv;
        klv[mt][vv] = 0.f;
        if (qr < TQ) {
          const int tqq = qry_t[qr];
          if (tqq >= 0 && !(it.diag && causal && u > tqq)) {
            const float lz = ri[mt][vv] * c_i - qry_lse[qr];   // log2 p_px
            const float ppx = exp2f(lz);
            float pbar = 0.f;
#pragma unroll
            for (int e = 0; e < G; ++e) pbar += Pb[(qr * G + e) * kBlock + key];
            pbar *= 1.0f / G;
            dz[mt][vv] = lam * (ppx - pbar);
            if (kl != nullptr && pbar > 0.f) klv[mt][vv] = pbar * (logf(pbar) - lz * kLn2);
          }
        }
      }
    {
      f4 zs0, zs1;
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        zs0[vv] = dz[0][vv] * scale_idx;
        zs1[vv] = dz[1][vv] * scale_idx;
      }
      const bf16x8 zb = cfrag16(zs0, zs1);
#pragma unroll
      for (int dt = 0; dt < DTI; ++dt) acc_dki[dt] = mma16(tfrag16(QIt, C::PR, 16 * dt + nn, lane), zb, acc_dki[dt]);
#pragma unroll
      for (int mt = 0; mt < MQ; ++mt)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int qr = 16 * mt + 4 * qg + vv;
          if (qr < TQ) dZs[qr * C::PKT + key] = (bf16)(mt == 0 ? zs0[vv] : zs1[vv]);
        }
    }
    if (dscore != nullptr) {
#pragma unroll
      for (int mt = 0; mt < MQ; ++mt)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          const int qr = 16 * mt + 4 * qg + vv;
          if (qr < TQ && qry_t[qr] >= 0)
            dscore[((((size_t)b * N + qry_t[qr]) * H_kv + g) * topk + qry_slot[qr]) * kBlock + key] = dz[mt][vv];
        }
    }
    if (kl != nullptr) {
#pragma unroll
      for (int mt = 0; mt < MQ; ++mt)
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
          float x = klv[mt][vv];
#pragma unroll
          for (int off = 8; off > 0; off >>= 1) x += __shfl_xor(x, off);   // over the 16 keys of the group
          const int qr = 16 * mt + 4 * qg + vv;
          if (nn == 0 && qr < TQ) atomicAdd(&qry_kl[qr], x);
        }
    }
    __syncthreads();   // dz and the KL partials complete

    // (e) dQ = dS K and dq_idx = dz K_idx: 16x16 output tiles over the waves;
    // lane = output column, slots = rows 4 qg + v of the tile.
    for (int tile = wave; tile < NT; tile += kBwdWaves) {
      const bool is_q = tile < NT_Q;
      const int rt = is_q ? tile / DT : (tile - NT_Q) / DTI;
      const int ct = is_q ? tile % DT : (tile - NT_Q) % DTI;
      const bf16* A = (is_q ? dSs : dZs) + (16 * rt + nn) * C::PKT + 8 * qg;
      const bf16* Bt = (is_q ? Kt : KIt) + (16 * ct + nn) * C::PKT + 8 * qg;
      f4 o = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        o = mma16(*reinterpret_cast<const bf16x8*>(A + 32 * kk), *reinterpret_cast<const bf16x8*>(Bt + 32 * kk), o);
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int r = 16 * rt + 4 * qg + vv;
        if (is_q) {
          const int tr = row_t[r];
          if (tr >= 0) atomicAdd(&dq_acc[(((size_t)b * N + tr) * H_q + row_h[r]) * D + 16 * ct + nn], o[vv]);
        } else if (r < TQ && qry_t[r] >= 0) {
          atomicAdd(&dq_idx[(((size_t)b * N + qry_t[r]) * H_kv + g) * DIDX + 16 * ct + nn], o[vv]);
        }
      }
    }
    if (kl != nullptr && threadIdx.x < TQ && qry_t[threadIdx.x] >= 0)
      atomicAdd(&kl[((size_t)b * N + qry_t[threadIdx.x]) * H_kv + g], qry_kl[threadIdx.x]);
  }

  // The block's dK, dV (group g) and dk_idx (shared by the groups): lane =
  // key, slots = d 16 dt + 4 qg + v.
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int vv = 0; vv < 4; ++vv) {
      const int dcol = 16 * dt + 4 * qg + vv;
      atomicAdd(&dk_acc[kv_row * D + dcol], acc_dk[dt][vv]);
      atomicAdd(&dv_acc[kv_row * D + dcol], acc_dv[dt][vv]);
    }
#pragma unroll
  for (int dt = 0; dt < DTI; ++dt)
#pragma unroll
    for (int vv = 0; vv < 4; ++vv)
      atomicAdd(&dk_idx[((size_t)b * N + u) * DIDX + 16 * dt + 4 * qg + vv], acc_dki[dt][vv]);
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
  auto kern = bwd_main_kernel<D, DIDX, G>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kMainThreads), C::LDS, s, static_cast<const bf16*>(a.q),
                     static_cast<const bf16*>(a.k), static_cast<const bf16*>(a.v), static_cast<const bf16*>(a.dO),
                     a.lse, w.D, static_cast<const bf16*>(a.q_idx), static_cast<const bf16*>(a.k_idx), w.lse_idx,
                     a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.dq_acc, w.dk_acc, w.dv_acc, a.dq_idx,
                     a.dk_idx, a.dscore, a.kl, P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb,
                     P.B * P.H_kv * P.nblk, P.scale, P.scale_idx, a.kl_weight, grid / 8);
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
  // Work items over the whole sequence.
  if ((e = launch_block_items(P, m, 0, P.N, kItemQueries, s)) != hipSuccess) return e;
  size_t grid = block_items_upper_bound(P, 0, P.N, kItemQueries);
  grid = (grid + 7) & ~size_t(7);
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int n_lists = P.B * P.H_kv * P.nblk;
  // Index log-sum-exp over the selected support.
  prof_begin("bwd_idx_lse", s);
  if (P.d_idx == 64)
    hipLaunchKernelGGL(idx_lse_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16*>(a.q_idx),
                       static_cast<const bf16*>(a.k_idx), a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.idx_part,
                       P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb, n_lists, P.scale_idx, (int)(grid / 8));
  else
    hipLaunchKernelGGL(idx_lse_kernel<32>, dim3((unsigned)grid), dim3(256), 0, s, static_cast<const bf16*>(a.q_idx),
                       static_cast<const bf16*>(a.k_idx), a.block_idx, m.pos, m.offs, m.rows, m.tiles, w.idx_part,
                       P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb, n_lists, P.scale_idx, (int)(grid / 8));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(idx_lse_merge_kernel, dim3((unsigned)((rows_g + 255) / 256)), dim3(256), 0, s, w.idx_part,
                     a.block_idx, w.lse_idx, rows_g, P.topk);
  prof_end(s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
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
