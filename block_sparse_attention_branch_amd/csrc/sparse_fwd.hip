// Main branch forward of MiniMax Sparse Attention: exact softmax attention of
// every (query, head) over the tokens of its selected KV blocks, plus LSE.
//
// Pages: "How to solve the memory problem with MiniMax Sparse Attention",
// 'Two-stage process' (exact softmax over the chosen tokens only; selection
// shared by a group's heads, so a KV block is read for all of them) and
// 'Kernel optimizations' (KV-outer: iterate over KV blocks and pack the
// queries that chose a block into one matmul); "How FlashAttention cuts GPU
// memory traffic without approximation", 'Tiling mechanism' and 'The online
// softmax trick' (each block contributes a partial result with its own max
// and normaliser; partials merge exactly by rescaling), 'Architectural
// compatibility' (the causal mask is needed only on the diagonal block);
// "How Flash-MSA cuts million-token training cost with sparse-k", 'Kernel
// design and execution' (the forward keeps the LSE for the backward).
//
// Structure (two kernels per query chunk):
//   1. sparse_fwd_kernel: one workgroup per work item = (b, g, KV block j,
//      up to 768 queries that selected j, or its own 128).  K_j and V_j^T are staged in LDS
//      once; each wave takes 32 (query, head) rows at a time:
//        S^T = K_j Q^T      (32x32 MFMA: keys are tile rows, a lane holds
//                            one (query, head) row and 16 keys per tile)
//        P^T = exp(S^T - max) in registers, the row max/sum being a register
//                            reduction plus one half-wave exchange
//        O^T = V_j^T P^T    (the P^T registers are the B operand as they are)
//      and writes the normalised partial o_j (dtype) and its log-sum-exp.
//   2. fwd_merge_kernel: per (query, head), LSE = logsumexp over its slots
//      and o = sum_j exp(lse_j - LSE) o_j.
//   Item i is workgroup i, so consecutive items (same KV block) are dealt to
//   different XCDs and the uneven item costs spread evenly over the chip.
#include "msa_internal.h"

namespace msa {
namespace {


constexpr int kItemQueries = 768;     // list entries per work item (the diagonal item has its 128)

template <typename T, int D>
struct FwdCfg {
  // bf16: 12 waves, one workgroup per CU (99 KB of LDS at d = 128), three
  // waves per SIMD (at most 168 VGPRs each), so that a SIMD has a third wave
  // to issue from while two wait.  fp32 tiles take twice the LDS: 4 waves,
  // two workgroups per CU at d = 64, one at d = 128.
  static constexpr int WAVES = sizeof(T) == 2 ? 12 : 4;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int KPL = Mma<T>::KPL;
  static constexpr int KSTEPS = D / (2 * KPL);           // k-steps of S^T over d
  static constexpr int KCH = 16 / KPL;                   // B-operand chunks per 32-key tile
  static constexpr int PK = D + 16 / (int)sizeof(T);     // K row pitch (elements), 16 B pad
  static constexpr int PV = kBlock + 8 / (int)sizeof(T); // V^T row pitch (elements), 8 B pad
  static constexpr size_t K_BYTES = (size_t)kBlock * PK * sizeof(T);
  static constexpr size_t V_BYTES = (size_t)D * PV * sizeof(T);
  // Per-wave staging of one 32-column slice of the partial output (32 rows),
  // so that the partials leave in 16-byte pieces, 64 bytes per row per slice.
  static constexpr int PO = 32 + 16 / (int)sizeof(T);                  // row pitch (elements)
  static constexpr size_t O_BYTES = (size_t)WAVES * 32 * PO * sizeof(T);
  // The item's queries, (t << 6) | slot or -1, staged once per item.
  static constexpr size_t E_BYTES = (size_t)(kItemQueries > kBlock ? kItemQueries : kBlock) * 4;
  static constexpr size_t LDS = K_BYTES + V_BYTES + O_BYTES + E_BYTES;
  static constexpr int DT = D / 32;
  static constexpr int CPR = D * (int)sizeof(T) / 16;    // 16-byte chunks per key row
  static constexpr int EPC = 16 / (int)sizeof(T);        // elements per chunk
};

// A operand of O^T = V^T P^T: lane l supplies V^T[drow][keys] for the keys
// that slot group kc of the P^T tile holds in this lane.
template <typename T> struct VtFrag;
template <> struct VtFrag<bf16> {
  __device__ static inline bf16x8 load(const bf16* Vt, int pitch, int drow, int key0, int kc, int lane) {
    const bf16* p = Vt + drow * pitch + key0 + 16 * kc + 4 * (lane >> 5);
    const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 8);
    bf16x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
  // B operand from the P^T slots 8*kc .. 8*kc+7 of one 32x32 tile.
  __device__ static inline bf16x8 pfrag(const f32x16& p, int kc) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (bf16)p[8 * kc + i];
    return r;
  }
};
template <> struct VtFrag<float> {
  __device__ static inline float load(const float* Vt, int pitch, int drow, int key0, int kc, int lane) {
    return Vt[drow * pitch + key0 + c_row(kc, lane)];
  }
  __device__ static inline float pfrag(const f32x16& p, int kc) { return p[kc]; }
};

template <typename T> struct Store4;
template <> struct Store4<bf16> {
  __device__ static inline void st(bf16* dst, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (bf16)a; v[1] = (bf16)b; v[2] = (bf16)c; v[3] = (bf16)d;
    *reinterpret_cast<bf16x4*>(dst) = v;
  }
};
template <> struct Store4<float> {
  __device__ static inline void st(float* dst, float a, float b, float c, float d) {
    f32x4 v;
    v[0] = a; v[1] = b; v[2] = c; v[3] = d;
    *reinterpret_cast<f32x4*>(dst) = v;
  }
};

template <typename T, int D, int G>
__global__ __launch_bounds__((FwdCfg<T, D>::THREADS), (FwdCfg<T, D>::WAVES / 4)) void sparse_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ offs, const int32_t* __restrict__ rows, const int32_t* __restrict__ tiles,
    T* __restrict__ po, float* __restrict__ plse, int N, int H_kv, int topk, int causal, int nblk,
    int nsb, int s_lo, int s_hi, int c0, int c1, int n_lists, float scale) {
  using C = FwdCfg<T, D>;
  using M = Mma<T>;
  constexpr int KPL = C::KPL;
  extern __shared__ __align__(16) char smem[];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vt = reinterpret_cast<T*>(smem + C::K_BYTES);
  const int H_q = H_kv * G;
  const int CQ = c1 - c0;

  const int w = xcd_item(tiles[n_lists]);
  if (w < 0) return;
  int lo = 0, hi = n_lists - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tiles[mid] <= w) lo = mid; else hi = mid - 1;
  }
  const int list = lo;
  const int local = w - tiles[list];
  const int j = list % nblk, bg = list / nblk, g = bg % H_kv, b = bg / H_kv;
  const bool has_diag = j >= c0 / kBlock && j < c1 / kBlock;
  const bool diag = has_diag && local == 0;
  int nq = kBlock;
  const int32_t* ent = nullptr;
  if (!diag) {
    const int32_t* pb = pos + (size_t)bg * (nsb + 1) * nblk + j;
    const int seg0 = pb[(size_t)s_lo * nblk], seg1 = pb[(size_t)s_hi * nblk];
    const int e0 = seg0 + (local - (has_diag ? 1 : 0)) * kItemQueries;
    nq = min(kItemQueries, seg1 - e0);
    ent = rows + (size_t)bg * N * topk + offs[(size_t)bg * (nblk + 1) + j] + e0;
  }

  // Stage the item's queries: (t << 6) | slot, or -1 for an entry that is
  // not a query of this chunk (a well-formed map only yields such queries;
  // anything else is dropped rather than trusted).  The diagonal item finds
  // each own query's slot in its selection here, once.
  int* qent = reinterpret_cast<int*>(smem + C::K_BYTES + C::V_BYTES + C::O_BYTES);
  for (int i = threadIdx.x; i < nq; i += C::THREADS) {
    int t, slot = 0;
    if (diag) {
      t = j * kBlock + i;
      const int32_t* brow = block_idx + (((size_t)b * N + t) * H_kv + g) * topk;
      for (int e = 0; e < topk; ++e)
        if (brow[e] == j) slot = e;
    } else {
      const int e = ent[i];
      t = e >> 6;
      slot = e & 63;
    }
    qent[i] = (t < c0 || t >= c1 || slot >= topk) ? -1 : ((t << 6) | slot);
  }
  // Stage K_j (row-major) and V_j^T in LDS.
  {
    const size_t base = (((size_t)b * N + (size_t)j * kBlock) * H_kv + g) * D;
    for (int c = threadIdx.x; c < kBlock * C::CPR; c += C::THREADS) {
      const int key = c / C::CPR, col = c % C::CPR;
      const size_t goff = base + (size_t)key * H_kv * D + col * C::EPC;
      const uint4 kv = *reinterpret_cast<const uint4*>(k + goff);
      *reinterpret_cast<uint4*>(Ks + key * C::PK + col * C::EPC) = kv;
      const uint4 vv = *reinterpret_cast<const uint4*>(v + goff);
      const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int i = 0; i < C::EPC; ++i) Vt[(col * C::EPC + i) * C::PV + key] = ve[i];
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_rows = nq * G;
  const float c_exp = scale * kLog2e;
  constexpr int NW = C::WAVES;
  // Query, slot and validity of this lane's row in the wave's row tile
  // starting at row r0 (rows r0 = 32 wave + 32 WAVES tile ..).
  auto locate = [&](int r0, int* t, int* slot, int* h, bool* valid) {
    const int r = r0 + (lane & 31);
    *h = g * G + r % G;
    const int e = qent[min(r, n_rows - 1) / G];
    *valid = r < n_rows && e >= 0;
    *t = e >= 0 ? (e >> 6) : c0;      // dropped entries are clamped for the loads
    *slot = e >= 0 ? (e & 63) : 0;
  };
  typename M::frag qn[C::KSTEPS];   // the next row tile's Q fragments, in flight
  auto load_q = [&](int t, int h) {
    const T* qrow = q + (((size_t)b * N + t) * H_q + h) * D + KPL * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qn[ks] = M::load(qrow + ks * 2 * KPL);
  };
  int nt, nslot, nh;
  bool nvalid;
  locate(wave * 32, &nt, &nslot, &nh, &nvalid);
  if (wave * 32 < n_rows) load_q(nt, nh);
#pragma unroll 1
  for (int r0 = wave * 32; r0 < n_rows; r0 += 32 * NW) {
    // Keep the K/V fragment reads inside the loop (re-read from LDS per row
    // tile) instead of letting them be hoisted into ~256 live registers.
    asm volatile("" ::: "memory");
    const int t = nt, slot = nslot, h = nh;
    const bool valid = nvalid;
    typename M::frag qf[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qf[ks] = qn[ks];
    // The next row tile's queries are located (from LDS) and their Q loads
    // issued at the top of this tile, so that the whole tile covers the
    // gather (14.2-14.7 -> 14.0 ms at 128K against issuing them after the
    // softmax).
    if (r0 + 32 * NW < n_rows) {
      locate(r0 + 32 * NW, &nt, &nslot, &nh, &nvalid);
      load_q(nt, nh);
    }

    // The S and O product stretches run at raised wave priority, so that of
    // two waves of a SIMD the one issuing products goes first and the other's
    // softmax fills the vector unit meanwhile.
    f32x16 s[4];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = zero16();
      const T* kp = Ks + (mt * 32 + (lane & 31)) * C::PK + KPL * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) s[mt] = M::mma(M::load(kp + ks * 2 * KPL), qf[ks], s[mt]);
    }
    __builtin_amdgcn_s_setprio(0);
    if (diag && causal) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int vv = 0; vv < 16; ++vv)
          if (j * kBlock + mt * 32 + c_row(vv, lane) > t) s[mt][vv] = -INFINITY;
    }
    float m = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) m = fmaxf(m, s[mt][vv]);
    m = fmaxf(m, swap_half(m));
    const float mc = m * c_exp;
    float lsum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int vv = 0; vv < 16; ++vv) {
        // The hardware exp2 (one instruction; its argument is <= 0 here, and
        // results below the fp32 normal range are negligible beside the
        // row's maximum of 1), not the library's range-reduced exp2f.
        const float p = __builtin_amdgcn_exp2f(s[mt][vv] * c_exp - mc);
        s[mt][vv] = p;
        lsum += p;
      }
    lsum += swap_half(lsum);

    // P^T as B-operand fragments (the fp32 score tile dies here).
    typename M::frag pf[4][C::KCH];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kc = 0; kc < C::KCH; ++kc) pf[mt][kc] = VtFrag<T>::pfrag(s[mt], kc);

    f32x16 o[C::DT];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      o[dt] = zero16();
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int kc = 0; kc < C::KCH; ++kc) {
          const typename M::frag a = VtFrag<T>::load(Vt, C::PV, dt * 32 + (lane & 31), mt * 32, kc, lane);
          o[dt] = M::mma(a, pf[mt][kc], o[dt]);
        }
    }
    __builtin_amdgcn_s_setprio(0);

    // Partial o of the row (normalised) and its LSE.  Each 32-column slice
    // goes through the wave's LDS staging tile: lane (row, half) writes its
    // 4 x 4 values, then lane l stores 16 bytes of row l / RPL (+ 32 / SPL..).
    const float inv = 1.f / lsum;
    // LSE partials [b, query, head, slot]; output partials [b, query, slot,
    // d / 32, head, 32]: the 32-column slices of one query, slot and slice are
    // contiguous over the group's heads, so a store instruction (whole slices
    // of consecutive rows, which are the heads of one or two queries) writes
    // whole cache lines.  sbase: slice-row of (query, slot, slice 0, head).
    const int lrow = valid ? (((b * CQ + (t - c0)) * H_q + h) * topk + slot) : -1;
    const int sbase = valid ? (((b * CQ + (t - c0)) * topk + slot) * (C::DT * H_q) + h) : -1;
    if (valid && lane < 32) plse[lrow] = m * scale + logf(lsum);
    {
      constexpr int EPC = C::EPC;                 // elements per 16-byte piece
      constexpr int PPR = 32 / EPC;               // pieces per 32-column row slice
      constexpr int RPI = 64 / PPR;               // rows per store instruction
      T* ost = reinterpret_cast<T*>(smem + C::K_BYTES + C::V_BYTES) + wave * 32 * C::PO;
      const int rl = lane & 31;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          Store4<T>::st(ost + rl * C::PO + 8 * v4 + 4 * (lane >> 5), o[dt][4 * v4] * inv, o[dt][4 * v4 + 1] * inv,
                        o[dt][4 * v4 + 2] * inv, o[dt][4 * v4 + 3] * inv);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's slice is in LDS
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int rr = i * RPI + lane / PPR, pc = lane % PPR;
          const int sb = __shfl(sbase, rr);
          const uint4 x = *reinterpret_cast<const uint4*>(ost + rr * C::PO + pc * EPC);
          // Streaming (nontemporal) store: the partials are read once, by the
          // merge, so they should not displace the Q rows and K/V blocks
          // that the other items re-read from the caches.
          if (sb >= 0)
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x),
                                        reinterpret_cast<u32x4*>(po + (size_t)(sb + dt * H_q) * 32 + pc * EPC));
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slice read before it is overwritten
      }
    }
  }
}

// Merge the per-block partials of every (query, head) of the chunk: LPR lanes
// per (query, head) row, 16 bytes of o each.  KM >= topk is the compile-time
// slot count: every partial load of the row is issued up front (slot indices
// past topk are clamped to the last slot and their weight is zero), together
// with the row's block indices and slot log-sum-exps, so that a row costs one
// memory round trip (two at KM = 64, whose loads go in chunks of 32).  The
// merge: LSE = logsumexp over the valid slots and o = sum_j exp(lse_j - LSE) o_j.  Padded slots (block index -1) hold
// unwritten memory: they are excluded by selection, never by multiplying
// with a zero weight.  Row indices fit in 32 bits (checked by the host).
template <typename T, int D, int KM>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const T* __restrict__ po, const float* __restrict__ plse,
                                                        const int32_t* __restrict__ block_idx, T* __restrict__ o,
                                                        float* __restrict__ lse, int B, int N, int H_kv, int G,
                                                        int topk, int c0, int CQ) {
  constexpr int EPL = 16 / (int)sizeof(T);   // elements per lane
  constexpr int LPR = D / EPL;               // lanes per row
  const int H_q = H_kv * G;
  const int row = blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  if (row >= B * CQ * H_q) return;
  const int part = threadIdx.x % LPR;
  const int h = row % H_q;
  const int bt = row / H_q;
  const int tl = bt % CQ, b = bt / CQ;
  const int t = c0 + tl, g = h / G;
  const int32_t* brow = block_idx + (((size_t)b * N + t) * H_kv + g) * topk;
  const float* lrow = plse + (size_t)row * topk;
  // Partials [b, query, slot, d / 32, head, 32]: this lane's 16 bytes lie in
  // slice (part EPL) / 32; slot e is e (D / 32) H_q 32 elements further.
  constexpr int NS = D / 32;
  const int col = part * EPL;
  const T* prow = po + ((size_t)(bt * topk * NS + col / 32) * H_q + h) * 32 + col % 32;
  // Partial loads in flight: all of the row's (KM <= 32), else chunks of 32.
  constexpr int KC = KM > 32 ? 32 : KM;
  uint4 raw[KC];
  auto load_chunk = [&](int e0) {
#pragma unroll
    for (int e = 0; e < KC; ++e)
      raw[e] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                             prow + (size_t)min(e0 + e, topk - 1) * NS * H_q * 32)));   // read once
  };
  load_chunk(0);
  // Slot log-sum-exps in log2 units, -inf for padded slots.
  float lv[KM];
  if (topk == KM) {
#pragma unroll
    for (int e = 0; e < KM; e += 4) {
      const int4 bi = *reinterpret_cast<const int4*>(brow + e);
      const float4 l4 = *reinterpret_cast<const float4*>(lrow + e);
      lv[e] = bi.x >= 0 ? l4.x * kLog2e : -INFINITY;
      lv[e + 1] = bi.y >= 0 ? l4.y * kLog2e : -INFINITY;
      lv[e + 2] = bi.z >= 0 ? l4.z * kLog2e : -INFINITY;
      lv[e + 3] = bi.w >= 0 ? l4.w * kLog2e : -INFINITY;
    }
  } else {
#pragma unroll
    for (int e = 0; e < KM; ++e) {
      const int ec = min(e, topk - 1);
      const int bi = brow[ec];
      const float l = lrow[ec];
      lv[e] = (e < topk && bi >= 0) ? l * kLog2e : -INFINITY;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < KM; ++e) mx = fmaxf(mx, lv[e]);   // finite: the own block is always valid
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < KM; ++e) den += __builtin_amdgcn_exp2f(lv[e] - mx);
  const float L2 = mx + __builtin_amdgcn_logf(den);   // log2 of the row's total
  float acc[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) acc[i] = 0.f;
#pragma unroll
  for (int e0 = 0; e0 < KM; e0 += KC) {
    if (e0 > 0) load_chunk(e0);
#pragma unroll
    for (int e = 0; e < KC; ++e) {
      if (lv[e0 + e] != -INFINITY) {
        const float wgt = __builtin_amdgcn_exp2f(lv[e0 + e] - L2);
        const T* x = reinterpret_cast<const T*>(&raw[e]);
#pragma unroll
        for (int c = 0; c < EPL; ++c) acc[c] = fmaf(wgt, to_f32(x[c]), acc[c]);
      }
    }
  }
  const float L = L2 * kLn2;
  uint4 outv;
  T* ov = reinterpret_cast<T*>(&outv);
#pragma unroll
  for (int i = 0; i < EPL; ++i) ov[i] = from_f32<T>(acc[i]);
  const size_t orow = ((size_t)b * N + t) * H_q + h;
  *reinterpret_cast<uint4*>(o + orow * D + part * EPL) = outv;
  if (part == 0) lse[orow] = L;
}

template <typename T, int D>
hipError_t launch_fwd_merge(const Problem& P, const T* po, const float* pl, const int32_t* block_idx, T* o,
                            float* lse, int c0, int CQ, hipStream_t s) {
  constexpr int LPR = D / (16 / (int)sizeof(T));
  const size_t rows = (size_t)P.B * CQ * P.H_q;
  if (rows > 0x7fffffff) return hipErrorInvalidConfiguration;
  const unsigned blocks = (unsigned)((rows + (256 / LPR) - 1) / (256 / LPR));
  auto kern = P.topk <= 4 ? fwd_merge_kernel<T, D, 4>
            : P.topk <= 8 ? fwd_merge_kernel<T, D, 8>
            : P.topk <= 16 ? fwd_merge_kernel<T, D, 16>
            : P.topk <= 32 ? fwd_merge_kernel<T, D, 32> : fwd_merge_kernel<T, D, 64>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, s, po, pl, block_idx, o, lse, P.B, P.N, P.H_kv, P.G,
                     P.topk, c0, CQ);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t run_fwd(const Problem& P, const T* q, const T* k, const T* v, const int32_t* block_idx, T* o,
                   float* lse, const BlockMap& m, void* partials, int chunk, hipStream_t s) {
  using C = FwdCfg<T, D>;
  auto kern = sparse_fwd_kernel<T, D, G>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  const int n_lists = P.B * P.H_kv * P.nblk;
  const int span = block_map_super_span(P);
  for (int c0 = 0; c0 < P.N; c0 += chunk) {
    const int c1 = c0 + chunk < P.N ? c0 + chunk : P.N;
    const int CQ = c1 - c0;
    T* po = static_cast<T*>(partials);
    float* pl = reinterpret_cast<float*>(static_cast<char*>(partials) +
                                         (((size_t)P.B * CQ * P.H_q * P.topk * D * sizeof(T) + 255) & ~size_t(255)));
    if ((e = launch_block_items(P, m, c0, c1, kItemQueries, s)) != hipSuccess) return e;
    size_t grid = block_items_upper_bound(P, c0, c1, kItemQueries);
    grid = (grid + 7) & ~size_t(7);
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    const int s_lo = c0 / span;
    const int s_hi = (c1 == P.N) ? m.nsb : c1 / span;
    {
      ProfScope prof("fwd_partial", s);
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), C::LDS, s, q, k, v, block_idx, m.pos,
                         m.offs, m.rows, m.tiles, po, pl, P.N, P.H_kv, P.topk, P.causal, P.nblk, m.nsb, s_lo,
                         s_hi, c0, c1, n_lists, P.scale);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
      ProfScope prof("fwd_merge", s);
      if ((e = launch_fwd_merge<T, D>(P, po, pl, block_idx, o, lse, c0, CQ, s)) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

template <typename T, int D>
hipError_t run_fwd_g(const Problem& P, const void* q, const void* k, const void* v, const int32_t* bi, void* o,
                     float* lse, const BlockMap& m, void* part, int chunk, hipStream_t s) {
  const T* Q = static_cast<const T*>(q);
  const T* K = static_cast<const T*>(k);
  const T* V = static_cast<const T*>(v);
  T* O = static_cast<T*>(o);
  switch (P.G) {
    case 1: return run_fwd<T, D, 1>(P, Q, K, V, bi, O, lse, m, part, chunk, s);
    case 2: return run_fwd<T, D, 2>(P, Q, K, V, bi, O, lse, m, part, chunk, s);
    case 4: return run_fwd<T, D, 4>(P, Q, K, V, bi, O, lse, m, part, chunk, s);
    case 8: return run_fwd<T, D, 8>(P, Q, K, V, bi, O, lse, m, part, chunk, s);
    case 16: return run_fwd<T, D, 16>(P, Q, K, V, bi, O, lse, m, part, chunk, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

size_t sparse_fwd_partials_bytes(const Problem& P, int chunk) {
  const size_t esz = P.dtype == MSA_BF16 ? 2 : 4;
  const size_t n = (size_t)P.B * chunk * P.H_q * P.topk;
  return ((n * P.d * esz + 255) & ~size_t(255)) + ((n * 4 + 255) & ~size_t(255));
}

hipError_t launch_sparse_fwd(const Problem& P, const void* q, const void* k, const void* v,
                             const int32_t* block_idx, void* o, float* lse, const BlockMap& m,
                             void* partials, int chunk, hipStream_t s) {
  if (P.dtype == MSA_BF16) {
    if (P.d == 128) return run_fwd_g<bf16, 128>(P, q, k, v, block_idx, o, lse, m, partials, chunk, s);
    return run_fwd_g<bf16, 64>(P, q, k, v, block_idx, o, lse, m, partials, chunk, s);
  }
  if (P.d == 128) return run_fwd_g<float, 128>(P, q, k, v, block_idx, o, lse, m, partials, chunk, s);
  return run_fwd_g<float, 64>(P, q, k, v, block_idx, o, lse, m, partials, chunk, s);
}

}  // namespace msa
