// Index branch of MiniMax Sparse Attention, fused in one pass: index scores
// (MFMA), block max-pool (in registers) and the exp-free top-k with the
// query's own block forced (a per-lane sorted list in registers).
//
// Pages: "How to solve the memory problem with MiniMax Sparse Attention",
// 'How the indexer works' (score visible tokens with the group's index query
// against the shared index key, max-pool per block, keep the top k with the
// own block always in) and 'Kernel optimizations' (softmax keeps the order,
// so the top-k skips exp and sum); "How Flash-MSA cuts million-token training
// cost with sparse-k", 'Block sparsity mechanism' and 'Kernel design and
// execution' (the proxy pass accumulates no output, only scores and top-k
// indices, kept in registers).
//
// Work split.  A workgroup of 4 waves streams the index keys of one batch
// row block by block (128 keys per block, staged in LDS, double buffered);
// two workgroups share a CU, so one's products run while the other waits at
// its barrier or pools.  Each wave owns 64 queries of one group.  For a block it computes the
// 128 x 64 score tile as S^T = K_idx Q_idx^T with 32x32 MFMA tiles: keys are
// the tile rows, queries the columns, so a lane holds one query and 16 keys
// per tile and the block max is a register max plus one exchange between the
// two half-waves.  After the exchange lane l owns query q0 + l and folds the
// block's pooled score into its sorted list of the best topk-1 other blocks
// (strictly greater wins, so equal scores keep the lower block index),
// through a per-lane candidate filter that keeps most blocks off the list.
// No pooled score ever reaches HBM unless the caller asks for it.
#include <float.h>
#include <limits.h>

#include "msa_internal.h"

namespace msa {
namespace {

constexpr int kIdxWaves = 4;
constexpr int kIdxThreads = kIdxWaves * kWave;
constexpr int kQPerWave = 64;
// Candidate slots per lane: blocks whose pooled score passes the lane's
// threshold wait here until one lane's slots are full, then join the list.
constexpr int kCandSlots = 8;

template <typename T, int DIDX>
struct IdxCfg {
  static constexpr int KPL = Mma<T>::KPL;
  static constexpr int KSTEPS = DIDX / (2 * KPL);
  static constexpr int PITCH = DIDX + 16 / (int)sizeof(T);    // LDS row, 16 B pad
  static constexpr int TILE_ELEMS = kBlock * PITCH;
  static constexpr int CHUNKS_PER_ROW = DIDX * (int)sizeof(T) / 16;
  static constexpr int CHUNKS_PER_THREAD = kBlock * CHUNKS_PER_ROW / kIdxThreads;
  static_assert(kBlock * CHUNKS_PER_ROW % kIdxThreads == 0, "tile load must split evenly");
  static constexpr size_t TILES_BYTES = 2 * TILE_ELEMS * sizeof(T);
  // Candidate slots after the two key tiles: [wave][slot][lane] of (score, block).
  static constexpr size_t LDS_BYTES = TILES_BYTES + (size_t)kIdxWaves * kCandSlots * kWave * 8;
};

// An empty asm that reads every 32-bit word of x: x must be in registers
// (its loads complete) at this point of the program.
template <typename F>
__device__ inline void hold_in_registers(const F& x) {
  static_assert(sizeof(F) % 4 == 0, "whole words");
  struct Words {
    unsigned w[sizeof(F) / 4];
  };
  const Words v = __builtin_bit_cast(Words, x);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(F) / 4); ++i) asm volatile("" ::"v"(v.w[i]));
}

// A list of 63 entries (topk 64) needs the registers of a whole SIMD: one
// workgroup per CU then; FP8 with lists of up to 15 (half-block passes) fits
// three, the others two.
template <typename T, int CAP>
constexpr int idx_workgroups_per_cu() {
  return CAP > 31 ? 1 : ((std::is_same<T, fp8e4m3>::value && CAP <= 15) ? 3 : 2);
}

template <typename T, int DIDX, int CAP>
__global__ __launch_bounds__(kIdxThreads, (idx_workgroups_per_cu<T, CAP>())) void index_topk_kernel(
    const T* __restrict__ q_idx, const T* __restrict__ k_idx, int32_t* __restrict__ block_idx,
    float* __restrict__ pooled, int N, int H_kv, int topk, int causal, int GT, int n_qtiles,
    int n_gtiles) {
  using C = IdxCfg<T, DIDX>;
  using M = Mma<T>;
  constexpr int KPL = C::KPL;
  extern __shared__ __align__(16) char smem_raw[];
  T* lds = reinterpret_cast<T*>(smem_raw);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int QW = kIdxWaves / GT;
  const int nblk = N / kBlock;

  // Heaviest (latest) query tiles first: causal work grows with the tile.
  const int per_q = gridDim.x / n_qtiles;
  const int qrev = blockIdx.x / per_q;
  const int rest = blockIdx.x % per_q;
  const int b = rest / n_gtiles;
  const int gtile = rest % n_gtiles;
  const int qtile = n_qtiles - 1 - qrev;
  const int g = gtile * GT + (wave % GT);
  const int wg_q0 = qtile * QW * kQPerWave;
  const int q0 = wg_q0 + (wave / GT) * kQPerWave;
  const bool wave_valid = q0 < N;
  const int own = (wave_valid ? q0 : N - 1) / kBlock;   // shared by the wave's 64 queries
  const int wg_last = min(wg_q0 + QW * kQPerWave - 1, N - 1);
  const int jlast = causal ? wg_last / kBlock : nblk - 1;

  // Index-query fragments (B operand) for the wave's two 32-query columns.
  typename M::frag qf[2][C::KSTEPS];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int t = min(q0 + nt * 32 + (lane & 31), N - 1);
    const T* qp = q_idx + (((size_t)b * N + t) * H_kv + g) * DIDX + KPL * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) qf[nt][ks] = M::load(qp + ks * 2 * KPL);
  }

  float tv[CAP];
  int ti[CAP];
#pragma unroll
  for (int i = 0; i < CAP; ++i) {
    tv[i] = -INFINITY;
    ti[i] = -1;
  }

  const char* kbase = reinterpret_cast<const char*>(k_idx + (size_t)b * N * DIDX);
  // Native 4 x 32-bit vectors, not HIP's uint4 class: the class copy kept
  // the staging array in scratch memory.
  u32x4 stage[C::CHUNKS_PER_THREAD];
  auto load_block = [&](int j) {
    const char* src = kbase + (size_t)j * kBlock * DIDX * sizeof(T);
#pragma unroll
    for (int c = 0; c < C::CHUNKS_PER_THREAD; ++c) {
      const int chunk = threadIdx.x + c * kIdxThreads;
      stage[c] = *reinterpret_cast<const u32x4*>(src + (size_t)chunk * 16);
    }
  };

  auto store_block = [&](int buf) {
#pragma unroll
    for (int c = 0; c < C::CHUNKS_PER_THREAD; ++c) {
      const int chunk = threadIdx.x + c * kIdxThreads;
      const int row = chunk / C::CHUNKS_PER_ROW, col = chunk % C::CHUNKS_PER_ROW;
      *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(lds + buf * C::TILE_ELEMS + row * C::PITCH) +
                                col * 16) = stage[c];
    }
  };

  load_block(0);
  // The query fragments are consumed here, before the loop, so their loads
  // complete in the prologue: left in flight into the loop, the wait-count
  // analysis merged them into the loop header and waited on every load in
  // flight (the next block's included) before each block's first products.
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) hold_in_registers(qf[nt][ks]);
  store_block(0);
  __syncthreads();

  // Insert a block's pooled score into the lane's sorted list (strictly
  // greater wins, so equal scores keep the lower block index).  A score that
  // does not beat the list's last entry changes nothing, so the wave skips
  // the insertion when no lane's does.
  auto insert = [&](float p, int jb) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(p > tv[CAP - 1]) == 0) return;
#pragma unroll
    for (int i = CAP - 1; i >= 1; --i) {
      const bool up = p > tv[i - 1];
      const bool here = p > tv[i];
      tv[i] = up ? tv[i - 1] : (here ? p : tv[i]);
      ti[i] = up ? ti[i - 1] : (here ? jb : ti[i]);
    }
    const bool here = p > tv[0];
    tv[0] = here ? p : tv[0];
    ti[0] = here ? jb : ti[0];
  };
  // Blocks reach the list through a filter: a pooled score that beats thr,
  // the list's last entry when the slots were last emptied, goes to the
  // lane's next candidate slot in LDS; when some lane's slots are full, every
  // lane inserts its candidates in the order they came.  The list only grows,
  // so thr never exceeds its last entry and every score the list would take
  // passes the filter; inserting in arrival order (increasing block index)
  // keeps the tie rule.  The list therefore ends exactly as with one
  // insertion per block, at a fraction of the vector work.
  int2* cand = reinterpret_cast<int2*>(smem_raw + C::TILES_BYTES) + (size_t)wave * kCandSlots * kWave + lane;
  float thr = -INFINITY;
  int ncand = 0;
  auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int sl = 0; sl < kCandSlots; ++sl) {
      const int2 e = cand[sl * kWave];
      insert(sl < ncand ? __int_as_float(e.x) : -INFINITY, e.y);
    }
    ncand = 0;
    thr = tv[CAP - 1];
  };
  auto offer = [&](float p, int jb) __attribute__((always_inline)) {
    if (p > thr) {
      cand[ncand * kWave] = make_int2(__float_as_int(p), jb);
      ++ncand;
    }
    if (__builtin_amdgcn_ballot_w64(ncand == kCandSlots) != 0) flush();
  };
  float p_prev = -INFINITY;
  int j_prev = -1;
  // S^T of block j (its tile in LDS buffer buf): accumulators a0 / a1 for the
  // wave's two 32-query columns, 4 row tiles of 32 keys each.
  typename M::frag nxt[C::KSTEPS];   // row tile 0 of a block, when read ahead
  auto products = [&](int buf, bool ahead, f32x16 (&a0)[4], f32x16 (&a1)[4]) __attribute__((always_inline)) {
    const T* tile = lds + buf * C::TILE_ELEMS;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      a0[mt] = zero16();
      a1[mt] = zero16();
      const T* ap = tile + (mt * 32 + (lane & 31)) * C::PITCH + KPL * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        const typename M::frag a = (ahead && mt == 0) ? nxt[ks] : M::load(ap + ks * 2 * KPL);
        a0[mt] = M::mma(a, qf[0][ks], a0[mt]);
        a1[mt] = M::mma(a, qf[1][ks], a1[mt]);
      }
    }
  };
  auto read_ahead = [&](int buf) __attribute__((always_inline)) {
    const T* ap = lds + buf * C::TILE_ELEMS + (lane & 31) * C::PITCH + KPL * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) nxt[ks] = M::load(ap + ks * 2 * KPL);
  };
  // Block j's pooled score per query, handed to the list one block later:
  // the offer of block j-1 runs after block j's products are issued, so its
  // arithmetic overlaps the matrix unit instead of following it.
  auto pool = [&](int j, bool is_own, f32x16 (&a0)[4], f32x16 (&a1)[4]) __attribute__((always_inline)) {
    float run0 = -INFINITY, run1 = -INFINITY;
    if (j_prev >= 0) {
      offer(p_prev, j_prev);
      j_prev = -1;
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (is_own && causal) {
        // Diagonal block: only keys u <= t are visible to query t.
        const int t0 = q0 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int u = j * kBlock + mt * 32 + c_row(v, lane);
          if (u > t0) a0[mt][v] = -INFINITY;
          if (u > t0 + 32) a1[mt][v] = -INFINITY;
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        run0 = fmaxf(run0, a0[mt][v]);
        run1 = fmaxf(run1, a1[mt][v]);
      }
    }
    // Lanes l and l^32 hold the two key halves of the same query column.
    const float recv = swap_half(lane < 32 ? run1 : run0);
    const float p = fmaxf(lane < 32 ? run0 : run1, recv);   // pooled score of query q0+lane
    const int tq = q0 + lane;
    if (pooled != nullptr && tq < N) pooled[(((size_t)b * N + tq) * H_kv + g) * nblk + j] = p;
    if (!is_own) {
      p_prev = p;
      j_prev = j;
    }
  };
  // Half-block passes (64 keys, 64 accumulator registers): the products of
  // row tiles 2h, 2h+1 and their running maximum.  FP8 with lists of up to 15
  // takes a block in two such passes, which leaves room for three waves per
  // SIMD (154 VGPRs against 210): 4.2 -> 3.7 ms at N = 128K, 233 -> 214 ms at
  // 1M.  bf16 keeps the whole-block products: its B operands and staging take
  // 24 more registers, so the same scheme spilled (8 VGPRs) and ran 2-8%
  // slower.
  auto products_half = [&](int buf, int h, f32x16 (&a0)[2], f32x16 (&a1)[2]) __attribute__((always_inline)) {
    const T* tile = lds + buf * C::TILE_ELEMS;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mt = 2 * h + m;
      a0[m] = zero16();
      a1[m] = zero16();
      const T* ap = tile + (mt * 32 + (lane & 31)) * C::PITCH + KPL * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        const typename M::frag a = M::load(ap + ks * 2 * KPL);
        a0[m] = M::mma(a, qf[0][ks], a0[m]);
        a1[m] = M::mma(a, qf[1][ks], a1[m]);
      }
    }
  };
  auto pool_half = [&](int j, int h, bool is_own, f32x16 (&a0)[2], f32x16 (&a1)[2], float& run0,
                       float& run1) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mt = 2 * h + m;
      if (is_own && causal) {
        const int t0 = q0 + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int u = j * kBlock + mt * 32 + c_row(v, lane);
          if (u > t0) a0[m][v] = -INFINITY;
          if (u > t0 + 32) a1[m][v] = -INFINITY;
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        run0 = fmaxf(run0, a0[m][v]);
        run1 = fmaxf(run1, a1[m][v]);
      }
    }
  };
  auto pool_finish = [&](int j, bool is_own, float run0, float run1) __attribute__((always_inline)) {
    const float recv = swap_half(lane < 32 ? run1 : run0);
    const float p = fmaxf(lane < 32 ? run0 : run1, recv);   // pooled score of query q0+lane
    const int tq = q0 + lane;
    if (pooled != nullptr && tq < N) pooled[(((size_t)b * N + tq) * H_kv + g) * nblk + j] = p;
    if (!is_own) {
      p_prev = p;
      j_prev = j;
    }
  };
  // The next block is loaded at the top of each block and goes to the other
  // LDS buffer right after this block's products are issued, so its
  // registers are not held (or re-loaded by the compiler) across the block's
  // vector work.
  if constexpr (std::is_same<T, fp8e4m3>::value && CAP <= 15) {
    for (int j = 0; j <= jlast; ++j) {
      const int buf = j & 1;
      const bool more = j < jlast;
      if (more) load_block(j + 1);
      const bool visible = wave_valid && (!causal || j <= own);
      const bool is_own = j == own;
      const bool work = visible && (!is_own || pooled != nullptr);
      f32x16 a0[2], a1[2];
      float run0 = -INFINITY, run1 = -INFINITY;
      if (work) products_half(buf, 0, a0, a1);
      if (more) store_block(buf ^ 1);
      if (work) {
        if (j_prev >= 0) {
          offer(p_prev, j_prev);
          j_prev = -1;
        }
        pool_half(j, 0, is_own, a0, a1, run0, run1);
        products_half(buf, 1, a0, a1);
      }
      __syncthreads();
      if (work) {
        pool_half(j, 1, is_own, a0, a1, run0, run1);
        pool_finish(j, is_own, run0, run1);
      }
    }
  } else if constexpr (!std::is_same<T, float>::value) {
    // bf16 and FP8: the barrier that completes the next block's tile comes
    // before this block's vector work (measured: FP8 3.6% faster at 1M).
    // bf16 up to topk 16 then reads the next block's row tile 0 right after
    // it, so that block's first products wait on no LDS read (1.7% faster at
    // 128K and 1M; the longer lists have no registers for it).
    constexpr bool kAhead = std::is_same<T, bf16>::value && CAP <= 15;
    if (kAhead) read_ahead(0);
    for (int j = 0; j <= jlast; ++j) {
      const int buf = j & 1;
      const bool more = j < jlast;
      if (more) load_block(j + 1);
      const bool visible = wave_valid && (!causal || j <= own);
      const bool is_own = j == own;
      const bool work = visible && (!is_own || pooled != nullptr);
      f32x16 a0[4], a1[4];
      if (work) products(buf, kAhead, a0, a1);
      if (more) store_block(buf ^ 1);
      __syncthreads();
      if (kAhead && more) read_ahead(buf ^ 1);
      if (work) pool(j, is_own, a0, a1);
    }
  } else {
    // fp32: the accumulators would not fit beside the list registers through
    // the barrier, which therefore closes the block.  The body is written out
    // rather than built from the lambdas above: with them the compiler
    // allocates the fp32 instances differently and several spill far more
    // (up to 174 VGPRs at topk 64).
    for (int j = 0; j <= jlast; ++j) {
      const int buf = j & 1;
      const bool more = j < jlast;
      // The next block is loaded here and goes to the other LDS buffer right
      // after this block's products are issued, so its registers are not held
      // (or re-loaded by the compiler) across the block's vector work.
      if (more) load_block(j + 1);
      const bool visible = wave_valid && (!causal || j <= own);
      const bool is_own = j == own;
      if (visible && (!is_own || pooled != nullptr)) {
        float run0 = -INFINITY, run1 = -INFINITY;
        const T* tile = lds + buf * C::TILE_ELEMS;
        f32x16 a0[4], a1[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          a0[mt] = zero16();
          a1[mt] = zero16();
          const T* ap = tile + (mt * 32 + (lane & 31)) * C::PITCH + KPL * (lane >> 5);
#pragma unroll
          for (int ks = 0; ks < C::KSTEPS; ++ks) {
            const typename M::frag a = M::load(ap + ks * 2 * KPL);
            a0[mt] = M::mma(a, qf[0][ks], a0[mt]);
            a1[mt] = M::mma(a, qf[1][ks], a1[mt]);
          }
        }
        if (more) store_block(buf ^ 1);
        if (j_prev >= 0) {
          offer(p_prev, j_prev);
          j_prev = -1;
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          if (is_own && causal) {
            // Diagonal block: only keys u <= t are visible to query t.
            const int t0 = q0 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int u = j * kBlock + mt * 32 + c_row(v, lane);
              if (u > t0) a0[mt][v] = -INFINITY;
              if (u > t0 + 32) a1[mt][v] = -INFINITY;
            }
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            run0 = fmaxf(run0, a0[mt][v]);
            run1 = fmaxf(run1, a1[mt][v]);
          }
        }
        // Lanes l and l^32 hold the two key halves of the same query column.
        const float recv = swap_half(lane < 32 ? run1 : run0);
        const float p = fmaxf(lane < 32 ? run0 : run1, recv);   // pooled score of query q0+lane
        const int tq = q0 + lane;
        if (pooled != nullptr && tq < N) pooled[(((size_t)b * N + tq) * H_kv + g) * nblk + j] = p;
        if (!is_own) {
          p_prev = p;
          j_prev = j;
        }
      } else if (more) {
        store_block(buf ^ 1);
      }
      __syncthreads();
    }
  }
  if (j_prev >= 0) offer(p_prev, j_prev);
  flush();

  const int tq = q0 + lane;
  if (!wave_valid || tq >= N) return;
  // Own block plus the first topk-1 list entries, written in ascending order.
  int E[CAP + 1];
  E[0] = own;
#pragma unroll
  for (int i = 0; i < CAP; ++i) E[i + 1] = (i < topk - 1) ? ti[i] : -1;
  int32_t* out = block_idx + (((size_t)b * N + tq) * H_kv + g) * topk;
#pragma unroll
  for (int i = 0; i <= CAP; ++i) {
    const int ki = E[i] < 0 ? INT_MAX : E[i];
    int rank = 0;
#pragma unroll
    for (int k = 0; k <= CAP; ++k) {
      const int kk = E[k] < 0 ? INT_MAX : E[k];
      rank += (kk < ki) || (kk == ki && k < i);
    }
    if (rank < topk) out[rank] = E[i];
  }
}

__global__ void fill_f32_kernel(float* __restrict__ p, size_t n, float value) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = value;
}

template <typename T, int DIDX, int CAP>
hipError_t launch_typed(const Problem& P, const void* q_idx, const void* k_idx, int32_t* block_idx,
                        float* pooled, hipStream_t s) {
  using C = IdxCfg<T, DIDX>;
  int GT = 1;
  while (GT < kIdxWaves && P.H_kv % (GT * 2) == 0) GT *= 2;
  const int QW = kIdxWaves / GT;
  const int n_qtiles = (P.N + QW * kQPerWave - 1) / (QW * kQPerWave);
  const int n_gtiles = P.H_kv / GT;
  const dim3 grid(n_qtiles * P.B * n_gtiles);
  auto kern = index_topk_kernel<T, DIDX, CAP>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  ProfScope prof("index_topk", s);
  hipLaunchKernelGGL(kern, grid, dim3(kIdxThreads), C::LDS_BYTES, s, static_cast<const T*>(q_idx),
                     static_cast<const T*>(k_idx), block_idx, pooled, P.N, P.H_kv, P.topk, P.causal,
                     GT, n_qtiles, n_gtiles);
  return hipGetLastError();
}

template <typename T, int DIDX>
hipError_t launch_cap(const Problem& P, const void* q, const void* k, int32_t* bi, float* pooled,
                      hipStream_t s) {
  const int need = P.topk - 1;
  if (need <= 3) return launch_typed<T, DIDX, 3>(P, q, k, bi, pooled, s);
  if (need <= 7) return launch_typed<T, DIDX, 7>(P, q, k, bi, pooled, s);
  if (need <= 15) return launch_typed<T, DIDX, 15>(P, q, k, bi, pooled, s);
  if (need <= 31) return launch_typed<T, DIDX, 31>(P, q, k, bi, pooled, s);
  return launch_typed<T, DIDX, 63>(P, q, k, bi, pooled, s);
}

}  // namespace

hipError_t launch_fill_f32(float* p, size_t n, float value, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t want = (n + 255) / 256;
  const int blocks = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks), dim3(256), 0, s, p, n, value);
  return hipGetLastError();
}

hipError_t launch_index_topk(const Problem& P, const void* q_idx, const void* k_idx,
                             int32_t* block_idx, float* pooled, hipStream_t s) {
  if (pooled != nullptr) {
    hipError_t e = launch_fill_f32(pooled, (size_t)P.B * P.N * P.H_kv * P.nblk, -INFINITY, s);
    if (e != hipSuccess) return e;
  }
  if (P.dtype == MSA_FP8_E4M3) return launch_cap<fp8e4m3, 64>(P, q_idx, k_idx, block_idx, pooled, s);
  if (P.dtype == MSA_BF16) {
    if (P.d_idx == 64) return launch_cap<bf16, 64>(P, q_idx, k_idx, block_idx, pooled, s);
    return launch_cap<bf16, 32>(P, q_idx, k_idx, block_idx, pooled, s);
  }
  if (P.d_idx == 64) return launch_cap<float, 64>(P, q_idx, k_idx, block_idx, pooled, s);
  return launch_cap<float, 32>(P, q_idx, k_idx, block_idx, pooled, s);
}

}  // namespace msa
