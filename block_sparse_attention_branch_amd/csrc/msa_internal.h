// Internal declarations and device helpers shared by the libmsa kernels.
// Not part of the public interface (include/msa.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/msa.h"

namespace msa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kBlock = 128;     // KV block size the kernels are built for
constexpr int kWave = 64;       // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// MFMA fragments.  A 32x32 output tile D[m][n] lives in 16 fp32 slots per
// lane: lane l holds column n = l % 32 and rows m = 8*(v/4) + 4*(l/32) + v%4
// for slot v (checked on gfx950 hardware).  A-operand lane l holds row
// m = l % 32, B-operand lane l holds column n = l % 32; both hold the same
// KPL consecutive k values, k = KPL*(l/32) + i, of the instruction's 2*KPL.
// ---------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  typedef bf16x8 frag;
  static constexpr int KPL = 8;   // k values per lane per instruction
  __device__ static inline frag load(const bf16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// One OCP FP8 E4M3 value (the element type of FP8 index inputs).
struct fp8e4m3 {
  uint8_t bits;
};
typedef int i32x8 __attribute__((ext_vector_type(8)));
// Native 4 x 32-bit vector (the type the nontemporal builtins take).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
// gfx950 FP8 matrix unit, 32x32x64 per instruction: lane l holds 32
// consecutive k values of row (A) or column (B) l % 32, the half of k chosen
// by l / 32, as for the other 32x32 forms; both operands E4M3 (format code 0)
// with unit block scales (E8M0 exponent 127).
template <> struct Mma<fp8e4m3> {
  typedef i32x8 frag;
  static constexpr int KPL = 32;
  __device__ static inline frag load(const fp8e4m3* p) {
    const uint4 lo = *reinterpret_cast<const uint4*>(p);
    const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
    frag r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
  }
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

template <> struct Mma<float> {
  typedef float frag;
  static constexpr int KPL = 1;
  __device__ static inline frag load(const float* p) { return *p; }
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Row index inside a 32x32 tile held by slot v of lane l.
__device__ inline int c_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Exchange a value with the lane 32 places away (lane l <-> l ^ 32).
__device__ inline float swap_half(float x) { return __shfl_xor(x, 32); }
__device__ inline int swap_half(int x) { return __shfl_xor(x, 32); }

// Work item of this workgroup among `total`, or -1: item i is workgroup i.
// Workgroups are dealt to the 8 XCDs in turn (workgroup i runs on XCD i % 8),
// so neighbouring items, which cover the same KV block, land on different
// XCDs.  That spreads the uneven item costs (ragged last tiles, diagonal
// items, long and short lists) evenly over the XCDs; a contiguous run of
// items per XCD kept a block's K/V in one L2 but measured slower (forward
// 16.4 -> 14.9 ms, backward 45.3 -> 43.5 ms at N = 128K), K/V being a small
// part of an item's bytes.
__device__ inline int xcd_item(int total) {
  const int w = (int)blockIdx.x;
  return w < total ? w : -1;
}

// ---------------------------------------------------------------------------
// Launchers (one per kernel family); each returns hipGetLastError().
// ---------------------------------------------------------------------------
struct Problem {
  int B, N, H_q, H_kv, G, d, d_idx, topk, causal, dtype, nblk;
  float scale, scale_idx;
};

hipError_t launch_fill_f32(float* p, size_t n, float value, hipStream_t s);

// Measurement hooks around kernel launches (no-ops unless timing is enabled
// through msa_profile_enable).  Each prof_begin is closed by one prof_end on
// the same thread and stream.
void prof_begin(const char* name, hipStream_t s);
void prof_end(hipStream_t s);
// One timed region: prof_begin on construction, prof_end on every way out of
// the scope (early error returns included), so a recorded start event is
// never left pending.
struct ProfScope {
  hipStream_t s;
  ProfScope(const char* name, hipStream_t st) : s(st) { prof_begin(name, st); }
  ~ProfScope() { prof_end(s); }
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;
};

hipError_t launch_index_topk(const Problem& P, const void* q_idx, const void* k_idx,
                             int32_t* block_idx, float* pooled, hipStream_t s);

// Inverted block map (CSR of the queries that selected each KV block).
struct BlockMap {
  int32_t* pos;      // [B*H_kv][nsb + 1][nblk]: entries of list j from super-blocks < s
  int32_t* offs;     // [B*H_kv][nblk + 1]: start of list j in the (b, g) entry region
  int32_t* rows;     // [B*H_kv][N * topk]: entries (t << 6) | slot, t-sorted per list
  int32_t* tiles;    // [B*H_kv*nblk + 1]: exclusive scan of work items per list
  int32_t* counters; // small scratch
  int SB;            // query blocks per super-block
  int nsb;           // super-blocks
};
size_t block_map_bytes(const Problem& P);
void block_map_carve(const Problem& P, void* ws, BlockMap* m);
hipError_t launch_block_map(const Problem& P, const int32_t* block_idx, const BlockMap& m,
                            int tile_rows, hipStream_t s);
// Work items of the KV-outer kernels for queries [q_lo, q_hi) (q_lo a
// multiple of the super-block span).
hipError_t launch_block_items(const Problem& P, const BlockMap& m, int q_lo, int q_hi,
                              int item_queries, hipStream_t s, int merge_diag = 0);
size_t block_items_upper_bound(const Problem& P, int q_lo, int q_hi, int item_queries);
int block_map_super_span(const Problem& P);  // queries per super-block

size_t sparse_fwd_partials_bytes(const Problem& P, int chunk_queries);
hipError_t launch_sparse_fwd(const Problem& P, const void* q, const void* k, const void* v,
                             const int32_t* block_idx, void* o, float* lse, const BlockMap& m,
                             void* partials, int chunk_queries, hipStream_t s);

// Backward: caller tensors and the library's scratch.
struct BwdArgs {
  const void *q, *k, *v, *o, *dO;
  const float* lse;
  const int32_t* block_idx;
  const void *q_idx, *k_idx;
  float kl_weight;
  void *dq, *dk, *dv;
  float *dq_idx, *dk_idx, *dscore, *kl;
};
struct BwdScratch {
  float* D;            // [B, N, H_q]   rowsum(dO * O)
  float2* idx_part;    // [B, N, H_kv, topk] per-slot (max, sum) of the index logits
  float* lse_idx;      // [B, N, H_kv]  index log-sum-exp over the selected support
  bf16* dq_part;       // [B, chunk, topk, H_q, d] + 1 spare row: dQ partials per selected block
  float* dk_acc;       // [B, N, H_kv, d] fp32
  float* dv_acc;       // [B, N, H_kv, d] fp32
};
int bwd_chunk_queries(const Problem& P);
size_t sparse_bwd_scratch_bytes(const Problem& P);
void sparse_bwd_scratch_carve(const Problem& P, void* ws, BwdScratch* w);
hipError_t launch_sparse_bwd(const Problem& P, const BwdArgs& a, const BlockMap& m, const BwdScratch& w,
                             hipStream_t s);

}  // namespace msa
