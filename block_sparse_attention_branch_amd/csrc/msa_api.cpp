// C-ABI entry points of libmsa: argument validation, workspace planning and
// kernel dispatch on the caller's stream.  The interface and its conventions
// are documented in include/msa.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "msa_internal.h"

// Fixed device scratch of msa_sparse_fwd_noalloc: the block map and the
// forward partials of one query chunk.  Each device holds its own copy from
// the moment the library's code object is loaded there until the process
// ends.  In host code `scratch` names a host-side stand-in, never the device
// array: kernels and copies take the address from scratch_ptr() instead.
static __device__ __align__(256) unsigned char scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MSA_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Largest sequence length the block map's entry encoding (t << 6 | slot)
// can hold in an int32.
constexpr int kMaxN = 1 << 22;

int check_dims(const msa_dims* d, msa::Problem* P) {
  if (d == nullptr) return fail(MSA_ERR_INVALID_ARG, "dims is NULL");
  if (d->B <= 0 || d->N <= 0 || d->H_q <= 0 || d->H_kv <= 0 || d->d <= 0 || d->d_idx <= 0 ||
      d->block_size <= 0 || d->topk <= 0)
    return fail(MSA_ERR_INVALID_ARG,
                "dimensions must be positive (B=%d N=%d H_q=%d H_kv=%d d=%d d_idx=%d block_size=%d topk=%d)",
                d->B, d->N, d->H_q, d->H_kv, d->d, d->d_idx, d->block_size, d->topk);
  if (d->H_q % d->H_kv != 0)
    return fail(MSA_ERR_INVALID_ARG, "H_q=%d is not a multiple of H_kv=%d", d->H_q, d->H_kv);
  if (d->causal != 0 && d->causal != 1) return fail(MSA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (d->dtype != MSA_F32 && d->dtype != MSA_BF16 && d->dtype != MSA_FP8_E4M3)
    return fail(MSA_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
  if (!std::isfinite(d->scale) || d->scale < 0.f || !std::isfinite(d->scale_idx) || d->scale_idx < 0.f)
    return fail(MSA_ERR_INVALID_ARG, "scale and scale_idx must be finite and >= 0");
  if (d->block_size != msa::kBlock)
    return fail(MSA_ERR_UNSUPPORTED, "block_size=%d (only %d is built)", d->block_size, msa::kBlock);
  if (d->N % msa::kBlock != 0)
    return fail(MSA_ERR_UNSUPPORTED, "N=%d is not a multiple of the block size %d", d->N, msa::kBlock);
  if (d->N > kMaxN) return fail(MSA_ERR_UNSUPPORTED, "N=%d exceeds %d", d->N, kMaxN);
  // Query-row indices (b, t, head) are 32-bit inside the kernels.
  if ((long long)d->B * d->N * d->H_q > 0x7fffffffLL)
    return fail(MSA_ERR_UNSUPPORTED, "B*N*H_q=%lld rows exceed 2^31-1", (long long)d->B * d->N * d->H_q);
  if (d->d != 64 && d->d != 128) return fail(MSA_ERR_UNSUPPORTED, "head dim d=%d (64 or 128)", d->d);
  if (d->d_idx != 32 && d->d_idx != 64)
    return fail(MSA_ERR_UNSUPPORTED, "index dim d_idx=%d (32 or 64)", d->d_idx);
  // Slots live in 6 bits of the block map's entries (t << 6 | slot).
  if (d->topk > 64) return fail(MSA_ERR_UNSUPPORTED, "topk=%d (at most 64)", d->topk);
  const int G = d->H_q / d->H_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(MSA_ERR_UNSUPPORTED, "group size H_q/H_kv=%d (1, 2, 4, 8 or 16)", G);
  P->B = d->B;
  P->N = d->N;
  P->H_q = d->H_q;
  P->H_kv = d->H_kv;
  P->G = G;
  P->d = d->d;
  P->d_idx = d->d_idx;
  P->topk = d->topk;
  P->causal = d->causal;
  P->dtype = d->dtype;
  P->nblk = d->N / msa::kBlock;
  P->scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->d);
  P->scale_idx = d->scale_idx > 0.f ? d->scale_idx : 1.0f / std::sqrt((float)d->d_idx);
  return MSA_OK;
}

// The main branch takes fp32 or bf16; FP8 is an index-branch format only.
int check_main_dtype(const msa::Problem& P) {
  if (P.dtype == MSA_FP8_E4M3)
    return fail(MSA_ERR_UNSUPPORTED, "dtype FP8 E4M3 is accepted by msa_index_topk only");
  return MSA_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (have < need) return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", have, need);
  if (need > 0 && ws == nullptr) return fail(MSA_ERR_INVALID_ARG, "workspace is NULL");
  return MSA_OK;
}

#define REQUIRE(ptr)                                                                       \
  do {                                                                                     \
    if ((ptr) == nullptr) return fail(MSA_ERR_INVALID_ARG, "required pointer %s is NULL", #ptr); \
  } while (0)

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Queries per forward launch, a multiple of the block map's super-block span.
// Two bounds:
// - the partial-result buffer (one output row in the dtype plus one fp32
//   log-sum-exp per (batch, query, head, slot)) stays within ~40 GiB;
// - the q rows that one (batch, group) slice of a chunk reads (G heads per
//   query) stay within 128 MiB. Work items run in (batch, group, block)
//   order, so about one such slice is live at a time, and a query's q rows,
//   read again for each of its selected blocks, then come back from the
//   256 MB last-level cache rather than HBM. At N = 128K with 64/8 heads and
//   d = 128 that gives two launches of 64K queries: 15.7 -> 14.4 ms against
//   one launch. The backward main kernel measured slower when chunked this
//   way, so its chunks keep the buffer bound alone.
int fwd_chunk_queries(const msa::Problem& P) {
  const size_t esz = P.dtype == MSA_BF16 ? 2 : 4;
  const size_t per_query = (size_t)P.B * P.H_q * P.topk * (P.d * esz + sizeof(float));
  const size_t cap = size_t(40) << 30;
  const size_t span = (size_t)msa::block_map_super_span(P);
  size_t q = cap / per_query;
  const size_t q_slice = (size_t(128) << 20) / ((size_t)P.G * P.d * esz);
  if (q > q_slice) q = q_slice;
  q -= q % span;
  if (q < span) q = span;
  if (q >= (size_t)P.N) q = P.N;
  return (int)q;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with hipGetSymbolAddress while that device is current.
int scratch_ptr(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_fwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_fwd_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
  if (s != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return hip_fail(e, "msa_sparse_fwd_noalloc: hipStreamGetDevice");
    if (sdev != dev)
      return fail(MSA_ERR_INVALID_ARG, "msa_sparse_fwd_noalloc: the stream belongs to device %d, device %d is current",
                  (int)sdev, dev);
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "msa_sparse_fwd_noalloc: hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(MSA_ERR_HIP, "msa_sparse_fwd_noalloc: scratch has no device address");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MSA_OK;
}

// Query chunk of the forward when the block map and the partials must share
// `cap` bytes: the default chunk if its partials fit beside the map, else the
// largest multiple of the super-block span that does; 0 when not even one
// span fits.
int fwd_chunk_within(const msa::Problem& P, size_t map_bytes, size_t cap) {
  if (map_bytes >= cap) return 0;
  auto fits = [&](int c) { return map_bytes + align_up(msa::sparse_fwd_partials_bytes(P, c)) <= cap; };
  const int chunk = fwd_chunk_queries(P);
  if (fits(chunk)) return chunk;
  const int span = msa::block_map_super_span(P);
  const size_t esz = P.dtype == MSA_BF16 ? 2 : 4;
  const size_t per_query = (size_t)P.B * P.H_q * P.topk * (P.d * esz + sizeof(float));
  size_t c = (cap - map_bytes) / per_query;
  if (c > (size_t)chunk) c = chunk;
  c -= c % span;
  // Each of the partials' two regions is rounded up to 256 bytes.
  while (c > 0 && !fits((int)c)) c -= span;
  return (int)c;
}

// Kernel timing (see msa_profile_enable in msa.h).
struct ProfRecord {
  const char* name;
  hipEvent_t start, stop;
};
std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
std::vector<ProfRecord> g_prof_records;
std::vector<hipEvent_t> g_prof_pool;
thread_local const char* t_prof_name = nullptr;
thread_local hipEvent_t t_prof_start = nullptr;

hipEvent_t prof_event() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace msa {

void prof_begin(const char* name, hipStream_t s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  hipEvent_t e = prof_event();
  if (e == nullptr) return;
  (void)hipEventRecord(e, s);
  t_prof_name = name;
  t_prof_start = e;
}

void prof_end(hipStream_t s) {
  if (t_prof_start == nullptr) return;
  hipEvent_t e = prof_event();
  if (e != nullptr) {
    (void)hipEventRecord(e, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_records.push_back({t_prof_name, t_prof_start, e});
  } else {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pool.push_back(t_prof_start);
  }
  t_prof_start = nullptr;
}

}  // namespace msa

extern "C" {

MSA_API int msa_profile_enable(int on) {
  g_prof_on.store(on != 0);
  return MSA_OK;
}

MSA_API int msa_profile_collect(int max, const char** names, int* launches, double* total_ms) {
  if (max < 0 || (max > 0 && (names == nullptr || launches == nullptr || total_ms == nullptr)))
    return fail(MSA_ERR_INVALID_ARG, "msa_profile_collect: bad output arrays");
  std::vector<ProfRecord> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof_records);
  }
  int n = 0;
  for (const ProfRecord& r : recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess)
      ms = 0.f;
    int i = 0;
    while (i < n && std::strcmp(names[i], r.name) != 0) ++i;
    if (i == n) {
      if (n == max) continue;
      names[n] = r.name;
      launches[n] = 0;
      total_ms[n] = 0.0;
      ++n;
    }
    launches[i] += 1;
    total_ms[i] += ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (const ProfRecord& r : recs) {
      g_prof_pool.push_back(r.start);
      g_prof_pool.push_back(r.stop);
    }
  }
  return n;
}

MSA_API int msa_version(void) { return 1; }

MSA_API const char* msa_status_string(int status) {
  switch (status) {
    case MSA_OK: return "ok";
    case MSA_ERR_INVALID_ARG: return "invalid argument";
    case MSA_ERR_UNSUPPORTED: return "unsupported problem";
    case MSA_ERR_WORKSPACE: return "workspace too small";
    case MSA_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

MSA_API const char* msa_last_error(void) { return g_last_error.c_str(); }

MSA_API size_t msa_index_topk_workspace(const msa_dims* dims) {
  msa::Problem P;
  if (check_dims(dims, &P) != MSA_OK) return 0;
  return 0;
}

MSA_API int msa_index_topk(const msa_dims* dims, const void* q_idx, const void* k_idx,
                           int32_t* block_idx, float* pooled, void* workspace,
                           size_t workspace_bytes, void* stream) {
  msa::Problem P;
  int st = check_dims(dims, &P);
  if (st != MSA_OK) return st;
  if (P.dtype == MSA_FP8_E4M3 && P.d_idx != 64)
    return fail(MSA_ERR_UNSUPPORTED, "FP8 E4M3 index inputs need d_idx=64 (got %d)", P.d_idx);
  REQUIRE(q_idx);
  REQUIRE(k_idx);
  REQUIRE(block_idx);
  st = check_ws(workspace, workspace_bytes, 0);
  if (st != MSA_OK) return st;
  hipError_t e = msa::launch_index_topk(P, q_idx, k_idx, block_idx, pooled, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "msa_index_topk launch");
  return ok();
}

MSA_API size_t msa_sparse_fwd_workspace(const msa_dims* dims) {
  msa::Problem P;
  if (check_dims(dims, &P) != MSA_OK || check_main_dtype(P) != MSA_OK) return 0;
  return align_up(msa::block_map_bytes(P)) + align_up(msa::sparse_fwd_partials_bytes(P, fwd_chunk_queries(P)));
}

MSA_API int msa_sparse_fwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                           const int32_t* block_idx, void* o, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  msa::Problem P;
  int st = check_dims(dims, &P);
  if (st != MSA_OK) return st;
  if ((st = check_main_dtype(P)) != MSA_OK) return st;
  REQUIRE(q);
  REQUIRE(k);
  REQUIRE(v);
  REQUIRE(block_idx);
  REQUIRE(o);
  REQUIRE(lse);
  const int chunk = fwd_chunk_queries(P);
  const size_t map_bytes = align_up(msa::block_map_bytes(P));
  st = check_ws(workspace, workspace_bytes, map_bytes + align_up(msa::sparse_fwd_partials_bytes(P, chunk)));
  if (st != MSA_OK) return st;
  msa::BlockMap m;
  msa::block_map_carve(P, workspace, &m);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = msa::launch_block_map(P, block_idx, m, 0, s);
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_fwd block map");
  e = msa::launch_sparse_fwd(P, q, k, v, block_idx, o, lse, m, static_cast<char*>(workspace) + map_bytes,
                             chunk, s);
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_fwd launch");
  return ok();
}

MSA_API int msa_sparse_fwd_noalloc(const msa_dims* dims, const void* q, const void* k, const void* v,
                                   const int32_t* block_idx, void* o, float* lse, void* stream) {
  msa::Problem P;
  int st = check_dims(dims, &P);
  if (st != MSA_OK) return st;
  if ((st = check_main_dtype(P)) != MSA_OK) return st;
  REQUIRE(q);
  REQUIRE(k);
  REQUIRE(v);
  REQUIRE(block_idx);
  REQUIRE(o);
  REQUIRE(lse);
  const size_t map_bytes = align_up(msa::block_map_bytes(P));
  const int chunk = fwd_chunk_within(P, map_bytes, MSA_NOALLOC_SCRATCH_BYTES);
  if (chunk == 0)
    return fail(MSA_ERR_UNSUPPORTED,
                "msa_sparse_fwd_noalloc: the block map (%zu bytes) and the partials of %d queries (%zu bytes) "
                "exceed the fixed scratch of %zu bytes; use msa_sparse_fwd with a workspace",
                map_bytes, msa::block_map_super_span(P),
                align_up(msa::sparse_fwd_partials_bytes(P, msa::block_map_super_span(P))),
                (size_t)MSA_NOALLOC_SCRATCH_BYTES);
  hipStream_t s = (hipStream_t)stream;
  void* ws = nullptr;
  if ((st = scratch_ptr(s, &ws)) != MSA_OK) return st;
  msa::BlockMap m;
  msa::block_map_carve(P, ws, &m);
  hipError_t e = msa::launch_block_map(P, block_idx, m, 0, s);
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_fwd_noalloc block map");
  e = msa::launch_sparse_fwd(P, q, k, v, block_idx, o, lse, m, static_cast<char*>(ws) + map_bytes, chunk, s);
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_fwd_noalloc launch");
  return ok();
}

MSA_API size_t msa_sparse_bwd_workspace(const msa_dims* dims) {
  msa::Problem P;
  if (check_dims(dims, &P) != MSA_OK || check_main_dtype(P) != MSA_OK) return 0;
  if (P.dtype != MSA_BF16) return 0;
  return align_up(msa::block_map_bytes(P)) + align_up(msa::sparse_bwd_scratch_bytes(P));
}

MSA_API int msa_sparse_bwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const int32_t* block_idx, const void* q_idx, const void* k_idx,
                           float kl_weight, void* dq, void* dk, void* dv, float* dq_idx,
                           float* dk_idx, float* dscore, float* kl, void* workspace,
                           size_t workspace_bytes, void* stream) {
  msa::Problem P;
  int st = check_dims(dims, &P);
  if (st != MSA_OK) return st;
  if ((st = check_main_dtype(P)) != MSA_OK) return st;
  REQUIRE(q);
  REQUIRE(k);
  REQUIRE(v);
  REQUIRE(o);
  REQUIRE(dO);
  REQUIRE(lse);
  REQUIRE(block_idx);
  REQUIRE(q_idx);
  REQUIRE(k_idx);
  REQUIRE(dq);
  REQUIRE(dk);
  REQUIRE(dv);
  REQUIRE(dq_idx);
  REQUIRE(dk_idx);
  if (!std::isfinite(kl_weight)) return fail(MSA_ERR_INVALID_ARG, "kl_weight must be finite");
  if (P.dtype != MSA_BF16) return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_bwd supports bf16 only");
  if ((size_t)P.B * P.N * P.H_q >= (size_t(1) << 31))
    return fail(MSA_ERR_UNSUPPORTED, "msa_sparse_bwd needs B * N * H_q < 2^31 (query rows are indexed in 32 bits)");
  const size_t map_bytes = align_up(msa::block_map_bytes(P));
  st = check_ws(workspace, workspace_bytes, map_bytes + align_up(msa::sparse_bwd_scratch_bytes(P)));
  if (st != MSA_OK) return st;
  msa::BlockMap m;
  msa::block_map_carve(P, workspace, &m);
  msa::BwdScratch w;
  msa::sparse_bwd_scratch_carve(P, static_cast<char*>(workspace) + map_bytes, &w);
  msa::BwdArgs a{q, k, v, o, dO, lse, block_idx, q_idx, k_idx, kl_weight, dq, dk, dv, dq_idx, dk_idx, dscore, kl};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = msa::launch_block_map(P, block_idx, m, 0, s);
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_bwd block map");
  e = msa::launch_sparse_bwd(P, a, m, w, s);
  if (e != hipSuccess) return hip_fail(e, "msa_sparse_bwd launch");
  return ok();
}

}  // extern "C"
