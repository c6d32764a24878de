// Inverted block map: for every (batch, group, KV block j) the queries t that
// selected j (other than the queries of block j itself, whose "own block" is
// always j), in increasing t.  This is the transpose of block_idx.
//
// Page: "How Flash-MSA cuts million-token training cost with sparse-k",
// 'Kernel design and execution': the fused backward inverts the block-index
// map so that query chunks can be scheduled around each sparse KV block;
// "How to solve the memory problem with MiniMax Sparse Attention", 'Kernel
// optimizations': the KV-outer kernels iterate over KV blocks rather than
// queries.  Both kernels here consume this map.
//
// Layout (per (b, g) region, bg = b * H_kv + g):
//   cnt/pos [nsb + 1][nblk]  pos[s][j] = entries of list j from query
//            super-blocks < s (a super-block is SB query blocks); row nsb holds
//            the list lengths.
//   offs [nblk + 1]          start of list j inside the (b, g) entry region
//   rows [N * topk]          entries (t << 6) | slot, slot = position of j in
//                            block_idx[b, t, g, :] (at most topk - 1 per query
//                            for a well-formed row; room for topk keeps a
//                            malformed row in bounds); one spare entry follows
//                            the last region, the target of dropped stores
// Built by count -> column scan -> row scan -> ordered scatter.  Every step is
// deterministic: the scatter walks each super-block's queries in order.
#include "msa_internal.h"

namespace msa {
namespace {

// Query blocks per super-block: the smallest power of two that keeps the
// count matrix under 256 MiB.
int super_block(const Problem& P) {
  int sb = 1;
  while (sb < 64) {
    const size_t nsb = (size_t)(P.nblk + sb - 1) / sb;
    const size_t bytes = (nsb + 1) * P.nblk * sizeof(int32_t) * P.B * P.H_kv;
    if (bytes <= (size_t(256) << 20)) break;
    sb *= 2;
  }
  return sb;
}

// Count the non-own selections of every KV block inside one super-block of
// queries.  One workgroup per (b, g, super-block); counters in LDS.
__global__ __launch_bounds__(256) void bm_count_kernel(const int32_t* __restrict__ block_idx,
                                                       int32_t* __restrict__ pos, int N, int H_kv,
                                                       int topk, int nblk, int nsb, int SB) {
  extern __shared__ int32_t cnt[];
  const int s = blockIdx.x % nsb;
  const int bg = blockIdx.x / nsb;
  const int b = bg / H_kv, g = bg % H_kv;
  for (int j = threadIdx.x; j < nblk; j += blockDim.x) cnt[j] = 0;
  __syncthreads();
  const int t0 = s * SB * kBlock;
  const int t1 = min(t0 + SB * kBlock, N);
  const int n = (t1 - t0) * topk;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int t = t0 + i / topk, e = i % topk;
    const int j = block_idx[(((size_t)b * N + t) * H_kv + g) * topk + e];
    if ((unsigned)j < (unsigned)nblk && j != t / kBlock) atomicAdd(&cnt[j], 1);
  }
  __syncthreads();
  int32_t* row = pos + ((size_t)bg * (nsb + 1) + s) * nblk;
  for (int j = threadIdx.x; j < nblk; j += blockDim.x) row[j] = cnt[j];
}

// Exclusive scan of every column over super-blocks; row nsb gets the totals.
// A workgroup takes 64 columns of one (b, g): each of its 16 waves sums a run
// of rows (64 columns = 256 contiguous bytes per row), the run totals are
// scanned in LDS, and each wave rewrites its run.
constexpr int kScanSegs = 16;
__global__ __launch_bounds__(64 * kScanSegs) void bm_scan_cols_kernel(int32_t* __restrict__ pos, int nblk,
                                                                      int nsb) {
  __shared__ int32_t seg_tot[kScanSegs][64];
  const int cpb = (nblk + 63) / 64;
  const int bg = blockIdx.x / cpb;
  const int c = threadIdx.x & 63, seg = threadIdx.x >> 6;
  const int j = (blockIdx.x % cpb) * 64 + c;
  const int per = (nsb + kScanSegs - 1) / kScanSegs;
  const int s0 = min(seg * per, nsb), s1 = min(s0 + per, nsb);
  const bool ok = j < nblk;
  int32_t* base = pos + (size_t)bg * (nsb + 1) * nblk + j;
  int32_t sum = 0;
  if (ok)
    for (int s = s0; s < s1; ++s) sum += base[(size_t)s * nblk];
  seg_tot[seg][c] = sum;
  __syncthreads();
  int32_t run = 0;
  for (int k = 0; k < seg; ++k) run += seg_tot[k][c];
  if (ok) {
    for (int s = s0; s < s1; ++s) {
      const int32_t v = base[(size_t)s * nblk];
      base[(size_t)s * nblk] = run;
      run += v;
    }
    if (seg == kScanSegs - 1) base[(size_t)nsb * nblk] = run;   // the list lengths
  }
}

// Block-wide exclusive scan of `in[0..n)` into `out[0..n]` (out[n] = total),
// one workgroup of 1024 threads; each thread owns a contiguous run.
__device__ void block_exclusive_scan(const int32_t* in, int32_t* out, int n, int stride_in) {
  __shared__ int32_t part[1024];
  const int T = blockDim.x;
  const int per = (n + T - 1) / T;
  const int lo = min(threadIdx.x * per, n), hi = min(lo + per, n);
  int32_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += in[(size_t)i * stride_in];
  part[threadIdx.x] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread sums.
  for (int off = 1; off < T; off <<= 1) {
    const int32_t add = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - sum;
  for (int i = lo; i < hi; ++i) {
    const int32_t c = in[(size_t)i * stride_in];
    out[i] = run;
    run += c;
  }
  if (threadIdx.x == T - 1) out[n] = part[T - 1];
}

// offs[bg][j] = exclusive scan over j of the list lengths.
__global__ __launch_bounds__(1024) void bm_offsets_kernel(const int32_t* __restrict__ pos,
                                                          int32_t* __restrict__ offs, int nblk, int nsb) {
  const int bg = blockIdx.x;
  block_exclusive_scan(pos + ((size_t)bg * (nsb + 1) + nsb) * nblk, offs + (size_t)bg * (nblk + 1), nblk, 1);
}

// Ordered scatter: one wave per (b, g, super-block) walks its queries in
// increasing t, QW = 64 / TP of them per pass (TP = topk rounded up to a
// power of two); lane q TP + e handles entry e of the pass's query q.  The
// passes go in batches of kBatch: the batch's rows are loaded first (all in
// flight together), then the queries take their list cursors in order, q = 0
// first within a pass, and the batch's entries are stored last.  The entries
// of one row name distinct blocks, so the lanes of one query never share a
// cursor, and a single wave's LDS accesses complete in program order, so each
// query sees the cursors that the queries before it advanced.
constexpr int kBatch = 16;
__global__ __launch_bounds__(64) void bm_scatter_kernel(const int32_t* __restrict__ block_idx,
                                                        const int32_t* __restrict__ pos,
                                                        const int32_t* __restrict__ offs,
                                                        int32_t* __restrict__ rows, int N, int H_kv,
                                                        int topk, int nblk, int nsb, int SB) {
  extern __shared__ int32_t cursor[];
  // Workgroup w runs on XCD w mod 8.  When nsb is a multiple of 8, XCD x
  // takes the x-th eighth of every (b, g)'s super-blocks, in order, so the
  // entries that neighbouring super-blocks append to one list (adjacent in
  // memory) meet in one L2 instead of leaving eight as partial lines.
  int s, bg;
  if (nsb % 8 == 0) {
    const int per = nsb / 8, k = blockIdx.x / 8;
    bg = k / per;
    s = (blockIdx.x % 8) * per + k % per;
  } else {
    s = blockIdx.x % nsb;
    bg = blockIdx.x / nsb;
  }
  const int b = bg / H_kv, g = bg % H_kv;
  const int32_t* prow = pos + ((size_t)bg * (nsb + 1) + s) * nblk;
  const int32_t* orow = offs + (size_t)bg * (nblk + 1);
  // Cursors: 8 columns per lane per round, all loads in flight together.
  for (int j0 = threadIdx.x; j0 < nblk; j0 += 8 * 64) {
    int32_t o[8], c[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int jc = min(j0 + 64 * k, nblk - 1);
      o[k] = orow[jc];
      c[k] = prow[jc];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (j0 + 64 * k < nblk) cursor[j0 + 64 * k] = o[k] + c[k];
  }
  __syncthreads();
  const int cap = N * topk;   // per (b, g): a row holds at most topk entries
  int32_t* out = rows + (size_t)bg * cap;
  int32_t* spare = rows + (size_t)(gridDim.x / nsb) * cap;   // one past the last region
  const int t0 = s * SB * kBlock;
  const int t1 = min(t0 + SB * kBlock, N);
  int TP = 1;
  while (TP < topk) TP *= 2;
  const int QW = 64 / TP;                      // queries per pass (TP <= 64)
  const int q = threadIdx.x / TP, e = threadIdx.x % TP;
  const bool lane_on = e < topk;
  // Loads at clamped, in-bounds addresses (t0 < t1 for every super-block);
  // lanes and queries out of range are dropped when the value is used.
  const int32_t* src = block_idx + (((size_t)b * N) * H_kv + g) * topk + min(e, topk - 1);
  const size_t tstride = (size_t)H_kv * topk;
  for (int tb0 = t0; tb0 < t1; tb0 += kBatch * QW) {
    int jr[kBatch], pr[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) jr[k] = src[(size_t)min(tb0 + k * QW + q, t1 - 1) * tstride];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int t = tb0 + k * QW + q;
      const int j = (lane_on && t < t1) ? jr[k] : -1;
      const bool on = (unsigned)j < (unsigned)nblk && j != t / kBlock;
      int p = -1;
      for (int qq = 0; qq < QW; ++qq) {
        if (on && q == qq) {
          p = cursor[j];
          cursor[j] = p + 1;
        }
      }
      pr[k] = on && (unsigned)p < (unsigned)cap ? p : -1;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int t = tb0 + k * QW + q;
      *(pr[k] >= 0 ? out + pr[k] : spare) = (t << 6) | e;   // dropped lanes write the spare entry
    }
  }
}

}  // namespace

int block_map_super_span(const Problem& P) { return super_block(P) * kBlock; }

size_t block_map_bytes(const Problem& P) {
  const int SB = super_block(P);
  const size_t nsb = (size_t)(P.nblk + SB - 1) / SB;
  const size_t bg = (size_t)P.B * P.H_kv;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  return al(bg * (nsb + 1) * P.nblk * 4) + al(bg * (P.nblk + 1) * 4) +
         al((bg * (size_t)P.N * P.topk + 1) * 4) + al((bg * P.nblk + 1) * 4) + al(64 * 4);
}

void block_map_carve(const Problem& P, void* ws, BlockMap* m) {
  const int SB = super_block(P);
  const size_t nsb = (size_t)(P.nblk + SB - 1) / SB;
  const size_t bg = (size_t)P.B * P.H_kv;
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  char* p = static_cast<char*>(ws);
  m->pos = reinterpret_cast<int32_t*>(p);
  p += al(bg * (nsb + 1) * P.nblk * 4);
  m->offs = reinterpret_cast<int32_t*>(p);
  p += al(bg * (P.nblk + 1) * 4);
  m->rows = reinterpret_cast<int32_t*>(p);
  p += al((bg * (size_t)P.N * P.topk + 1) * 4);   // + the spare entry
  m->tiles = reinterpret_cast<int32_t*>(p);
  p += al((bg * P.nblk + 1) * 4);
  m->counters = reinterpret_cast<int32_t*>(p);
  m->SB = SB;
  m->nsb = (int)nsb;
}

hipError_t launch_block_map(const Problem& P, const int32_t* block_idx, const BlockMap& m,
                            int /*tile_rows*/, hipStream_t s) {
  const int n_bg = P.B * P.H_kv;
  const size_t lds = (size_t)P.nblk * sizeof(int32_t);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  hipError_t e;
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bm_count_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(bm_scatter_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  ProfScope prof("block_map", s);
  hipLaunchKernelGGL(bm_count_kernel, dim3(n_bg * m.nsb), dim3(256), lds, s, block_idx, m.pos, P.N,
                     P.H_kv, P.topk, P.nblk, m.nsb, m.SB);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int cols_per_bg = (P.nblk + 63) / 64;
  hipLaunchKernelGGL(bm_scan_cols_kernel, dim3(n_bg * cols_per_bg), dim3(64 * kScanSegs), 0, s, m.pos, P.nblk,
                     m.nsb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bm_offsets_kernel, dim3(n_bg), dim3(1024), 0, s, m.pos, m.offs, P.nblk, m.nsb);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (P.topk > 1) {
    hipLaunchKernelGGL(bm_scatter_kernel, dim3(n_bg * m.nsb), dim3(64), lds, s, block_idx, m.pos, m.offs,
                       m.rows, P.N, P.H_kv, P.topk, P.nblk, m.nsb, m.SB);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// Work items of the KV-outer kernels for the query range [c0, c1): per list
// (b, g, j) one diagonal item when block j lies in the range (its own 128
// queries, causal mask) plus ceil(len / item_queries) items over the list
// segment of the range; with merge_diag the diagonal queries join the first
// list item instead (at least one item per list in range).  tiles[] =
// exclusive scan over lists, tiles[n] = total.
namespace {
__global__ __launch_bounds__(1024) void bm_items_kernel(const int32_t* __restrict__ pos,
                                                        int32_t* __restrict__ tiles, int nblk, int nsb,
                                                        int n_bg, int s_lo, int s_hi, int jb_lo, int jb_hi,
                                                        int item_queries, int merge_diag) {
  // Count items per list into tiles[], then scan in place (two passes over a
  // small array; one workgroup).
  const int n = n_bg * nblk;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int bg = i / nblk, j = i % nblk;
    const int32_t* pb = pos + (size_t)bg * (nsb + 1) * nblk + j;
    const int len = pb[(size_t)s_hi * nblk] - pb[(size_t)s_lo * nblk];
    const int diag = (j >= jb_lo && j < jb_hi) ? 1 : 0;
    const int lists = (len + item_queries - 1) / item_queries;
    // merge_diag: the diagonal queries ride along with the first list item.
    tiles[i] = merge_diag ? (diag ? max(1, lists) : lists) : diag + lists;
  }
  __syncthreads();
  // In-place exclusive scan with a one-workgroup pass over contiguous runs.
  __shared__ int32_t part[1024];
  const int T = blockDim.x;
  const int per = (n + T - 1) / T;
  const int lo = min((int)threadIdx.x * per, n), hi = min(lo + per, n);
  int32_t sum = 0;
  for (int i = lo; i < hi; ++i) sum += tiles[i];
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < T; off <<= 1) {
    const int32_t add = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  int32_t run = part[threadIdx.x] - sum;
  for (int i = lo; i < hi; ++i) {
    const int32_t c = tiles[i];
    tiles[i] = run;
    run += c;
  }
  if (threadIdx.x == T - 1) tiles[n] = part[T - 1];
}
}  // namespace

hipError_t launch_block_items(const Problem& P, const BlockMap& m, int q_lo, int q_hi, int item_queries,
                              hipStream_t s, int merge_diag) {
  const int n_bg = P.B * P.H_kv;
  const int s_lo = q_lo / (m.SB * kBlock);
  const int s_hi = (q_hi == P.N) ? m.nsb : q_hi / (m.SB * kBlock);
  ProfScope prof("block_items", s);
  hipLaunchKernelGGL(bm_items_kernel, dim3(1), dim3(1024), 0, s, m.pos, m.tiles, P.nblk, m.nsb, n_bg, s_lo,
                     s_hi, q_lo / kBlock, (q_hi + kBlock - 1) / kBlock, item_queries, merge_diag);
  return hipGetLastError();
}

size_t block_items_upper_bound(const Problem& P, int q_lo, int q_hi, int item_queries) {
  const size_t n_bg = (size_t)P.B * P.H_kv;
  const size_t diag = (size_t)(q_hi - q_lo + kBlock - 1) / kBlock;
  const size_t entries = (size_t)(q_hi - q_lo) * P.topk;
  return n_bg * (diag + P.nblk + entries / item_queries + 1);
}

}  // namespace msa
