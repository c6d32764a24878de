/*
 * libmsa: MiniMax Sparse Attention (MSA) over grouped-query attention, for
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Pages this interface follows (title; section):
 *   [FMSA] "How Flash-MSA cuts million-token training cost with sparse-k"
 *   [FA]   "How FlashAttention cuts GPU memory traffic without approximation"
 *   [MSA]  "How to solve the memory problem with MiniMax Sparse Attention"
 *
 * The method ([MSA] "Two-stage process: Index-Branch and Main-Branch"): an
 * index branch picks, for every query and GQA group, k KV blocks of
 * block_size tokens; a main branch then runs an exact softmax attention over
 * only the tokens of those blocks.  Training adds a KL-alignment gradient for
 * the index branch ([FMSA] "Removing the KL-divergence bottleneck").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers to caller-owned, contiguous,
 *    row-major buffers, 16-byte aligned.  The library never calls an
 *    allocator, frees or synchronises; every call only enqueues work on
 *    `stream` (a hipStream_t passed as void*; NULL means the default stream)
 *    and returns.  Its one device array of its own (the scratch of
 *    msa_sparse_fwd_noalloc) comes with its code object on each device.
 *  - Layouts ([FA] "Tiling mechanism" gives per-head Q, K, V of N rows and d
 *    columns; heads are stacked innermost-but-one):
 *        q, o, dO, dq      [B, N, H_q,  d]
 *        k, v, dk, dv      [B, N, H_kv, d]      query head h reads KV head h / G
 *        q_idx, dq_idx     [B, N, H_kv, d_idx]  one index query per group
 *        k_idx, dk_idx     [B, N, d_idx]        one index key per token, shared
 *        block_idx         [B, N, H_kv, topk]   int32
 *        lse               [B, N, H_q]          fp32, natural log
 *    with G = H_q / H_kv.  Element type of q/k/v/o/dO/dq/dk/dv/q_idx/k_idx is
 *    dims->dtype (fp32 or bf16); the types named above are fixed.
 *  - Validation runs before any launch.  On failure nothing is written and a
 *    negative status is returned; msa_last_error() then holds a message (per
 *    calling thread).  No C++ exception crosses this interface.
 *  - Workspaces: query the size with the matching *_workspace() call; pass a
 *    device buffer at least that large (NULL allowed when the size is 0).
 *    Its contents on entry do not matter and are clobbered.  Calls that share
 *    a workspace must be ordered on one stream.
 *  - Supported: block_size == 128, N a multiple of 128 and at most 2^22,
 *    B*N*H_q below 2^31, d in {64, 128},
 *    d_idx in {32, 64}, 1 <= topk <= 64, H_q % H_kv == 0 ([FA]
 *    "Architectural compatibility": GQA needs the query heads to divide into
 *    the KV heads evenly) with G = H_q / H_kv in {1, 2, 4, 8, 16}.
 *    Anything else returns MSA_ERR_UNSUPPORTED (or MSA_ERR_INVALID_ARG when it
 *    is not a valid problem at all).
 */
#ifndef LIBMSA_MSA_H
#define LIBMSA_MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_API __attribute__((visibility("default")))

/* Status codes. */
enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1,  /* null required pointer, bad dimension, H_q % H_kv != 0 */
  MSA_ERR_UNSUPPORTED = -2,  /* valid problem outside the supported shapes/dtypes */
  MSA_ERR_WORKSPACE = -3,    /* workspace smaller than the *_workspace() size */
  MSA_ERR_HIP = -4           /* a HIP launch failed (see msa_last_error) */
};

/* Element types.  MSA_FP8_E4M3 is the OCP 8-bit float E4M3 in its finite
 * form (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
 * codes 0x7F and 0xFF are NaN).  It is accepted by msa_index_topk only: the
 * indexer in a lighter format, [MSA] "Kernel optimizations". */
enum { MSA_F32 = 0, MSA_BF16 = 1, MSA_FP8_E4M3 = 2 };

/* Problem description, passed by pointer to every call. */
typedef struct msa_dims {
  int32_t B;          /* batch */
  int32_t N;          /* tokens per sequence */
  int32_t H_q;        /* query heads */
  int32_t H_kv;       /* KV heads = GQA groups = index heads */
  int32_t d;          /* head dimension of q, k, v */
  int32_t d_idx;      /* index-branch dimension of q_idx, k_idx */
  int32_t block_size; /* tokens per KV block (128 on the pages) */
  int32_t topk;       /* blocks kept per query and group (16 on the pages) */
  int32_t causal;     /* 1: query t sees keys u <= t; 0: sees every key */
  int32_t dtype;      /* element type of the call's floating inputs: MSA_F32 or
                         MSA_BF16; msa_index_topk also takes MSA_FP8_E4M3 */
  float scale;        /* main-branch score scale; 0 selects 1/sqrt(d) */
  float scale_idx;    /* index-logit scale of the KL student; 0 selects 1/sqrt(d_idx) */
} msa_dims;

/*
 * Index branch: scores, block max-pool and top-k selection.
 * [MSA] "How the indexer works"; [FMSA] "Block sparsity mechanism";
 * [MSA] "Kernel optimizations" (the exp-free top-k).
 *
 * For every (b, t, g): r[u] = q_idx[b,t,g,:] . k_idx[b,u,:] over the visible
 * keys u; pooled[j] = max of r over the visible tokens of block j;
 * block_idx[b,t,g,:] = the query's own block t / block_size plus the best
 * topk-1 other visible blocks by (pooled descending, block index ascending),
 * written in ascending order and padded with -1 when fewer than topk blocks
 * are visible.  No softmax is applied (it preserves the order).
 *
 *   q_idx      in   [B, N, H_kv, d_idx]  dtype
 *   k_idx      in   [B, N, d_idx]        dtype
 *   block_idx  out  [B, N, H_kv, topk]   int32
 *   pooled     out  [B, N, H_kv, N / block_size] fp32, nullable.  When given,
 *                   the pooled score of every block (the own block included,
 *                   pooled over its visible tokens), -inf for invisible
 *                   blocks.  Meant for tests: it costs an extra N^2/128 write.
 * Scores accumulate in fp32; for integer-valued inputs they are exact, so
 * block_idx is reproducible bit for bit.
 * dtype MSA_FP8_E4M3 (d_idx = 64 only): q_idx and k_idx are E4M3 bytes and
 * the products run on the FP8 matrix unit, accumulating in fp32.  A product
 * of two E4M3 values is exact in fp32, so the same holds for integer-valued
 * inputs.  NaN codes give an unspecified selection.
 */
MSA_API size_t msa_index_topk_workspace(const msa_dims* dims);
MSA_API int msa_index_topk(const msa_dims* dims, const void* q_idx, const void* k_idx,
                           int32_t* block_idx, float* pooled,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Main branch forward: exact softmax attention over the selected blocks,
 * storing the log-sum-exp.  [MSA] "Two-stage process" (softmax over only the
 * selected tokens, selection shared by a group's heads); [FMSA] "Kernel
 * design and execution" (output plus LSE kept for the backward pass);
 * [FA] "The online softmax trick" (partial results merged by their running
 * max and normaliser); [FA] "Architectural compatibility" (causal mask only
 * where a block straddles the diagonal).
 *
 * For head h of group g = h / G, S(t) = visible keys of the blocks in
 * block_idx[b,t,g,:] (entries < 0 ignored):
 *   s_u = scale * q[b,t,h,:] . k[b,u,g,:],  o[b,t,h,:] = sum_u softmax(s)_u v[b,u,g,:],
 *   lse[b,t,h] = ln sum_u exp(s_u).
 * block_idx must be what msa_index_topk writes: ascending, distinct, each
 * row holding the query's own block; every other entry a visible block.
 *
 *   q in [B,N,H_q,d], k, v in [B,N,H_kv,d]  dtype
 *   block_idx in [B,N,H_kv,topk] int32
 *   o   out [B,N,H_q,d] dtype;   lse out [B,N,H_q] fp32
 * Deterministic: o and lse do not depend on scheduling.
 */
MSA_API size_t msa_sparse_fwd_workspace(const msa_dims* dims);
MSA_API int msa_sparse_fwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                           const int32_t* block_idx, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * msa_sparse_fwd without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation.  Same arguments (minus the workspace), same
 * results: o and lse equal msa_sparse_fwd's bit for bit.
 *
 * The block map and the partial results live in one fixed device array of
 * MSA_NOALLOC_SCRATCH_BYTES inside the library; each device that runs this
 * call holds its own copy from the first call until the process ends.  When
 * the partials of all queries do not fit, queries run in more launches.
 * Nothing in the array needs clearing between calls (every launch writes
 * what it later reads), and no hipMemset is issued.
 *   - Device: the current device; `stream` must belong to it.  The first
 *     call on a device looks the array's address up there.
 *   - Rejected with MSA_ERR_UNSUPPORTED, before any launch, when the block
 *     map plus the partials of one super-block of queries exceed the array
 *     (for N = 128K with H_kv = 8, topk = 16, the block map alone needs
 *     64 MiB).  Other errors as msa_sparse_fwd.
 *   - Calls that overlap in time on one device race on the array: order
 *     them on one stream (or otherwise serialise them).
 * Allocates no device or host memory (with kernel timing, msa_profile_enable,
 * left off).
 */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
MSA_API int msa_sparse_fwd_noalloc(const msa_dims* dims, const void* q, const void* k, const void* v,
                                   const int32_t* block_idx, void* o, float* lse, void* stream);

/*
 * Fused backward of both branches.  [FA] "Training and the backward pass"
 * (probabilities rebuilt from the stored LSE; dV += P^T dO, dP = dO V^T);
 * [FMSA] "Kernel design and execution" (backward of the proxy and the main
 * attention fused, since the proxy's training signal needs both
 * distributions); [FMSA] "Removing the KL-divergence bottleneck" (index-score
 * gradient = proxy probability minus main probability); [MSA] "Training
 * sparse attention" (teacher = main softmax averaged over the group's heads;
 * no KL gradient into the backbone).
 *
 * Main branch, with P the softmax of the forward and D = sum_c dO*o:
 *   dS = P (dO.v_u - D);  dq = scale sum_u dS_u k_u;  dk_u += scale dS_u q;
 *   dv_u += P_u dO  (dk, dv summed over the group's heads).
 * Index branch, per (b,t,g) on the same support S(t):
 *   pbar_u = mean over the group's heads of P_u (treated as a constant),
 *   p_px = softmax_u(scale_idx * q_idx . k_idx_u),
 *   dz_u = kl_weight * (p_px_u - pbar_u),
 *   dq_idx = scale_idx sum_u dz_u k_idx_u;  dk_idx_u += scale_idx dz_u q_idx
 *   (dk_idx summed over groups).  This is the gradient of
 *   kl_weight * sum_{b,t,g} KL(pbar || p_px).
 *
 *   q, k, v, o, dO   in  as in msa_sparse_fwd (o, lse from that call)
 *   lse              in  [B,N,H_q] fp32
 *   block_idx        in  [B,N,H_kv,topk] int32
 *   q_idx, k_idx     in  as in msa_index_topk
 *   dq  out [B,N,H_q,d], dk, dv out [B,N,H_kv,d]          dtype
 *   dq_idx out [B,N,H_kv,d_idx] fp32;  dk_idx out [B,N,d_idx] fp32
 *   dscore out nullable [B,N,H_kv,topk,block_size] fp32: dz at key
 *          block_idx[slot]*block_size + offset, 0 where masked or padded.
 *          Meant for tests (it is large).
 *   kl     out nullable [B,N,H_kv] fp32: KL(pbar || p_px) per row, unweighted.
 * Only dtype bf16 is supported here.  dq is deterministic: each selected
 * block's contribution is stored as a bf16 partial and the partials of a row
 * are summed in fp32 in a fixed order.  dk, dv, dq_idx, dk_idx (and kl)
 * accumulate in fp32 with atomics, so their last bits may vary from run to run.
 */
MSA_API size_t msa_sparse_bwd_workspace(const msa_dims* dims);
MSA_API int msa_sparse_bwd(const msa_dims* dims, const void* q, const void* k, const void* v,
                           const void* o, const void* dO, const float* lse,
                           const int32_t* block_idx, const void* q_idx, const void* k_idx,
                           float kl_weight, void* dq, void* dk, void* dv,
                           float* dq_idx, float* dk_idx, float* dscore, float* kl,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Kernel timing, for measurement only.  While enabled (process-wide), every
 * entry point brackets each of its internal kernel launches with a pair of
 * hipEvents recorded on the caller's stream; msa_profile_collect() waits for
 * the recorded events and returns, per kernel name, the number of launches
 * and their summed duration since the previous collect, then forgets them.
 * Events come from a pool the library creates on first use and keeps.
 * Returns the number of entries written (at most max), or a negative status.
 * Disabled by default; costs nothing when disabled.
 */
MSA_API int msa_profile_enable(int on);
MSA_API int msa_profile_collect(int max, const char** names, int* launches, double* total_ms);

/* Text for a status code (static storage). */
MSA_API const char* msa_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
MSA_API const char* msa_last_error(void);
/* Interface version, bumped on any ABI change. */
MSA_API int msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMSA_MSA_H */
