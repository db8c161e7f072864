/*
 * cobs.h - C ABI of the MI355X (gfx950) block-sparse attention library with the
 * COBS second-order block selector.
 *
 * What it computes (sources cited by page title and section):
 *   - "COBS: Cumulant Order Block Sparse Attention" (gist.science explainer,
 *     Technisches Resuemee): sec. 2.1 ranks KV blocks by attention mass
 *     m_b = sum_{r in b} exp(q.k_r); sec. 2.2 expands ln m_b in cumulants,
 *     kappa_1 = block mean of the keys, kappa_2 = within-block key covariance;
 *     sec. 2.3 scores blocks with q.mean + 1/2 q^T Sigma q from a query-independent
 *     summary (mean + compressed covariance, top-r scaled eigenvectors).
 *   - "cumulant-order-block-sparse-attention" skill card, "Method" and
 *     "Implementation steps": keep the top-k blocks of score
 *     first-order + alpha * cumulant term.
 *   - GitHub issue "four dimensions regarding importance and connection
 *     strength" (Janus #181): compression, selection and sliding-window paths
 *     with gates g_cmp, g_slc.
 *
 * Definitions used throughout (logits are scale * q.k, scale = 1/sqrt(d) by default):
 *   blocks      b = 0..NB-1, keys [64b, min(64b+64, L)), n_b keys, NB = ceil(L/64)
 *   mu_b        mean of the block's keys
 *   diag        var_b[j] = (1/n_b) sum_r (k_r[j] - mu_b[j])^2
 *   lowrank     v_{b,i} = sqrt(lambda_i) u_i, the `rank` largest eigenpairs of
 *               C_b = (1/n_b) sum_r (k_r - mu_b)(k_r - mu_b)^T (v = 0 if lambda <= 0)
 *   score       s_{h,b} = ln n_b + scale q_h.mu_b + alpha/2 scale^2 Q2,
 *               Q2 = sum_j q_{h,j}^2 var_b[j]  or  sum_i (q_h.v_{b,i})^2
 *   group rank  shat_b = ln sum_{h in group} exp(s_{h,b} - LSE_{b' in cand} s_{h,b'})
 *   candidates  blocks whose keys all lie at positions <= t (decode: t = L-1, all blocks)
 *   selection   top-k by (shat desc, block index asc), listed in ascending block
 *               order, padded with -1 when fewer than k candidates exist
 *   branches    SLC: exact softmax over the keys of the selected blocks
 *               WIN: exact softmax over positions [max(0, t-W+1), t]       (W = window)
 *               CMP: exact softmax over pooled tokens (mean of 32 keys/values at
 *                    stride 16; token j covers [16j, 16j+32), visible iff 16j+31 <= t)
 *   output      g_cmp o_cmp + g_slc o_slc + g_win o_win, an empty branch gives 0
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; the library never
 *     allocates, frees or keeps them, and keeps no per-call state on the host.
 *   - Layouts are dense row-major, head_dim innermost, 16-byte aligned.
 *   - Calls only enqueue work on `stream` (a hipStream_t; NULL = default stream)
 *     and return without synchronising.  Asynchronous faults surface at the
 *     caller's next synchronisation.
 *   - Arguments are validated on the host before any HIP call; an invalid call
 *     returns COBS_ERR_INVALID_ARG / COBS_ERR_UNSUPPORTED / COBS_ERR_WORKSPACE
 *     and enqueues nothing.  A failed launch returns COBS_ERR_HIP.
 *   - No C++ exception crosses this boundary.  Calls are reentrant; two calls
 *     that share one workspace must not run concurrently.
 *   - Inputs holding NaN or Inf give unspecified (but in-bounds) results.
 */
#ifndef COBS_H_
#define COBS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cobs_status {
  COBS_OK = 0,
  COBS_ERR_INVALID_ARG = 1,  /* null pointer, size out of range, inconsistent shape */
  COBS_ERR_UNSUPPORTED = 2,  /* valid but not built: head_dim, group size, block size */
  COBS_ERR_WORKSPACE = 3,    /* ws_bytes smaller than cobs_workspace_bytes() */
  COBS_ERR_HIP = 4           /* a kernel launch failed */
} cobs_status;

typedef enum cobs_dtype { COBS_BF16 = 0, COBS_F32 = 1 } cobs_dtype;
/* Second-order channel of the block summaries (COBS Technisches Resuemee 2.3):
 * the diagonal of the block's key covariance, its top-r eigenvectors scaled by
 * sqrt(eigenvalue) in fp32, or the same vectors in the compressed storage of 2.3
 * (bf16 mean, FP4 eigenvectors; see cobs_summary_shapes for the layout). */
typedef enum cobs_so_kind { COBS_SO_DIAG = 0, COBS_SO_LOWRANK = 1, COBS_SO_LOWRANK_FP4 = 2 } cobs_so_kind;

/* Method parameters.  Shared by every call of one attention layer. */
typedef struct cobs_params {
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t n_q_heads;    /* H_q >= 1 */
  int32_t n_kv_heads;   /* H_kv >= 1, H_q % H_kv == 0, group G = H_q/H_kv in {1,2,4,8,16} */
  int32_t block_size;   /* must be 64 */
  int32_t top_k;        /* k in [1, 64] */
  int32_t window;       /* W >= 0; 0 disables the sliding-window branch */
  int32_t cmp_len;      /* 0 disables the compressed branch; otherwise 32 */
  int32_t cmp_stride;   /* 16 (required when cmp_len == 32) */
  int32_t so_kind;      /* cobs_so_kind */
  int32_t rank;         /* r in [1, 8] for the low-rank kinds; ignored for diag */
  float alpha;          /* >= 0; 0 = first-order (mean-pool) selector */
  float scale;          /* logit scale > 0; 0 selects 1/sqrt(head_dim) */
  int32_t kv_dtype;     /* cobs_dtype of Q, K, V and the pooled tokens */
  /* Query-subspace projection of the second-order channel (COBS Technisches
   * Resuemee 2.3, "Subraum-Projektion"; low-rank kinds only).  subspace_dim = s in
   * [1, head_dim] projects each block covariance into the span of the rows of
   * `subspace`, C' = P C P^T, and stores the top-r scaled eigenvectors of C' with
   * length vlen = s rounded up to 32 (zeros beyond s); the quadratic term becomes
   * sum_i ((P q) . v_i)^2 while the linear term keeps the full q . mu.  0 = off
   * (vlen = head_dim; `subspace` is ignored). */
  int32_t subspace_dim;
  const float* subspace; /* DEVICE [H_kv][s][d] fp32, rows orthonormal (e.g. from
                          * cobs_query_subspace); caller-owned, read by the build,
                          * update, selection, decode and prefill calls */
} cobs_params;

/* Human-readable name of a status code (static storage, never NULL). */
const char* cobs_status_string(int32_t status);

/* Checks `p` alone.  Host only. */
cobs_status cobs_validate_params(const cobs_params* p);

/* Sizes of the caller-allocated summary tensors for a [batch][H_kv][max_len][d] KV cache
 * (with a query subspace, every rank-r vector below has length vlen instead of d):
 * mu [batch][H_kv][NB][d] f32, so (diag) [batch][H_kv][NB][d] f32 or
 * so (lowrank) [batch][H_kv][NB][rank][d] f32, pooled tokens kc/vc
 * [batch][H_kv][NC][d] of kv_dtype, with NB = ceil(max_len/64) and
 * NC = (max_len-32)/16 + 1 (0 if max_len < 32 or the branch is off).
 * COBS_SO_LOWRANK_FP4: mu [batch][H_kv][NB][d] bf16 (nearest, ties to even) and
 * so [batch][H_kv][NB] records of R = round_up(rank * (d/2 + d/32), 16) bytes: for
 * each vector i, d/2 bytes of FP4 E2M1 codes (two per byte, low nibble first;
 * entry 16u + 4g + c at nibble (g * d/16 + u) * 4 + c), then for each vector
 * d/32 bytes of shared exponents (E8M0, 2^(byte-127) scales entries [32j, 32j+32))
 * and zero padding.  A group's exponent is floor(log2 max|v|) - 2, clamped to
 * [-127, 127] (an all-zero group stores byte 0 and zero codes); each entry is the
 * nearest of +-{0, .5, 1, 1.5, 2, 3, 4, 6} times the scale, ties to the even code,
 * saturating at 6 (the OCP microscaling FP4 format).  The mu and so pointers of the
 * other calls take these bytes.
 * Each out-pointer may be NULL.  Returns COBS_ERR_INVALID_ARG on bad input. */
cobs_status cobs_summary_shapes(const cobs_params* p, int32_t batch, int32_t max_len,
                                int64_t* nb_max, int64_t* nc_max,
                                size_t* mu_bytes, size_t* so_bytes, size_t* pooled_bytes);

/* Workspace bytes needed by cobs_select_topk / cobs_sparse_attn_decode /
 * cobs_sparse_attn_prefill for these sizes (n_q_tokens = 1 for decode).
 * The workspace must be zero-filled before its first use (its counters are left
 * zero by every call that completes).  Returns 0 when the arguments are invalid. */
size_t cobs_workspace_bytes(const cobs_params* p, int32_t batch, int32_t max_len, int32_t n_q_tokens);

/* Summary build (COBS Technisches Resuemee 2.2-2.3; NSA compression path).
 * Reads K once (and V for the pooled values) and writes, per (sequence, kv-head, block),
 * mu and the second-order channel, plus the pooled tokens kc, vc.
 *   seq_lens  [batch] int32 device, 1 <= L_b <= max_len
 *   K, V      [batch][H_kv][max_len][d] kv_dtype; positions >= L_b are never read
 *   mu, so    see cobs_summary_shapes; entries of blocks >= NB(L_b) are left untouched
 *   kc, vc    see cobs_summary_shapes; may be NULL iff cmp_len == 0; tokens j with
 *             16j+32 > L_b are left untouched.  Stored as kv_dtype (bf16: RNE of the
 *             fp32 mean). */
cobs_status cobs_build_summaries(const cobs_params* p, int32_t batch, int32_t max_len,
                                 const int32_t* seq_lens, const void* K, const void* V,
                                 void* mu, void* so, void* kc, void* vc, void* stream);

/* Incremental summary update after tokens are appended to the cache (the summaries
 * stay compact and query-independent as the prefix grows: COBS Technisches
 * Resuemee 2.1-2.3; NSA compression path).  K and V hold every sequence at its new
 * length; mu, so, kc, vc hold summaries valid for old_lens (from cobs_build_summaries
 * or an earlier update).  Every block that holds a position in [old_len, new_len)
 * is recomputed from its keys (mean, diagonal or rank-r channel) and every pooled
 * token whose rows [16j, 16j+32) become complete is written; all other entries are
 * left untouched, so afterwards the summaries equal a build at new_lens.
 *   old_lens, new_lens  [batch] int32 device, 0 <= old_len <= new_len <= max_len
 *                       (not checked on the device: the caller's guarantee)
 *   max_append          host upper bound of new_len - old_len (>= 1); it only sizes the
 *                       launch, every touched block is updated whatever its value
 *   K, V, mu, so, kc, vc as for cobs_build_summaries (same layouts and max_len)
 * Errors as for cobs_build_summaries; INVALID_ARG also when max_append < 1. */
cobs_status cobs_update_summaries(const cobs_params* p, int32_t batch, int32_t max_len,
                                  const int32_t* old_lens, const int32_t* new_lens, int32_t max_append,
                                  const void* K, const void* V, void* mu, void* so, void* kc, void* vc,
                                  void* stream);

/* Block scoring, group aggregation and top-k (COBS 2.1-2.3; skill card "Method").
 * Decode when q_pos0 < 0: n_q_tokens must be 1 and each sequence's query sits at
 * t = L_b - 1.  Chunked prefill when q_pos0 >= 0: query i of every sequence sits at
 * t = q_pos0 + i, and the caller guarantees q_pos0 + n_q_tokens <= L_b (checked on the
 * host only against max_len).
 *   Q          [batch][n_q_tokens][H_q][d] kv_dtype
 *   mu, so     from cobs_build_summaries over the same K
 *   sel        [batch][n_q_tokens][H_kv][top_k] int32 out, ascending, -1 padded
 *   sel_score  NULL or [batch][n_q_tokens][H_kv][NB] f32 out: shat of candidate
 *              blocks, -inf for the others
 *   ws         workspace of at least cobs_workspace_bytes(p, batch, max_len, n_q_tokens) */
cobs_status cobs_select_topk(const cobs_params* p, int32_t batch, int32_t max_len,
                             const int32_t* seq_lens, int32_t n_q_tokens, int32_t q_pos0,
                             const void* Q, const void* mu, const void* so,
                             int32_t* sel, float* sel_score,
                             void* ws, size_t ws_bytes, void* stream);

/* Selection by exact attention mass (the selection oracle of COBS Technisches
 * Resuemee 2.1, a quality diagnostic: it reads every key of every candidate block).
 * Decode only (query at t = L_b - 1).  Each block is scored by
 * ln m_b = ln sum_{r in b} exp(scale q_h . k_r) instead of the cumulant estimate; the
 * group aggregation, candidate rule, tie-break and outputs are those of
 * cobs_select_topk, so comparing the two selections measures the estimate's recall.
 *   Q    [batch][1][H_q][d] kv_dtype;  K  [batch][H_kv][max_len][d] kv_dtype
 *   sel, sel_score, ws  as for cobs_select_topk (decode).
 * Errors as for cobs_select_topk. */
cobs_status cobs_select_topk_exact(const cobs_params* p, int32_t batch, int32_t max_len,
                                   const int32_t* seq_lens, const void* Q, const void* K, int32_t* sel,
                                   float* sel_score, void* ws, size_t ws_bytes, void* stream);

/* One decode step for every sequence: selection (unless sel_in is given), then the
 * SLC, WIN and CMP branches and the gated combine (NSA three paths, COBS 2.3).
 *   Q        [batch][H_q][d] kv_dtype, query at t = L_b - 1
 *   K, V     [batch][H_kv][max_len][d] kv_dtype
 *   mu, so   summaries; may be NULL iff sel_in != NULL
 *   kc, vc   pooled tokens; may be NULL iff cmp_len == 0
 *   gates    NULL (= g_cmp 0, g_slc 1, g_win 0) or [batch][H_q][3] f32 (cmp, slc, win)
 *   sel_in   NULL or [batch][H_kv][top_k] int32 selection to use instead of scoring
 *            (entries must be -1 or valid block indices of that sequence)
 *   sel_out  NULL or [batch][H_kv][top_k] int32 out (the selection used)
 *   out      [batch][H_q][d] f32 out */
cobs_status cobs_sparse_attn_decode(const cobs_params* p, int32_t batch, int32_t max_len,
                                    const int32_t* seq_lens, const void* Q,
                                    const void* K, const void* V,
                                    const void* mu, const void* so,
                                    const void* kc, const void* vc, const float* gates,
                                    const int32_t* sel_in, int32_t* sel_out, float* out,
                                    void* ws, size_t ws_bytes, void* stream);

/* cobs_sparse_attn_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The workspace is a file-scope device array of
 * COBS_STATIC_SCRATCH_BYTES (16 MiB) that each GPU holds until the process ends; the
 * call allocates and frees nothing.
 *   Arguments, layouts and results as for cobs_sparse_attn_decode.
 *   Errors as for cobs_sparse_attn_decode; COBS_ERR_WORKSPACE when
 *   cobs_workspace_bytes(p, batch, max_len, 1) exceeds COBS_STATIC_SCRATCH_BYTES.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.  The first
 * call on a device looks the array up and zero-fills it with a kernel on `stream`;
 * make that call outside stream capture.  The status word of cobs_decode_status is in
 * the array too: query it with ws = NULL and ws_bytes = 0 (see below). */
#define COBS_STATIC_SCRATCH_BYTES (16u << 20)
cobs_status cobs_sparse_attn_decode_static(const cobs_params* p, int32_t batch, int32_t max_len,
                                           const int32_t* seq_lens, const void* Q, const void* K, const void* V,
                                           const void* mu, const void* so, const void* kc, const void* vc,
                                           const float* gates, const int32_t* sel_in, int32_t* sel_out, float* out,
                                           void* stream);

/* Status of the decode steps run on a workspace since the last query (host,
 * synchronous: waits for `stream`, then reads and clears the workspace's status word).
 * A decode step whose selected-branch workgroups wait for the selection published by
 * the unit's selecting workgroup bounds that wait (about 0.1 s of polling); a wave that
 * gives up attends to no block for that tile, so the step's output is incomplete, and
 * sets bit 0 of *flags (COBS_STATUS_WAIT_GAVE_UP).  *flags == 0 means every step since
 * the last query completed as specified.
 *   p, batch, max_len, ws, ws_bytes  as passed to cobs_sparse_attn_decode; ws = NULL with
 *           ws_bytes = 0 reads the array of cobs_sparse_attn_decode_static on the
 *           current device (flags 0 before its first call there)
 *   flags   host out
 * Errors: INVALID_ARG (null flags, null ws with ws_bytes > 0, bad sizes), WORKSPACE, HIP. */
#define COBS_STATUS_WAIT_GAVE_UP 1u
cobs_status cobs_decode_status(const cobs_params* p, int32_t batch, int32_t max_len, void* ws, size_t ws_bytes,
                               uint32_t* flags, void* stream);

/* Test hook: polls of one published selection code before a selected-branch wave gives
 * up, for every later decode call of this process (0 = give up at once, which makes a
 * step whose selected workgroups must wait report COBS_STATUS_WAIT_GAVE_UP;
 * 0xFFFFFFFF restores the default).  Not for production use. */
void cobs_set_poll_limit(uint32_t polls);

/* Chunked causal prefill of one sequence (NSA's three paths with the COBS selector at
 * every query position: COBS Technisches Resuemee 2.1-2.3 and the skill card
 * "Implementation steps"; causal candidates as in cobs_select_topk): queries at t = q_pos0 .. q_pos0+n_q_tokens-1
 * against a KV prefix of seq_len positions whose summaries were built once over
 * all seq_len keys; per (token, kv-head group) selection over the candidate blocks
 * of that token, then the three branches and the gated combine.
 *   Q        [n_q_tokens][H_q][d] kv_dtype
 *   K, V     [H_kv][seq_len][d] kv_dtype
 *   mu, so   summaries built with batch 1, max_len = seq_len
 *   kc, vc   pooled tokens (NULL iff cmp_len == 0)
 *   gates    NULL or [n_q_tokens][H_q][3] f32
 *   sel_out  NULL or [n_q_tokens][H_kv][top_k] int32 out
 *   out      [n_q_tokens][H_q][d] f32 out
 * Requires 0 <= q_pos0 and q_pos0 + n_q_tokens <= seq_len. */
cobs_status cobs_sparse_attn_prefill(const cobs_params* p, int32_t seq_len, int32_t n_q_tokens,
                                     int32_t q_pos0, const void* Q, const void* K, const void* V,
                                     const void* mu, const void* so,
                                     const void* kc, const void* vc, const float* gates,
                                     int32_t* sel_out, float* out,
                                     void* ws, size_t ws_bytes, void* stream);

/* Query subspace from calibration queries (COBS Technisches Resuemee 2.3,
 * "Subraum-Projektion": the span of the top eigenvectors of the queries' second
 * moment).  For each kv-head group, M = (1/N) sum q q^T over the group's heads of
 * every calibration token (uncentred, fp64), and P_out[h] = its top-s eigenvectors
 * (s = p->subspace_dim >= 1) as rows, largest eigenvalue first, each signed so its
 * largest-magnitude entry is positive; ties in the ranking go to the lower index.
 *   Q      [n_tokens][H_q][d] kv_dtype, DEVICE
 *   P_out  [H_kv][s][d] fp32 out, DEVICE (the buffer to pass as p->subspace)
 *   ws     DEVICE workspace of at least cobs_query_subspace_workspace_bytes(p)
 * p->subspace is not read.  Errors: INVALID_ARG (null pointer, n_tokens < 1,
 * subspace_dim < 1 or > head_dim, a diagonal so_kind), WORKSPACE, HIP. */
size_t cobs_query_subspace_workspace_bytes(const cobs_params* p);
cobs_status cobs_query_subspace(const cobs_params* p, int32_t n_tokens, const void* Q, float* P_out,
                                void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* COBS_H_ */
