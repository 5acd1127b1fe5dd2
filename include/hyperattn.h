/*
 * hyperattn.h -- C ABI of the MI355X (gfx950) HyperAttention forward pass.
 *
 * The method: "HyperAttention: Long-context Attention in Near-Linear Time"
 * (ICLR 2024).  Sources cited below:
 *   [S] the atlas.scime.ai research-map summary of that paper, sections
 *       "Approach", "Limitations", "Experimental setup";
 *   [A] the OpenReview forum page of that paper, "Abstract".
 * It approximates softmax attention D^-1 A V, A = exp(Q K^T), D = diag of
 * the row sums of A ([S] Approach): queries and keys are hashed with
 * Hamming-sorted LSH and sorted by bucket, attention is exact inside the
 * equal-size diagonal blocks of the sorted matrix, the mass outside a
 * row's block is estimated from uniformly sampled key columns, and causal
 * masking recurses on the two diagonal halves with the off-diagonal
 * quadrant handled unmasked ([S] summary and Limitations).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked "device" are HIP device pointers owned by the caller;
 *    the library never allocates or frees device memory and keeps no
 *    device state between calls, apart from the fixed scratch array of
 *    hyperattn_forward_noalloc.  "host" pointers are ordinary memory.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Device work
 *    is enqueued on it and the call returns without waiting; errors raised
 *    while the kernels run surface at the caller's next synchronisation
 *    (set HYPERATTN_SYNC=1 to wait and check after every stage).
 *  - Failure injection, for testing error propagation: with the environment
 *    variable HYPERATTN_FAIL_AT set to a stage name (proj, hash, sort,
 *    samples, gather, attend, merge, leaf, quadrant, bwd_dq, bwd_dkv), the
 *    launcher of that stage returns HA_EHIP, with a message naming the stage,
 *    before it enqueues anything; the call stops there.  Work of earlier
 *    stages is already enqueued, and outputs are undefined after any
 *    error other than an argument error.
 *  - Return value: HA_OK (0) or a negative HA_E* code.  Argument errors are
 *    detected on the host before anything is enqueued, so no output buffer
 *    is written when one is returned.  hyperattn_last_error() gives a
 *    thread-local message for the last failure of the calling thread.
 *  - Tensors are dense, row-major, with the innermost dimension last;
 *    dtype HA_BF16 (bfloat16) or HA_F32 (float32).
 *  - A = exp(Q K^T) carries no softmax scale: callers pre-scale Q and K.
 *  - Results are bitwise deterministic for fixed inputs, sizes and seed.
 */
#ifndef HYPERATTN_H
#define HYPERATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { HA_BF16 = 0, HA_F32 = 1 };

/* status codes */
enum {
  HA_OK = 0,
  HA_EINVAL = -1,       /* null pointer, negative size, bad enum value       */
  HA_EUNSUPPORTED = -2, /* valid for the method, not built here (e.g. d=96)  */
  HA_EWORKSPACE = -3,   /* workspace missing or smaller than required        */
  HA_ESHAPE = -4,       /* sizes the method cannot split (see forward)       */
  HA_EHIP = -5          /* a HIP runtime call failed                         */
};

/* hyperattn_forward_ex flags */
enum {
  /* Materialise sorted copies of Q, K, V with hyperattn_gather before the
   * attention kernel instead of loading rows through the permutations
   * (non-causal only; same results, more HBM traffic). */
  HA_FLAG_MATERIALIZE = 1,
  /* Run the block part, the sampled part and the merge as three kernels
   * (hyperattn_attend twice, then hyperattn_merge_unsort) instead of one
   * fused kernel (non-causal only; same results up to fp32 rounding). */
  HA_FLAG_UNFUSED = 2,
  /* Row-norm-sampling variant of the product ("HyperAttention: Long-context
   * Attention in Near-Linear Time", research-map summary, section Approach:
   * the product with V by row-norm sampling; "Builds on": approximate matrix
   * multiplication via row norm sampling).  The normaliser is unchanged
   * (block row sums + uniform samples, weight seg / samples); the residual
   * product (keys outside the row's block) is estimated from `samples`
   * key positions drawn with probability p_t proportional to the squared
   * norm of the value row, each kept draw weighted 1 / (samples p_t):
   *   out = (N_block + N_rownorm) / (D_block + D_uniform),
   *   lse = ln(D_block + D_uniform).
   * The draws are defined exactly (hyperattn_rownorm_samples).  Causal:
   * the leaves stay exact and every quadrant of the recursion (node id
   * `node`, keys [lo, mid)) is such a problem over its own keys -- its
   * largest weight, its CDF and Philox counters (i / 4, node, head,
   * 2 batch + 2) -- merged with the rest of the row by log-sum-exp, so a
   * row's normaliser is the plain method's.  samples = 0 gives the plain
   * method.  Not combined with the other flags. */
  HA_FLAG_ROWNORM = 4
};

/* Thread-local text of the last error returned on this thread ("" if none). */
const char* hyperattn_last_error(void);

/* Library version string. */
const char* hyperattn_version(void);

/* ------------------------------------------------------------------------
 * Whole forward pass
 * ------------------------------------------------------------------------ */

/*
 * Bytes of device workspace hyperattn_forward / hyperattn_forward_ex need
 * for these sizes.  Returns 0 for sizes that forward would reject.
 */
size_t hyperattn_workspace_bytes(int batch, int n, int d, int heads, int kv_heads,
                                 int block, int samples, int proj_bits, int causal,
                                 int min_seq_len, int dtype, int flags);

/*
 * HyperAttention forward ([S] Approach; causal recursion [S] summary and
 * Limitations).
 *
 *   q    device, [batch, heads,    n, d] of dtype
 *   k, v device, [batch, kv_heads, n, d] of dtype; query head h uses KV head
 *        h / (heads / kv_heads)
 *   out  device, [batch, heads, n, d] of dtype, written in full
 *   lse  device, [batch, heads, n] float32, natural log of the row's
 *        estimated normaliser D; may be NULL
 *   workspace  device, >= hyperattn_workspace_bytes(...) bytes, 256-byte
 *        aligned; its contents on entry do not matter
 *
 * Method parameters: block b (rows per diagonal block), samples m (uniform
 * key columns per problem), proj_bits r in [1, 16] (hash bits), causal,
 * min_seq_len s (causal leaf length bound), seed (64-bit Philox key of
 * the projections and the samples).
 *
 * Readings taken where the pages are silent: one Gaussian projection
 * matrix per call shared by Q, K, every head and every recursion node;
 * bucket order = position in the reflected-binary Gray sequence of the
 * sign code; stable sort (ties by original row); m samples iid uniform
 * with replacement over the problem's sorted key positions, shared by its
 * rows, drawn per query head, excluded for rows whose block holds them,
 * weight ns/m; the product with V re-uses those samples; non-causal calls
 * ignore min_seq_len; causal spans of length <= s are exact causal
 * attention and longer spans split into halves.
 *
 * Errors: HA_EINVAL for null q/k/v/out/workspace (when needed), batch,
 * n, heads, kv_heads < 0 or heads % kv_heads != 0, samples < 0, block < 1,
 * proj_bits outside [1, 16], bad dtype; HA_EUNSUPPORTED for d not in
 * {64, 128}, samples above 4096 (1952 for fp32 at d = 128, where the
 * kernel's K/V tiles leave less LDS for the sample lists), or flags other
 * than HA_FLAG_ROWNORM combined with causal; HA_EWORKSPACE when
 * workspace_bytes is too small.  A segment that is not a multiple of the
 * block gets a short last block, and a causal span of odd length splits
 * with its extra row in the right half (rectangular quadrant).  n == 0 or
 * batch == 0 returns HA_OK and writes nothing.
 */
int hyperattn_forward(const void* q, const void* k, const void* v, int dtype,
                      int batch, int n, int d, int heads, int kv_heads,
                      int block, int samples, int proj_bits, int causal, int min_seq_len,
                      uint64_t seed, void* out, float* lse,
                      void* workspace, size_t workspace_bytes, void* stream);

/* As hyperattn_forward, with HA_FLAG_* flags. */
int hyperattn_forward_ex(const void* q, const void* k, const void* v, int dtype,
                         int batch, int n, int d, int heads, int kv_heads,
                         int block, int samples, int proj_bits, int causal, int min_seq_len,
                         uint64_t seed, int flags, void* out, float* lse,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Forward with its intermediates ("HyperAttention: Long-context Attention in
 * Near-Linear Time", research-map summary, section Approach: the sortLSH
 * permutations, the uniform column samples, the exact block part and the
 * sampled estimate merged per row; the one-line summary and section
 * Limitations: the recursive causal split, whose quadrants are solved
 * unmasked and merged with the halves' results).
 * ------------------------------------------------------------------------ */

/*
 * Levels of sorted problems: 1 for a non-causal forward (one problem per
 * head); for a causal forward the depth of the recursion, i.e. the smallest
 * L >= 0 with ceil(n / 2^L) <= min_seq_len (0: the whole sequence is one
 * exact leaf).  Level l (0-based) holds the quadrants of the spans at depth
 * l: a span [lo, hi) longer than min_seq_len splits at mid = lo +
 * floor((hi - lo) / 2) into node ids 2 id and 2 id + 1 (root id 1), and its
 * quadrant is the non-causal problem of queries [mid, hi) over keys
 * [lo, mid).  The non-causal forward's one level is the problem of queries
 * and keys [0, n) with node id 1.  Returns -1 for n < 0, or causal with
 * min_seq_len < 1.
 */
int hyperattn_debug_levels(int n, int causal, int min_seq_len);

/*
 * Optional device buffers filled by hyperattn_forward_debug; any pointer may
 * be NULL (that buffer is not written), but o_X and lse_X of one part go
 * together.  L = hyperattn_debug_levels(...), BH = batch * heads,
 * BK = batch * kv_heads, P = 2^(L-1), m = samples.  Within level l the
 * problem whose queries start at row q0 and keys at row k0 of a head writes
 * its sorted position t at index q0 + t (queries) or k0 + t (keys) of that
 * head's n entries; entries no problem of the level covers are not written.
 */
typedef struct {
  int32_t* perm_q;   /* [L][BH][n]  sorted query position -> row (within the head) */
  int32_t* perm_k;   /* [L][BK][n]  sorted key position -> row */
  int32_t* idx;      /* [L][BH][P][m]  sample positions (sorted key positions of the
                        problem) of node id, at slot id - 2^l */
  float* o_blk;      /* [L][BH][n][d]  block part alone: softmax over the row's block keys */
  float* lse_blk;    /* [L][BH][n]     its natural-log mass (-inf when empty) */
  float* o_smp;      /* [L][BH][n][d]  sampled part alone: kept samples, weight ns / m */
  float* lse_smp;    /* [L][BH][n]     its natural-log mass, ln(ns / m) included */
  float* o_leaf;     /* [BH][n][d]     causal: exact causal attention inside each leaf, at
                        the row (not written by non-causal calls) */
  float* lse_leaf;   /* [BH][n] */
} ha_debug_dump;

/*
 * As hyperattn_forward (flags 0, same workspace) and, on the same stream,
 * the buffers of `dump`: the permutations and samples are copied from the
 * forward's own workspace after the sort and sample kernels of each level;
 * the parts come from the forward's attention kernel run once more per level
 * with the block keys alone and the samples alone, written before the
 * level's merge; the leaves from the exact-leaf kernel run once more into
 * o_leaf.  out and lse are those of hyperattn_forward.
 * Errors: as hyperattn_forward; HA_EINVAL for a null dump or an o_X / lse_X
 * pair with one pointer missing.
 */
int hyperattn_forward_debug(const void* q, const void* k, const void* v, int dtype,
                            int batch, int n, int d, int heads, int kv_heads,
                            int block, int samples, int proj_bits, int causal, int min_seq_len,
                            uint64_t seed, void* out, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream,
                            const ha_debug_dump* dump);

/* ------------------------------------------------------------------------
 * Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 * ------------------------------------------------------------------------ */

/* Size of the device scratch array behind hyperattn_forward_noalloc. */
#define HA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * As hyperattn_forward (flags 0), with the workspace taken from a device
 * array of HA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each
 * GPU it runs on until the process ends.  The call allocates nothing: no
 * hipMalloc / hipFree, no allocating library routine.  The array of the
 * current device is used (`stream` must belong to it); its device address
 * is looked up once per device, on the first call there.
 *
 * Every call on one GPU shares that GPU's array and leaves its last
 * contents in it (nothing in it has to start at zero).  Calls that overlap
 * on one GPU -- on different streams, or from different threads without
 * ordering -- race on the array and give undefined results; calls on one
 * stream are ordered and safe.
 *
 * Errors: as hyperattn_forward; HA_EWORKSPACE when these sizes need more
 * than HA_NOALLOC_SCRATCH_BYTES of workspace (hyperattn_workspace_bytes
 * gives the need: e.g. n = 131072, 32 heads, d = 64 non-causal needs about
 * 51 MB and fits; its causal forward needs an fp32 accumulator of 1.1 GB
 * and is refused); HA_EHIP when the array's address cannot be obtained.
 * Argument and size errors return before anything is enqueued.
 */
int hyperattn_forward_noalloc(const void* q, const void* k, const void* v, int dtype,
                              int batch, int n, int d, int heads, int kv_heads,
                              int block, int samples, int proj_bits, int causal, int min_seq_len,
                              uint64_t seed, void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * Rectangular non-causal problems: n_q queries and n_k keys per head (the
 * pages are silent on rectangular shapes; the reading keeps the square
 * case's structure).  Query blocks are runs of b = min(block, n_q) sorted
 * query positions, key blocks runs of b_k = ceil(b n_k / n_q) sorted key
 * positions (b_k = b when n_k = n_q); query block t pairs with key block t
 * (a short or empty last key block is allowed); `samples` key positions
 * are drawn uniformly over the n_k keys (hyperattn_sample_indices with
 * ns = n_k) with weight n_k / samples and excluded from the rows of their
 * block.
 * ------------------------------------------------------------------------ */

/* Workspace bytes for hyperattn_forward_rect (0 for invalid arguments). */
size_t hyperattn_rect_workspace_bytes(int batch, int n_q, int n_k, int d, int heads, int kv_heads, int block,
                                      int samples, int proj_bits, int dtype);

/* As hyperattn_forward (non-causal) with q [batch, heads, n_q, d], k, v
 * [batch, kv_heads, n_k, d], out [batch, heads, n_q, d], lse [batch,
 * heads, n_q].  Errors: as hyperattn_forward; HA_EINVAL when n_q > 0 and
 * n_k = 0. */
int hyperattn_forward_rect(const void* q, const void* k, const void* v, int dtype, int batch, int n_q, int n_k,
                           int d, int heads, int kv_heads, int block, int samples, int proj_bits, uint64_t seed,
                           void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Squared row norms for the row-norm variant: w[i] = ||x_i||^2 in fp32,
 * each square rounded, groups of 8 consecutive squares summed by halving
 * (pairs 4, 2, 1 apart), the group sums by halving; no multiply-add
 * contraction.  x device [rows, d] (bf16 or fp32, d 64 or 128), w device
 * [rows] fp32, written.  Errors: HA_EINVAL (bad arguments),
 * HA_EUNSUPPORTED (d or dtype). */
int hyperattn_row_sqnorms(const void* x, int dtype, int64_t rows, int d, float* w, void* stream);

/* Draws of the row-norm variant for non-causal problems.
 *   w        device [batch * kv_heads][n] fp32, squared norms of the value
 *            rows (hyperattn_row_sqnorms), row order
 *   perm_k   device [batch * kv_heads][n] i32, the keys' sort permutation
 *            (row within the head for each sorted position)
 *   cum      device [batch * kv_heads][n] int64, written: with max w =
 *            f 2^e (f in [0.5, 1)) and n_t = floor(w[perm_k[t]] 2^(40 - e)),
 *            cum[t] = n_0 + ... + n_t (exact integers)
 *   sidx     device [batch * heads][samples] i32, written: draw i of query
 *            head h of batch entry b takes word i % 4 of Philox4x32-10 under
 *            the seed with counter (i / 4, 1, h, 2 b + 2), r = floor(word T
 *            / 2^32) with T = cum[n - 1] of the head's KV head, and is the
 *            smallest sorted position t with cum[t] > r (0 when T = 0)
 *   workspace device scratch of at least
 *            hyperattn_rownorm_samples_workspace_bytes(batch, kv_heads, n)
 *            bytes, owned by the caller, contents undefined afterwards
 * Errors: HA_EINVAL (bad arguments), HA_EWORKSPACE (workspace missing or
 * too small). */
size_t hyperattn_rownorm_samples_workspace_bytes(int batch, int kv_heads, int n);
int hyperattn_rownorm_samples(const float* w, const int32_t* perm_k, int batch, int heads, int kv_heads,
                              int n, int samples, uint64_t seed, int64_t* cum, int32_t* sidx,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics: the method's fine-grained parameters ("HyperAttention:
 * Long-context Attention in Near-Linear Time", research-map summary,
 * sections Approach and Limitations -- alpha, the largest squared column
 * norm of the softmax matrix D^-1 A, and the ratio of row norms of A after
 * the large entries are removed; section Surprising findings -- alpha taken
 * without the first 32 columns for chatglm2).
 * ------------------------------------------------------------------------ */

/* Squared column mass of the exact softmax matrix and alpha.
 *   q, k       device bf16, [batch, heads, n, d] and [batch, kv_heads, n, d]
 *   lse        device [batch, heads, n] fp32, the exact attention's natural
 *              log row sums (hyperattn_forward with block >= n, or causal
 *              with min_seq_len >= n)
 *   colmass    device [batch, heads, n] fp32, written: c_j = sum_i
 *              exp(2 (q_i . k_j - lse_i)) (causal: over i >= j)
 *   alpha      device [batch, heads] fp32 or NULL, written: max over
 *              columns j >= skip of c_j (-inf if skip >= n)
 * Errors: HA_EINVAL (bad arguments), HA_EUNSUPPORTED (not bf16, d not 64
 * or 128). */
int hyperattn_column_sqmass(const void* q, const void* k, const float* lse, int dtype, int batch, int n, int d,
                            int heads, int kv_heads, int causal, int skip, float* colmass, float* alpha,
                            void* stream);

/* Ratio of the largest to the smallest residual row sum, r_i = sum of A_ij
 * over the keys outside row i's sortLSH block = exp(lse_exact_i) (1 -
 * exp(lse_block_i - lse_exact_i)), per problem (fp64 inside).
 *   lse_exact  device [problems, n] fp32, exact lse, row order
 *   lse_block  device [problems, n] fp32, the block part's lse at sorted
 *              positions (hyperattn_attend with parts = 1)
 *   perm_q     device [problems, n] i32, the queries' sort permutation
 *   kappa      device [problems] fp32, written (+inf if some r_i is 0)
 * Errors: HA_EINVAL. */
int hyperattn_residual_ratio(const float* lse_exact, const float* lse_block, const int32_t* perm_q,
                             int64_t problems, int n, float* kappa, void* stream);

/* ------------------------------------------------------------------------
 * Backward ("HyperAttention: Long-context Attention in Near-Linear Time",
 * research-map summary, section Key results: the method is timed forward
 * and backward; the pages print no backward formulas).  For the ranks and
 * samples the forward draws (recomputed here from the same seed) the
 * forward is a softmax with fixed key multiplicities W -- 1 inside the
 * query's block of the sorted matrix, seg / samples per kept sample, and for
 * causal calls the exact leaves' lower triangles plus every level's quadrant
 * weights (the log-sum-exp merge of the parts is the joint softmax) -- so
 * with P = W * exp(Q K^T - lse), D = rowsum(dout * out) and
 * dS = P * (dout V^T - D) the gradients are dQ = dS K, dK = dS^T Q,
 * dV = P^T dout (dK, dV of a KV head summed over its query heads).
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace hyperattn_backward needs (0 for invalid
 * shapes).  Arguments as hyperattn_workspace_bytes. */
size_t hyperattn_backward_workspace_bytes(int batch, int n, int d, int heads, int kv_heads,
                                          int block, int samples, int proj_bits, int causal,
                                          int min_seq_len, int dtype);

/*
 * Gradients of sum(dout * out) for out = hyperattn_forward(q, k, v, ...)
 * with the same shape and method arguments and seed.
 *   q, k, v    device, as for hyperattn_forward (bf16 or fp32)
 *   out, lse   device, the forward's outputs (out [B, H, n, d] of dtype,
 *              lse [B, H, n] fp32 natural log)
 *   dout       device [B, H, n, d] of dtype, upstream gradient of out
 *   dq         device [B, H, n, d] fp32, written (every element)
 *   dk, dv     device [B, Hkv, n, d] fp32, written (every element)
 *   workspace  device, >= hyperattn_backward_workspace_bytes(...) bytes,
 *              256-byte aligned, owned by the caller, clobbered
 *   stream     hipStream_t or NULL; asynchronous on it
 * Results are bitwise deterministic: the sampled keys' contributions to dK
 * and dV are summed in a fixed order (per KV head and problem, sorted by key
 * position, query head and draw), one writer per key row.  For that sort,
 * (heads / kv_heads) * samples must not exceed 8192 (else HA_EUNSUPPORTED).
 * Causal calls run the exact leaves first (dq, dk, dv stored), then every
 * level's quadrant problems (added); when some span splits unevenly, node
 * by node with rectangular quadrants (n_q = n_k + 1), as the forward.
 * bf16 inputs run the MFMA kernels; fp32 inputs run fp32 vector kernels
 * (one wave per query row, key and sample slot; for small problems).
 * Errors: as hyperattn_forward.
 */
int hyperattn_backward(const void* q, const void* k, const void* v, const void* out,
                       const float* lse, const void* dout, int dtype,
                       int batch, int n, int d, int heads, int kv_heads,
                       int block, int samples, int proj_bits, int causal, int min_seq_len,
                       uint64_t seed, float* dq, float* dk, float* dv,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Backward of the rectangular forward (hyperattn_forward_rect): q, out,
 * dout [batch, heads, n_q, d], k, v [batch, kv_heads, n_k, d] (bf16 or fp32),
 * lse [batch, heads, n_q]; dq [batch, heads, n_q, d], dk, dv [batch,
 * kv_heads, n_k, d] fp32, written (every element).  The same weighted
 * softmax backward over the rectangular problem's weights (query blocks of
 * b_eff = min(block, n_q) paired with key blocks of ceil(b_eff n_k / n_q),
 * samples over the n_k keys with weight n_k / samples).
 * Errors: as hyperattn_forward_rect. */
size_t hyperattn_backward_rect_workspace_bytes(int batch, int n_q, int n_k, int d, int heads, int kv_heads,
                                               int block, int samples, int proj_bits, int dtype);
int hyperattn_backward_rect(const void* q, const void* k, const void* v, const void* out, const float* lse,
                            const void* dout, int dtype, int batch, int n_q, int n_k, int d, int heads,
                            int kv_heads, int block, int samples, int proj_bits, uint64_t seed, float* dq,
                            float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Stages of the forward, exported for parity checks and timing.  The
 * forward calls the same kernels.
 * ------------------------------------------------------------------------ */

/*
 * Projection matrix R of the sortLSH hash ([S] Approach, "Hamming-sorted
 * LSH"; [A] Abstract, LSH finds the large entries): float32 [proj_bits][d],
 * Gaussian by Box-Muller from Philox4x32-10 words (counter (e/4, 0, 0, 0)
 * for element e = p*d + col, key = seed).
 *   _host: host_out is host memory of proj_bits*d floats, computed on the
 *          host with the same arithmetic as the device kernel.
 *   plain: dev_out is device memory; enqueued on stream.
 * Errors: HA_EINVAL for null output, d < 1, proj_bits outside [1, 16].
 */
int hyperattn_projections_host(uint64_t seed, int d, int proj_bits, float* host_out);
int hyperattn_projections(uint64_t seed, int d, int proj_bits, float* dev_out, void* stream);

/*
 * Bucket rank of each row of x ([S] Approach, Hamming-sorted LSH):
 * bit p of the code is 1 iff the exact real dot product <x_row, R_p> is
 * positive (no rounding: an exact zero gives 0, and a row or projection
 * holding a NaN or an infinity gives 0); rank = position of the code in
 * the reflected-binary Gray sequence.
 *   x         device, [rows, d] of dtype (d in {64, 128})
 *   proj_dev  device, float32 [proj_bits, d] (from hyperattn_projections)
 *   rank_out  device, uint16 [rows]
 * Errors: HA_EINVAL (null pointers, rows < 0, bad dtype, proj_bits outside
 * [1, 16]); HA_EUNSUPPORTED (d not in {64, 128}).
 */
int hyperattn_hash(const void* x, int dtype, int64_t rows, int d, int proj_bits,
                   const float* proj_dev, uint16_t* rank_out, void* stream);

/*
 * Stable segmented sort of bucket ranks ([S] Approach: rows are sorted by
 * bucket; ties keep their original order).  The ranks are uint16
 * [heads, n]; segment i of head hd covers rows
 * first + i*stride ... first + i*stride + len - 1 of that head, for
 * i < pieces.  perm_out (device, int32 [heads, pieces, len]) receives, for
 * each sorted position, the row index (within the head, 0..n-1) of the
 * element that lands there.  proj_bits <= 8 takes one counting pass,
 * 9..16 two.  Workspace: hyperattn_sort_workspace_bytes(...) bytes.
 * Errors: HA_EINVAL (null pointers, negative sizes, segments outside
 * [0, n)), HA_EWORKSPACE.
 */
size_t hyperattn_sort_workspace_bytes(int64_t heads, int len, int pieces, int proj_bits);
int hyperattn_sort(const uint16_t* rank, int64_t heads, int n, int len, int first,
                   int stride, int pieces, int proj_bits, int32_t* perm_out,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Uniform sample positions ([S] Approach: uniform column sampling):
 * for batch b < batch, query head h < heads and node
 * node_first + j (j < node_count), `samples` positions in [0, ns):
 * word i of Philox counters (i/4, node, h, 2b+1) under seed, mapped to
 * floor(word * ns / 2^32).  idx_out: device int32
 * [batch, heads, node_count, samples].
 * Errors: HA_EINVAL (null output with samples > 0, negative sizes, ns < 1).
 */
int hyperattn_sample_indices(uint64_t seed, int batch, int heads, int node_first,
                             int node_count, int ns, int samples, int32_t* idx_out,
                             void* stream);

/*
 * Permutation gather: dst[hd, j, :] = src[hd, perm[hd*rows_per_head + j], :]
 * for hd < heads, j < rows_per_head; src [heads, n, d], dst
 * [heads, rows_per_head, d], both device, of dtype.  (Sorted copies of
 * Q, K, V, [S] Approach.)  Errors: HA_EINVAL.
 */
int hyperattn_gather(const void* src, int dtype, int64_t heads, int n, int d,
                     const int32_t* perm, int rows_per_head, void* dst, void* stream);

/*
 * One part of a non-causal problem per (batch, head), in sorted order
 * ([S] Approach: exact masked row sums over the diagonal blocks; the
 * uniform column samples for the rest).
 *   parts = 1: block part -- sorted query p attends the sorted keys of its
 *              block, positions [t b', (t+1) b'), t = p / b', b' = min(block, n);
 *   parts = 2: sampled part -- the sorted keys at idx (device int32
 *              [batch, heads, samples]) except those in the row's block,
 *              each with weight n / samples;
 *   parts = 3: both in one softmax (the forward's fused kernel).
 *   perm_q device int32 [batch*heads, n], perm_k [batch*kv_heads, n]:
 *          sorted position -> original row (from hyperattn_sort).
 *   o_out  device float32 [batch, heads, n, d], lse_out float32
 *          [batch, heads, n]: normalised output and natural-log mass of
 *          that part at each *sorted* position (lse = -inf, o = 0 when no
 *          key is left).
 * Errors: as hyperattn_forward for the shared arguments; HA_EINVAL for
 * parts outside 1..3.
 */
int hyperattn_attend(const void* q, const void* k, const void* v, int dtype,
                     int batch, int n, int d, int heads, int kv_heads,
                     int block, int samples, const int32_t* perm_q, const int32_t* perm_k,
                     const int32_t* idx, int parts, float* o_out, float* lse_out,
                     void* stream);

/*
 * Log-sum-exp merge of two parts and unsort: for each head and sorted
 * position p, lse = ln(e^lse1 + e^lse2), o = o1 e^(lse1-lse) + o2 e^(lse2-lse),
 * written to row perm_q[hd*n + p] of out (dtype, [heads, n, d]) and of
 * lse_out (float32 [heads, n], may be NULL).  Inputs float32 [heads, n, d]
 * and [heads, n], all device.  Errors: HA_EINVAL.
 */
int hyperattn_merge_unsort(const float* o1, const float* lse1, const float* o2,
                           const float* lse2, const int32_t* perm_q, int64_t heads,
                           int n, int d, int dtype, void* out, float* lse_out,
                           void* stream);

/*
 * Exact causal attention inside consecutive leaves of leaf_len rows (the
 * recursion's fallback below min_seq_len): row i of leaf [a, a+leaf_len)
 * attends keys a..i.  o_out float32 [batch, heads, n, d], lse_out float32
 * [batch, heads, n], device.  Errors: HA_EINVAL; HA_ESHAPE when n is not a
 * multiple of leaf_len.
 */
int hyperattn_causal_leaves(const void* q, const void* k, const void* v, int dtype,
                            int batch, int n, int d, int heads, int kv_heads,
                            int leaf_len, float* o_out, float* lse_out, void* stream);

/* ------------------------------------------------------------------------
 * Timing hooks (used by the benchmark): when enabled, the library records
 * a pair of HIP events around each kernel launch on its stream and sums
 * the elapsed times per kernel class on the next hyperattn_timing_read.
 * ------------------------------------------------------------------------ */
enum {
  HA_K_PROJ = 0, HA_K_HASH, HA_K_SORT, HA_K_SAMPLES, HA_K_GATHER,
  HA_K_ATTEND, HA_K_MERGE, HA_K_LEAF, HA_K_QUADRANT, HA_K_BWD_DQ, HA_K_BWD_DKV,
  HA_K_COUNT
};
/* Enable (1) or disable (0) event timing; clears the accumulators. */
int hyperattn_timing_enable(int enable);
/* Synchronises the recorded events, then fills ms[HA_K_COUNT] (total
 * milliseconds per kernel class) and launches[HA_K_COUNT] (launch counts)
 * since the last enable, and clears them.  Either pointer may be NULL. */
int hyperattn_timing_read(double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* HYPERATTN_H */
