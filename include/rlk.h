/*
 * rlk.h -- C ABI of the batch-invariant selected-token log-probability library
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  For hidden states h[T][H], an LM-head weight w[V][H]
 * (both bfloat16) and target ids y[T] (int32):
 *     z[t][v]  = sum_k h[t][k] * w[v][k]          logits, fp32 accumulation
 *     lse[t]   = log sum_v exp(z[t][v])           vocabulary log-sum-exp
 *     logp[t]  = z[t][y[t]] - lse[t]              selected-token log-prob
 * Sources: the RL-Kernel blog (princepride.github.io, "RL-Kernel ... LogP"):
 * section 一 names the quantity (the selected token's log-probability that
 * rollout and training must agree on); section 四 puts it in the Linear-LogP
 * reduction class, whose LSE runs over the whole vocabulary, computed as
 * m + log sum exp(x - m) from per-block maxima and exponent sums merged in a
 * fixed order; section 二 ties GEMM drift to how the K dimension is split;
 * sections 六/七 require a GEMM with one workgroup per output tile and the full
 * K in a fixed order (no split-K) and a vocabulary reduction merged in a fixed
 * vocabulary-tile order.  The vLLM blog summary (papercache.org, "Finish RL
 * Training Faster ...", the consistency criteria) requires that a request's
 * result not depend on the batch it shares (batch independence), nor on
 * prefill vs decode (phase consistency).
 *
 * Numerical contract (fixed for RLK_ABI_VERSION):
 *   - Inputs are bfloat16 bit patterns; products are exact in fp32, sums are
 *     fp32, accumulated over k = 0 .. H-1 in chunks of 16 in increasing order,
 *     one workgroup per tile of 256 vocabulary rows x 256 token rows -- the
 *     same tile for every batch size; rows past T are predicated off inside
 *     it -- and no split-K.
 *   - Logits are never rounded to bf16 and never written to memory.
 *   - Per (row, 128-wide vocabulary tile): tile max m_j and
 *     s_j = sum exp(z - m_j) with a reduction tree that depends only on the
 *     tile geometry; tiles are merged per row with a fold whose shape depends
 *     only on ceil(V / 128): lse = M + log(sum_j s_j exp(m_j - M)),
 *     M = max_j m_j.
 *   - A row's logp and lse are bitwise identical whatever the other rows of
 *     the call are, whatever the row's position, the batch size T, the stream,
 *     and across repeated calls.  (Bitwise equality across GPUs of other
 *     models or other library versions is not promised.)
 *   - Target outside [0, V): logp = NaN (lse still written).
 *   - A NaN or +Inf logit in a row: lse = logp = NaN for that row only.
 *     -Inf logits carry probability zero.  All logits -Inf: lse = -Inf,
 *     logp = NaN.  fp32 overflow of a logit, and subnormal bf16 inputs
 *     (which the matrix cores may flush), are outside the contract.
 *   - The LSE covers exactly the V rows of w passed in; pass the real
 *     vocabulary size to leave out padding rows.  No temperature, no masking:
 *     callers drop inactive rows themselves.
 *
 * Memory and execution.
 *   - Every pointer argument of the compute calls is a device pointer on the
 *     current HIP device.  The caller owns every buffer; the library allocates
 *     nothing and keeps no pointer after returning.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and never synchronise.  Results are valid once the caller has
 *     synchronised with that stream.  Device faults surface at that sync.
 *   - Outputs must not alias inputs or the workspace.
 *   - A workspace serves one call at a time: it holds the call's tile
 *     statistics and the counters its GEMM workgroups claim tiles from, so
 *     calls that may run at the same time (on different streams) need
 *     workspaces of their own.  The one exception is vocabulary slices of
 *     rlk_vocab_stats_shard that are narrower than V: they write disjoint
 *     statistics and use no counters.
 *   - Validation runs before any HIP call: on an error status nothing was
 *     launched and nothing was written.
 */
#ifndef RLK_H
#define RLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Version history: 1 the first contract; 2 added the options, backward,
 * RMSNorm and top-k entry points; 3 gave rlk_selected_logp_workspace_bytes
 * the (T, H, V) signature, named the logits stage rlk_debug_logits (rlk_logits
 * stays as an alias), documented the workspace layout (rlk_workspace_layout)
 * and lowered the T and V limits to 2^31 - 4096; 4 added the top-k entry point
 * without stored logits (rlk_topk_logp_direct) and shrank the backward's
 * workspace (the weight is read as stored, with no transposed copy); 5
 * requires grad_weight to be 16-byte aligned and drops dz^T from the
 * backward's workspace (grad_weight reads dz as stored). */
#define RLK_ABI_VERSION 5

/* Status codes returned by every entry point that can fail. */
#define RLK_OK                      0
#define RLK_ERR_NULL_POINTER        1  /* a required pointer is NULL */
#define RLK_ERR_INVALID_SHAPE       2  /* T < 0, H <= 0, V <= 0, ld < H, n < 0 */
#define RLK_ERR_UNSUPPORTED         3  /* H % 64 != 0, or a size above the
                                          limits below */
#define RLK_ERR_MISALIGNED          4  /* pointer or row stride alignment */
#define RLK_ERR_WORKSPACE_TOO_SMALL 5
#define RLK_ERR_HIP                 6  /* a launch failed; rlk_last_hip_error()
                                          has the hipError_t */
#define RLK_ERR_INVALID_VALUE       7  /* an option out of range: inverse
                                          temperature not finite and > 0, or
                                          unknown flag bits */
#define RLK_ERR_SCRATCH_LIMIT       8  /* T and V need more workspace than
                                          rlk_selected_logp_noalloc's static
                                          scratch */

/* Option flags of the _ex entry points. */
#define RLK_LOGITS_BF16 1  /* round every (scaled) logit to bfloat16 */
#define RLK_ENTROPY     2  /* also produce the per-row entropy */

/* Size limits: T <= 2^31 - 4096 rows, V <= 2^31 - 4096, H <= 65536, row
 * strides ld_hidden, ld_weight <= 2^21 elements, and ceil(T/256) *
 * ceil(V/256) at most 2^31 - 8192 workgroup tiles.  Beyond them:
 * RLK_ERR_UNSUPPORTED. */

/* Version of this ABI and of the numerical contract above. */
int rlk_abi_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *rlk_status_string(int status);

/* The hipError_t (as int) behind the calling thread's most recent
 * RLK_ERR_HIP; hipSuccess (0) if there was none. */
int rlk_last_hip_error(void);

/* Width of one vocabulary statistics tile (128 rows of w): the unit whose
 * max and sum of exponentials are merged.  Part of the numerical contract. */
int rlk_vocab_tile(void);

/* Bytes of device workspace rlk_selected_logp needs for T rows, hidden size
 * H and a vocabulary of V (H does not change the size).  Returns 0 when
 * T <= 0, H <= 0 or V <= 0, or a size is above the limits.  The static-size
 * workspace the caller allocates once is what lets the hot path run with no
 * allocation and no host synchronisation (the vLLM blog summary's CUDA Graph
 * requirements).  The layout is given by rlk_workspace_layout. */
size_t rlk_selected_logp_workspace_bytes(int64_t T, int64_t H, int64_t V);

/* Byte offsets of the regions of a workspace for (T, V, flags), for callers
 * that exchange tile statistics between devices that hold different
 * vocabulary shards (the RL-Kernel blog, section 七: every shard computes
 * local statistics, merged in a fixed vocabulary-tile order).  With
 * nST = ceil(V / 128):
 *   *off_m   part_m, fp32 [nST][T]: part_m[j][t] = max of row t's logits in
 *            vocabulary tile j (rows 128 j .. 128 j + 127 of w);
 *   *off_s   part_s, fp32 [nST][T]: sum of exp(z - part_m[j][t]) over tile j;
 *   *off_xt  xt, fp32 [T]: z[t][y[t]], written by the call (or slice) whose
 *            vocabulary range holds y[t]; not written otherwise;
 *   *off_u   part_u, fp32 [nST][T]: sum of exp(z - m_j) (z - m_j) over tile
 *            j; present with RLK_ENTROPY only (without it nothing of the
 *            caller's lies at this offset).
 * The statistics of the tiles [j0, j1) of a slice are the contiguous bytes
 * [j0 T 4, j1 T 4) after off_m and after off_s (and off_u): a shard's part of
 * the workspace is one contiguous piece per region.  Anything past the
 * regions (tile-claim counters) is private to the library.  Any pointer may
 * be NULL.  Returns RLK_ERR_INVALID_SHAPE / RLK_ERR_UNSUPPORTED /
 * RLK_ERR_INVALID_VALUE for sizes or flags rlk_workspace_bytes_ex refuses. */
int rlk_workspace_layout(int64_t T, int64_t V, int flags, size_t *off_m, size_t *off_s,
                         size_t *off_xt, size_t *off_u);

/* Selected-token log-probabilities: the hot path.
 *   hidden    bf16 [T][ld_hidden] row-major, only the first H columns read;
 *             16-byte aligned, ld_hidden >= H and a multiple of 8.
 *   weight    bf16 [V][ld_weight] row-major (the LM head, one row per
 *             vocabulary entry), same alignment rules.
 *   targets   int32 [T], 4-byte aligned.
 *   logp, lse fp32 [T] outputs, 4-byte aligned; every one of the T entries
 *             is overwritten.
 *   T         rows (T == 0: returns RLK_OK, launches nothing).
 *   H         hidden size, a multiple of 64.
 *   V         vocabulary size (rows of weight taken into the LSE).
 *   workspace device scratch of at least
 *             rlk_selected_logp_workspace_bytes(T, H, V) bytes, 16-byte
 *             aligned; its contents on entry do not matter.
 *   stream    hipStream_t or NULL.
 * Three kernels run on `stream`: a reset of the workspace's tile-claim
 * counters, the logit GEMM with the per-tile statistics and target capture
 * fused into its epilogue, then the fixed-order vocabulary merge that writes
 * lse and logp.  Which workgroup computes a tile changes no bit. */
int rlk_selected_logp(const void *hidden, int64_t ld_hidden,
                      const void *weight, int64_t ld_weight,
                      const int32_t *targets, float *logp, float *lse,
                      int64_t T, int64_t H, int64_t V,
                      void *workspace, size_t workspace_bytes, void *stream);

/* The two stages of rlk_selected_logp, for callers that time or overlap
 * them separately (or exchange the tile statistics between devices that
 * hold different vocabulary shards).  Same argument rules as above; the
 * workspace written by rlk_vocab_stats is read by rlk_vocab_merge and must be
 * passed with the same T and V.  rlk_selected_logp is exactly these two
 * calls in sequence on one stream.
 *   rlk_vocab_stats  the logit GEMM with the fused per-(row, 128-wide tile)
 *                    max / sum of exponentials and the target-logit capture
 *                    (RL-Kernel blog, section 七: local statistics per
 *                    vocabulary tile).  Writes only the workspace.
 *   rlk_vocab_merge  the per-row fixed-order fold of the tile statistics and
 *                    the gather (section 四: merging blocks of the LSE in a
 *                    fixed order).  Reads the workspace, writes logp, lse. */
int rlk_vocab_stats(const void *hidden, int64_t ld_hidden, const void *weight,
                    int64_t ld_weight, const int32_t *targets, int64_t T,
                    int64_t H, int64_t V, void *workspace,
                    size_t workspace_bytes, void *stream);
int rlk_vocab_merge(const int32_t *targets, float *logp, float *lse, int64_t T,
                    int64_t V, const void *workspace, size_t workspace_bytes,
                    void *stream);

/* rlk_vocab_stats on one slice of the LM head: rows [v_begin, v_begin +
 * v_count) of the full V-row weight, passed as `weight_shard` (its row 0 is
 * global row v_begin).  The slice's statistics tiles are written at their
 * global positions in a workspace sized for (T, V), and the target logit of
 * every row whose (global) target falls in the slice.  Running the slices of
 * any partition of [0, V) into one workspace and then calling rlk_vocab_merge
 * once gives bitwise the result of the unsliced call, whatever the number of
 * slices: each statistics tile is computed exactly as it is there, and the
 * merge folds the tiles in the same fixed order.  This is the RL-Kernel blog's
 * LogP rule under tensor parallelism (section 七: every shard computes local
 * statistics, merged in a fixed vocabulary-tile order), made independent of
 * the shard count.  Slices written on one stream, or on streams ordered before
 * the merge, may share the workspace: their writes are disjoint.
 *   v_begin  multiple of 256; v_count > 0; v_begin + v_count <= V; a slice
 *            that does not end at V has v_count a multiple of 256
 *            (RLK_ERR_INVALID_SHAPE / RLK_ERR_UNSUPPORTED otherwise).
 *   targets  global ids (out of [0, V): no slice writes the row's target
 *            logit and the merge gives NaN logp).
 * Other arguments and errors as for rlk_vocab_stats. */
int rlk_vocab_stats_shard(const void *hidden, int64_t ld_hidden,
                          const void *weight_shard, int64_t ld_weight,
                          const int32_t *targets, int64_t T, int64_t H, int64_t V,
                          int64_t v_begin, int64_t v_count, void *workspace,
                          size_t workspace_bytes, void *stream);

/* The same path with the contract options (the variants an RL step needs
 * from one pass over the LM head):
 *   inv_temperature  every logit is first multiplied by this fp32 value, once
 *                    (1/tau of sampling at temperature tau: the trainer must
 *                    score softmax(z / tau) if the sampler drew from it).
 *                    Finite and > 0.  1.0f changes no bit.
 *   RLK_LOGITS_BF16  then every logit is rounded to bfloat16 (nearest, ties
 *                    to even) and used as that value, for engines whose
 *                    logits tensor is bf16 (the RL-Kernel blog, sections 二
 *                    and 四, names this fp32 -> bf16 conversion as one point
 *                    where the two sides drift apart; matching it is the
 *                    caller's choice).
 *   RLK_ENTROPY      also write entropy[t] = -sum_v p_v log p_v of softmax(z')
 *                    (NaN where lse is not finite).  It costs one more
 *                    statistic per tile: the workspace grows by a third.
 * lse and logp are those of z' (the transformed logits); the numerical
 * contract above holds for z' unchanged: a row's lse, logp and entropy are
 * bitwise the same whatever the batch.  With inv_temperature == 1.0f and no
 * RLK_LOGITS_BF16, lse and logp are bitwise those of the plain calls (also
 * with RLK_ENTROPY).
 *   entropy  fp32 [T], 4-byte aligned; required with RLK_ENTROPY, else
 *            ignored (may be NULL).
 *   workspace  at least rlk_workspace_bytes_ex(T, V, flags) bytes.
 * rlk_vocab_stats_ex takes the slice arguments of rlk_vocab_stats_shard
 * (v_begin = 0, v_count = V for the whole head); rlk_vocab_merge_ex must get
 * the same flags as the stats call that filled the workspace.  Errors as for
 * the plain calls, plus RLK_ERR_INVALID_VALUE. */
size_t rlk_workspace_bytes_ex(int64_t T, int64_t V, int flags);
int rlk_selected_logp_ex(const void *hidden, int64_t ld_hidden, const void *weight,
                         int64_t ld_weight, const int32_t *targets, float *logp,
                         float *lse, float *entropy, int64_t T, int64_t H, int64_t V,
                         float inv_temperature, int flags, void *workspace,
                         size_t workspace_bytes, void *stream);
int rlk_vocab_stats_ex(const void *hidden, int64_t ld_hidden, const void *weight_shard,
                       int64_t ld_weight, const int32_t *targets, int64_t T, int64_t H,
                       int64_t V, int64_t v_begin, int64_t v_count, float inv_temperature,
                       int flags, void *workspace, size_t workspace_bytes, void *stream);
int rlk_vocab_merge_ex(const int32_t *targets, float *logp, float *lse, float *entropy,
                       int64_t T, int64_t V, int flags, const void *workspace,
                       size_t workspace_bytes, void *stream);

/* Backward of the selected-token log-probability (the training side's
 * gradient; the vLLM blog summary's trainer differentiates the logprob it
 * recomputes, and checks the backward on its own).  For an upstream gradient
 * g[t] = dL/dlogp[t] of L = sum_t g[t] logp[t]:
 *     dz[t][v]          = g[t] inv_tau (1[v == y_t] - exp(inv_tau z[t][v] - lse[t]))
 *     grad_hidden[t][k] = sum_v dz[t][v] w[v][k]
 *     grad_weight[v][k] = sum_t dz[t][v] h[t][k]
 * Rows whose target lies outside [0, V) contribute nothing (dz = 0).
 * Numerical contract:
 *   - z is recomputed by the forward's GEMM main loop (the forward's bits);
 *     lse is the forward's output for the same inv_temperature (plain or _ex
 *     without RLK_LOGITS_BF16; rounded logits are not differentiated).
 *   - dz is formed in fp32 and rounded to bf16 (nearest, ties to even): it is
 *     the bf16 operand of the two gradient GEMMs, each accumulated in fp32
 *     with one workgroup per output tile over the whole contraction in
 *     increasing order (v for grad_hidden, t for grad_weight), no split, no
 *     atomics.
 *   - grad_hidden[t] depends only on row t: bitwise the same whatever the
 *     batch.  grad_weight sums over the rows of the call in order: bitwise
 *     reproducible for the same rows, and unchanged by appending rows whose
 *     dz is zero (g = 0 or ignored targets).
 *   hidden, weight, targets, T, H, V  as for the forward.
 *   lse, grad_logp  fp32 [T], 4-byte aligned.
 *   grad_hidden     fp32 [T][H] (row stride H) or NULL: not computed.
 *   grad_weight     fp32 [V][H] (row stride H), 16-byte aligned, or NULL:
 *                   not computed.  Both NULL: returns RLK_OK, launches
 *                   nothing.  T == 0: grad_weight is set to zero.
 *   inv_temperature finite, > 0 (RLK_ERR_INVALID_VALUE otherwise).
 *   workspace       rlk_selected_logp_backward_workspace_bytes(T, H, V)
 *                   bytes, 16-byte aligned: bf16 dz [T][Vp] and h^T [H][Tp]
 *                   with Vp, Tp = V, T rounded up to 64 (zero padded); about
 *                   2 V T + 2 H T bytes.  (grad_hidden reads the weight as
 *                   stored and grad_weight reads dz as stored, with no
 *                   transposed copy of either.)
 * Extra limit: V and T rounded up to 64 must not exceed 2^21
 * (RLK_ERR_UNSUPPORTED). */
size_t rlk_selected_logp_backward_workspace_bytes(int64_t T, int64_t H, int64_t V);
int rlk_selected_logp_backward(const void *hidden, int64_t ld_hidden, const void *weight,
                               int64_t ld_weight, const int32_t *targets, const float *lse,
                               const float *grad_logp, float *grad_hidden, float *grad_weight,
                               int64_t T, int64_t H, int64_t V, float inv_temperature,
                               void *workspace, size_t workspace_bytes, void *stream);

/* The backward's first stage alone (stage comparison): the bf16 bits of dz
 * as defined above, written to dz[t * ld_dz + v] for t < T, v < V, with
 * columns V .. Vp-1 set to 0.  ld_dz >= V rounded up to 64, a multiple of 8;
 * dz 16-byte aligned. */
int rlk_logp_grad_logits(const void *hidden, int64_t ld_hidden, const void *weight,
                         int64_t ld_weight, const int32_t *targets, const float *lse,
                         const float *grad_logp, void *dz, int64_t ld_dz, int64_t T,
                         int64_t H, int64_t V, float inv_temperature, void *stream);

/* RMSNorm feeding the LM head: the final normalisation whose output is the
 * `hidden` of rlk_selected_logp.  The RL-Kernel blog (section 四) lists RMSNorm
 * among the reductions whose result depends on the order of accumulation
 * over the hidden dimension, and its H100 recipe (section 六) fixes one
 * normalisation semantics.  Per row t:
 *     r    = 1 / sqrt(sum_k x[t][k]^2 / H + eps)        (fp32)
 *     y[k] = bf16( bf16(x[t][k] * r) * gamma[k] )       (nearest, ties to even)
 * The sum of squares runs in an order fixed by H alone (one wave per row:
 * lane l takes the 8-element chunks l, l+64, ..., in element order, then a
 * butterfly over the 64 lanes), so a row's output is bitwise the same
 * whatever the batch.
 *   x      bf16 [T][ld_x], y bf16 [T][ld_y] (may not alias x), gamma bf16 [H];
 *          16-byte aligned, ld_x, ld_y >= H and multiples of 8.
 *   H      a multiple of 8 (RLK_ERR_UNSUPPORTED otherwise).
 *   eps    finite, >= 0 (Qwen3: 1e-6); RLK_ERR_INVALID_VALUE otherwise. */
int rlk_rmsnorm(const void *x, int64_t ld_x, const void *gamma, float eps, void *y,
                int64_t ld_y, int64_t T, int64_t H, void *stream);

/* The logits stage alone, for stage-by-stage comparison (the RL-Kernel blog,
 * section 五: compare intermediate results to find the first divergence).
 * Runs the very same GEMM main loop as rlk_selected_logp and stores the fp32
 * accumulators: logits[t * V + v], row-major [T][V], 4-byte aligned.
 * Argument rules as above, and V <= 2^24 (RLK_ERR_UNSUPPORTED beyond: 32 rows
 * of the output must span less than 2^31 bytes); no workspace.  Test,
 * debugging and top-k use: it writes 4*T*V bytes.  rlk_logits is the same
 * call under its earlier name. */
int rlk_debug_logits(const void *hidden, int64_t ld_hidden, const void *weight,
                     int64_t ld_weight, float *logits, int64_t T, int64_t H,
                     int64_t V, void *stream);
int rlk_logits(const void *hidden, int64_t ld_hidden, const void *weight,
               int64_t ld_weight, float *logits, int64_t T, int64_t H,
               int64_t V, void *stream);

/* Top-k log-probabilities of each row (the per-token logprob outputs an RL
 * step reads next to the selected token's; the vLLM blog summary lists
 * them), from the logits rlk_logits stores and the lse and workspace of the
 * statistics pass with the same options.  Per row: the k largest entries of
 * z' - lse, z' = z * inv_temperature (then rounded to bf16 with
 * RLK_LOGITS_BF16), in decreasing order, ties to the smaller token id; NaN
 * entries are never selected; with fewer than k others the tail holds id -1
 * and -inf.  z' and the subtraction are those of the statistics pass, so
 * the entry of any id is bitwise the selected-token logp of that id.  The
 * workspace's tile maxima limit the search to the tiles whose maximum is at
 * least the k-th largest tile maximum (no other tile can hold a top-k entry).
 *   logits       fp32 [T][ld_logits] (ld_logits >= V), 4-byte aligned.
 *   lse          fp32 [T] from rlk_selected_logp(_ex) with the same options.
 *   workspace    the workspace that call (or rlk_vocab_stats(_ex), with the
 *                same T, V and options) filled; only read.
 *   k            1 .. 64 and <= V (RLK_ERR_INVALID_VALUE otherwise).
 *   flags        as for the _ex calls (RLK_ENTROPY is ignored here).
 *   topk_logp    fp32 [T][k], topk_ids int32 [T][k], 4-byte aligned. */
int rlk_topk_logp(const float *logits, int64_t ld_logits, const float *lse,
                  const void *workspace, size_t workspace_bytes, int64_t T, int64_t V, int k,
                  float inv_temperature, int flags, float *topk_logp, int32_t *topk_ids,
                  void *stream);

/* The same top-k log-probabilities without stored logits: the logits of the
 * candidate tiles only are recomputed from hidden and weight, by the same
 * MFMA instruction over the same operands in the same K order as the logit
 * GEMM, so every output is bitwise that of rlk_topk_logp on the logits
 * rlk_debug_logits stores.  A row's candidate tiles (m* its k-th largest tile
 * maximum): those whose maximum exceeds m*, and the first of those whose
 * maximum equals m* by tile index, k tiles in all; no other tile can hold a
 * top-k entry under the order (value descending, id ascending).  A row whose
 * m* is -inf (fewer than k tiles hold a value above -inf: rows of NaN or
 * infinities) needs all ceil(V / 128) tiles: when that is more than k, the
 * first max_degenerate_rows such rows (in row order) get room in the
 * workspace, and any further one gets id -2 and NaN in all k places.
 *   hidden, weight, T, H, V  as for rlk_selected_logp.
 *   lse, stats_workspace  the lse and workspace of rlk_selected_logp(_ex) or
 *                   rlk_vocab_stats(_ex) with the same T, V and options (the
 *                   tile maxima); only read.
 *   k, flags, inv_temperature, topk_logp, topk_ids  as for rlk_topk_logp.
 *   max_degenerate_rows  >= 0 (RLK_ERR_INVALID_VALUE otherwise).
 *   workspace       rlk_topk_logp_direct_workspace_bytes(T, V, k,
 *                   max_degenerate_rows) bytes, 16-byte aligned: 512 bytes per
 *                   (row, candidate tile) pair, T k + max_degenerate_rows *
 *                   ceil(V / 128) pairs (the second term only when
 *                   ceil(V / 128) > k), plus small tables.  The pair count
 *                   must not exceed 2^30 (RLK_ERR_UNSUPPORTED; the size query
 *                   returns 0).
 * Six launches on the stream (candidates, plan, buckets, tile logits,
 * selection, and a counter reset); no host synchronisation. */
size_t rlk_topk_logp_direct_workspace_bytes(int64_t T, int64_t V, int k,
                                            int64_t max_degenerate_rows);
int rlk_topk_logp_direct(const void *hidden, int64_t ld_hidden, const void *weight,
                         int64_t ld_weight, const float *lse, const void *stats_workspace,
                         size_t stats_workspace_bytes, int64_t T, int64_t H, int64_t V, int k,
                         float inv_temperature, int flags, int64_t max_degenerate_rows,
                         void *workspace, size_t workspace_bytes, float *topk_logp,
                         int32_t *topk_ids, void *stream);

/* Consistency statistics of two fp32 arrays a (the side under test, e.g.
 * training) and b (the reference, e.g. rollout), as the pages measure them:
 * the mismatch count and maximum absolute logp difference (RL-Kernel blog,
 * sections 六/七), and mean / spread of the absolute difference plus the k3
 * estimator r - 1 - log r with r = exp(a - b) (vLLM blog summary, "diff = 0"
 * definition).  One workgroup, fixed reduction order, so the statistics are
 * themselves deterministic.
 *   a, b   fp32 [n] device arrays, 4-byte aligned.  0 <= n <= 2^31 - 1.
 *   stats  fp64 [8] device array, 8-byte aligned, overwritten with:
 *          [0] n
 *          [1] mismatch count: entries whose 32-bit patterns differ
 *          [2] max |a - b| in fp64 (0 where bits are equal, +inf where
 *              exactly one side is NaN)
 *          [3] sum |a - b|      [4] sum |a - b|^2
 *          [5] sum of k3 over entries where both sides are finite
 *          [6] number of such entries        [7] 0 (reserved)
 * No workspace; asynchronous on `stream`. */
int rlk_compare(const float *a, const float *b, int64_t n, double *stats,
                void *stream);

/* Allocation-free variant of rlk_selected_logp, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  The same kernels
 * and the same bits as rlk_selected_logp; its workspace is a static device
 * array of the library, RLK_NOALLOC_SCRATCH_BYTES (64 MiB), of which each GPU
 * the library runs on holds one copy until the process ends.  It calls no
 * allocating routine.
 *   Arguments and errors as for rlk_selected_logp (no workspace), plus
 *   RLK_ERR_SCRATCH_LIMIT when rlk_selected_logp_workspace_bytes(T, H, V)
 *   exceeds RLK_NOALLOC_SCRATCH_BYTES (checked before any HIP call; at
 *   V = 151936 up to about 7000 rows fit).
 *   Every call on a GPU shares that GPU's array: calls that may overlap on one
 *   GPU (several streams or threads) race and must be serialised by the
 *   caller; each call resets the parts it needs (the tile-claim counters by a
 *   kernel), so a call does not depend on what an earlier one left there. */
#define RLK_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int rlk_selected_logp_noalloc(const void *hidden, int64_t ld_hidden, const void *weight,
                              int64_t ld_weight, const int32_t *targets, float *logp,
                              float *lse, int64_t T, int64_t H, int64_t V, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RLK_H */
