/*
 * rkl.h -- C ABI of librkl.so: fused LM-head projection + exact
 * full-vocabulary reverse KL (forward and backward) on one MI355X (gfx950).
 *
 * What is computed (NeMo-RL pull request "add full-vocabulary on-policy
 * distillation to SingleController"):
 *   - summary: per token t, over the whole vocabulary V,
 *         L_t = sum_v p_s(v) (log p_s(v) - log p_t(v)),
 *     p_s = softmax(z_s), p_t = softmax(z_t), natural log, no temperature;
 *   - summary, payload paths: the teacher side arrives either as hidden
 *     states h_t projected through the teacher LM-head weight W_t
 *     (z_t = h_t W_t^T), or as precomputed full-vocabulary logits z_t;
 *   - implementation notes: the shared backward is
 *         dL/dz_s = p_s (w - L),  w = log p_s - log p_t,
 *     with both log-softmaxes recomputed in the backward rather than cached.
 * Loss-mask compaction (slime pull request "compact actor logits before
 * projection", summary): only the N trainable rows of the T = B(S-1)
 * positions are projected, and per-row scalars are scattered back to the
 * [B, S-1] layout with zeros elsewhere; an empty mask still yields a (zero)
 * gradient.
 *
 * Conventions shared by every entry point
 *   - Pointers without a "host" note are device pointers (hipMalloc'd or
 *     torch CUDA tensors) on the current device.  Every buffer is owned by
 *     the caller; the library allocates no device memory (the fixed scratch
 *     array of rkl_noalloc.h aside), keeps no state between calls (the
 *     events of rkl_kernel_timing aside), and may be called from several
 *     host threads.
 *   - bf16 values are passed as raw 16-bit patterns (rkl_bf16).  Matrices are
 *     row-major and densely packed: h [rows, H], W [V, H] (the nn.Linear /
 *     output-layer layout), logits [rows, V].
 *   - Device pointers must be 16-byte aligned.  H (Hs, Ht) must be a multiple
 *     of 64, else RKL_UNSUPPORTED.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = null stream),
 *     except rkl_compact_rows when it returns the count to the host.
 *   - Argument checks run before anything is launched.  On failure the call
 *     returns a nonzero status, launches nothing, and rkl_last_error() (per
 *     host thread) describes the problem.  Launch failures return
 *     RKL_DEVICE_ERROR.  Nothing is thrown or aborted across this ABI.
 *   - Outputs must not alias inputs.  Teacher inputs are read only; no
 *     teacher gradient is produced (the teacher head is a frozen tensor).
 *   - Results are bitwise reproducible for identical inputs and shapes.  A
 *     row's loss, statistics, dz and dh do not depend on N or on the row's
 *     position, so compacted rows and the same rows in full-row mode agree
 *     bit for bit.
 */
#ifndef RKL_H
#define RKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* rkl_stream_t;   /* hipStream_t */
typedef uint16_t rkl_bf16;    /* raw bfloat16 bits */

#define RKL_OK 0
#define RKL_INVALID_ARG 1
#define RKL_UNSUPPORTED 2
#define RKL_WORKSPACE_TOO_SMALL 3
#define RKL_DEVICE_ERROR 4

/* Message for the last nonzero status returned on this host thread. */
const char* rkl_last_error(void);

/* Library version string (static storage). */
const char* rkl_version(void);

/*
 * Per-kernel device time, for measurement (the pages define no such call;
 * it exists so that a benchmark can price each kernel of the path against
 * the chip's peak).  rkl_kernel_timing(1) turns timing on for the calling
 * host thread: from then on every kernel that thread's calls launch carries
 * two hipEvents that the launch stamps with the kernel's own begin and end
 * (hipExtLaunchKernel: no marker packets join the stream; the events come
 * from a per-thread pool and are reused; no device memory).
 * rkl_kernel_timing(0) turns it off.  rkl_kernel_times waits for the
 * recorded events, sums the elapsed time per kernel name and forgets them:
 * entry k < min(*count, cap) gets names[k] (static storage), total_ms[k] and
 * launches[k]; *count receives the number of distinct kernels (may exceed
 * cap).  Host pointers.  Names: fwd_tiles, fwd_combine, bwd_dz_tiles,
 * dw_gemm, dh_gemm, dh_reduce, grad_scale, absmax_bf16, convert_h, w_rescale,
 * compact, gather, scatter, fill_zero, fwd_rows_logits, bwd_rows_logits,
 * group_by_teacher, topk_terms, topk_dz_add.
 */
int rkl_kernel_timing(int enable);
int rkl_kernel_times(int cap, const char** names, double* total_ms, int* launches, int* count);

/*
 * Row compaction (slime page, summary: project only the loss-masked rows).
 *   mask       [T] uint8, nonzero = trainable position (the [B, S-1] layout).
 *   row_idx    [T] int32 capacity; receives the N selected positions in
 *              ascending order (entries past N are left untouched).
 *   n_rows_dev [1] int32 device; receives N.
 *   n_rows_host optional host int64*; when non-NULL the call waits for the
 *              stream and stores N there (the one host synchronisation of
 *              the path).
 * T = 0 is allowed (N = 0).  T must be < 2^31.
 */
int rkl_compact_rows(const uint8_t* mask, int64_t T, int32_t* row_idx, int32_t* n_rows_dev,
                     int64_t* n_rows_host, rkl_stream_t stream);

/*
 * Gather (slime page, summary: the compacted rows are what gets projected):
 * dst[i, :] = src[row_idx[i], :] for i < N, a bit copy of row_bytes
 * bytes per row.  row_bytes must be a positive multiple of 4; every row_idx
 * entry must lie in [0, T) (not checked on the device).  N = 0 is a no-op.
 */
int rkl_gather_rows(const void* src, int64_t T, int64_t row_bytes, const int32_t* row_idx, int64_t N,
                    void* dst, rkl_stream_t stream);

/*
 * Scatter (slime page, summary: scalar results back to the response layout):
 * every one of the T rows of dst is written -- rows named by row_idx get
 * src[i, :], all others literal +0.0 (zero bytes).  Same constraints as
 * gather; row_idx entries must be distinct.
 */
int rkl_scatter_rows(const void* src, int64_t N, int64_t row_bytes, const int32_t* row_idx, int64_t T,
                     void* dst, rkl_stream_t stream);

/*
 * Device workspace (NeMo-RL page, implementation notes: chunked functions
 * that recompute their log-softmaxes in the backward -- the per-chunk
 * buffers live here) in bytes that rkl_forward_* and rkl_backward_* need for
 * N rows, vocabulary V, student width Hs (0 = student given as logits) and
 * teacher width Ht (0 = teacher given as logits).  The log-probability /
 * entropy calls pass their H as Hs and 0 as Ht; the per-row-teacher calls
 * need rkl_workspace_bytes_teachers instead.  Returns 0 on bad sizes.
 * The backward's part dominates: the fp16 dz of one vocabulary chunk
 * (whole 65536-column units, at most 2 GiB unless one unit alone is
 * larger), and, when dh's tiles are too few to fill the GPU (N * Hs below
 * about 2^23), dh's fp32 sums per 16384-column vocabulary segment.
 */
size_t rkl_workspace_bytes(int64_t N, int64_t V, int64_t Hs, int64_t Ht);

/*
 * Workspace (bytes) of rkl_forward_hidden_teachers and
 * rkl_backward_hidden_teachers: rkl_workspace_bytes(N, V, Hs, Ht) plus the
 * rows regrouped by teacher (h_s, h_t, ids, mask, per-row scalars and dh,
 * N (6 Hs + 2 Ht + 29) bytes, each piece 256-byte aligned).  Returns 0 on
 * bad sizes.
 */
size_t rkl_workspace_bytes_teachers(int64_t N, int64_t V, int64_t Hs, int64_t Ht);

/*
 * Forward, hidden-state teacher (NeMo-RL page, summary: hidden_states payload).
 *   h_s [N, Hs], W_s [V, Hs], h_t [N, Ht], W_t [V, Ht]   bf16
 *   row_mask  NULL: all N rows are live (compacted input).
 *             [N] uint8: full-row mode -- rows with 0 get loss 0 and stats 0.
 *   loss      [N] fp32 out: L per row.
 *   stats     [N, 4] fp32 out: (lse_s, lse_t, L, lpmax) per row -- the two
 *             log-sum-exps, the loss and the log of the row's largest student
 *             probability; the only state the backward needs (the
 *             log-softmaxes themselves are recomputed).
 * z_s and z_t are formed tile by tile in fp32 and never written to memory.
 * N = 0 is allowed and launches nothing.
 */
int rkl_forward_hidden(int64_t N, int64_t V, int64_t Hs, int64_t Ht,
                       const rkl_bf16* h_s, const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t,
                       const uint8_t* row_mask, float* loss, float* stats,
                       void* workspace, size_t workspace_bytes, rkl_stream_t stream);

/*
 * Forward, logits teacher (NeMo-RL page, summary: logits payload).
 *   z_t [N, V] fp32 teacher logits.
 *   Student either as hidden states (h_s [N, Hs], W_s [V, Hs] bf16, z_s NULL)
 *   or as fp32 logits (z_s [N, V], h_s = W_s = NULL, Hs = 0).
 *   z_rows, T: NULL, 0 for the above.  Otherwise z_t (and z_s) hold T rows
 *     [T, V] -- e.g. every position of the batch -- and row i of this call
 *     reads row z_rows[i] of them (z_rows [N] int32, device; typically the
 *     row_idx of rkl_compact_rows, which spares the gather of the logits
 *     rows the slime page's compaction would otherwise copy).  1 <= T <=
 *     2^30.  Values are not checked on the device: they are clamped to
 *     [0, T), so a wrong index reads a wrong row, never outside the buffers.
 * Other arguments as rkl_forward_hidden (h_s, row_mask, loss and stats keep
 * their N rows).
 */
int rkl_forward_logits(int64_t N, int64_t V, int64_t Hs,
                       const rkl_bf16* h_s, const rkl_bf16* W_s, const float* z_s, const float* z_t,
                       const int32_t* z_rows, int64_t T, const uint8_t* row_mask, float* loss, float* stats,
                       void* workspace, size_t workspace_bytes, rkl_stream_t stream);

/*
 * Backward, hidden-state teacher (NeMo-RL page, implementation notes:
 * dL/dz_s = p_s (w - L), log-softmaxes recomputed per vocabulary chunk).
 * Inputs as rkl_forward_hidden, plus
 *   grad_loss [N] fp32 upstream gradient g (NULL = all ones); the caller's
 *             token reduction decides it.
 *   stats     [N, 4] from the forward on the same inputs.
 * Outputs (gradient of sum_i g_i L_i with respect to the student):
 *   dh_s  [N, Hs] fp32, overwritten; rows with row_mask 0 are exactly 0.
 *   dW_s  [V, Hs] fp32; overwritten, or added to when accumulate_dW != 0.
 * At most 2^22 rows per call (RKL_UNSUPPORTED beyond; split the batch).
 */
int rkl_backward_hidden(int64_t N, int64_t V, int64_t Hs, int64_t Ht,
                        const rkl_bf16* h_s, const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t,
                        const uint8_t* row_mask, const float* grad_loss, const float* stats,
                        float* dh_s, float* dW_s, int accumulate_dW,
                        void* workspace, size_t workspace_bytes, rkl_stream_t stream);

/*
 * Backward, logits teacher.  Student as hidden states: outputs dh_s, dW_s as
 * in rkl_backward_hidden (dz_s must be NULL).  Student as logits (h_s = W_s
 * = NULL, Hs = 0): output dz_s [N, V] fp32 = g p_s (w - L), rows with
 * row_mask 0 exactly 0 (dh_s, dW_s must be NULL; dz_s has the call's N rows
 * also when z_rows indexes the inputs).  z_rows, T as rkl_forward_logits.
 */
int rkl_backward_logits(int64_t N, int64_t V, int64_t Hs,
                        const rkl_bf16* h_s, const rkl_bf16* W_s, const float* z_s, const float* z_t,
                        const int32_t* z_rows, int64_t T, const uint8_t* row_mask, const float* grad_loss,
                        const float* stats, float* dh_s, float* dW_s, int accumulate_dW, float* dz_s,
                        void* workspace, size_t workspace_bytes, rkl_stream_t stream);

/*
 * One vocabulary shard of the hidden-state path (NeMo-RL page, implementation
 * notes: the reverse-KL autograd functions are tensor-parallel over the
 * vocabulary and the divergence is formed where the vocabulary-parallel group
 * is held).  A rank owns vocabulary rows [v0, v0 + V) of W_s and W_t; it
 * passes pointers to those rows and V = its row count.  Arguments as
 * rkl_forward_hidden, except that nothing is finalised:
 *   partial [5, N] fp32 out: per row, over the shard's columns only,
 *       m_s = max z_s, S_s = sum exp(z_s - m_s), A = sum exp(z_s - m_s)(z_s - z_t),
 *       m_t = max z_t, S_t = sum exp(z_t - m_t)   (planes of N, in that order).
 * These 20 bytes per row are what the ranks exchange (an all-gather into
 * [G, 5, N]); rkl_combine_shards then gives every rank the loss and stats.
 * Workspace: rkl_workspace_bytes(N, V, Hs, Ht) with the shard's V.
 */
int rkl_forward_hidden_shard(int64_t N, int64_t V, int64_t Hs, int64_t Ht, const rkl_bf16* h_s,
                             const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t, float* partial,
                             void* workspace, size_t workspace_bytes, rkl_stream_t stream);

/*
 * The same for the teacher-logits payload: the shard's teacher logits z_t
 * [N, V] fp32 (its V columns, densely packed) and the student as the shard's
 * (h_s, W_s) rows or as its fp32 logits z_s [N, V]; arguments otherwise as
 * rkl_forward_logits.  Workspace: rkl_workspace_bytes(N, V, Hs, 0) (0 when
 * the student is given as logits).  The shard's backward is
 * rkl_backward_logits on the shard with the merged stats.
 */
int rkl_forward_logits_shard(int64_t N, int64_t V, int64_t Hs, const rkl_bf16* h_s, const rkl_bf16* W_s,
                             const float* z_s, const float* z_t, float* partial, void* workspace,
                             size_t workspace_bytes, rkl_stream_t stream);

/*
 * Merge G shards' partials [G, 5, N] (outputs of rkl_forward_hidden_shard or
 * rkl_forward_logits_shard, in shard order) with the log-sum-exp rule --
 * M = max_g m_g, S = sum_g S_g exp(m_g - M), A likewise with the student's
 * factors -- and finalise as rkl_forward_hidden: loss [N], stats [N, 4]
 * (lse_s, lse_t, L, log p_max over the whole vocabulary); rows with
 * row_mask 0 get zeros.  1 <= G <= 2^20.
 * The backward of a shard is rkl_backward_hidden (or rkl_backward_logits) on
 * the shard's rows of W_s and W_t, or its logits columns (V = the shard's
 * count), with these merged stats: it writes the shard's rows of dW_s (or
 * its dz_s columns) and its term of dh_s, which the ranks then sum.
 */
int rkl_combine_shards(int64_t G, int64_t N, const float* partials, const uint8_t* row_mask, float* loss,
                       float* stats, rkl_stream_t stream);

/*
 * Reverse KL with the teacher chosen per row (NeMo-RL page, first-version
 * limits: one teacher checkpoint in that version, with the payload column
 * shaped for a per-row teacher index).  As rkl_forward_hidden, except:
 *   W_t [K, V, Ht] bf16   the K teachers' output-layer weights, back to back.
 *   teacher [N] int32     device; row i is projected through W_t[teacher[i]].
 *                         Ids outside [0, K) are not checked on the device: such
 *                         a row gets teacher logits 0 (nothing is addressed
 *                         with the id).
 *   1 <= K <= 31.
 * Rows of one teacher need not be contiguous.  The call first groups the
 * rows by teacher id (a stable sort, ids outside [0, K) last) and copies
 * their h_s, h_t (and mask bytes) into the workspace in that order, so that
 * a 128-row tile holds one teacher except at group boundaries; a tile that
 * holds several runs one teacher pass per teacher in it.  Loss and stats are
 * written back to the caller's row order.  A row's results do not depend on
 * which rows share its tile, so they are the same bit for bit whatever the
 * order of the rows.
 * Workspace: rkl_workspace_bytes_teachers(N, V, Hs, Ht).
 */
int rkl_forward_hidden_teachers(int64_t N, int64_t V, int64_t Hs, int64_t Ht, int64_t K, const rkl_bf16* h_s,
                                const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t, const int32_t* teacher,
                                const uint8_t* row_mask, float* loss, float* stats, void* workspace,
                                size_t workspace_bytes, rkl_stream_t stream);

/* Backward of rkl_forward_hidden_teachers: arguments as rkl_backward_hidden
 * plus K, W_t [K, V, Ht] and teacher [N] as above.  Rows are grouped by
 * teacher as in the forward (grad_loss and stats are copied in that order,
 * dh_s is written back to the caller's); dW_s sums the rows in the grouped
 * order.  Workspace: rkl_workspace_bytes_teachers(N, V, Hs, Ht). */
int rkl_backward_hidden_teachers(int64_t N, int64_t V, int64_t Hs, int64_t Ht, int64_t K, const rkl_bf16* h_s,
                                 const rkl_bf16* W_s, const rkl_bf16* h_t, const rkl_bf16* W_t,
                                 const int32_t* teacher, const uint8_t* row_mask, const float* grad_loss,
                                 const float* stats, float* dh_s, float* dW_s, int accumulate_dW, void* workspace,
                                 size_t workspace_bytes, rkl_stream_t stream);

/*
 * Log-probability of the sampled token and entropy of one projection (slime
 * page, summary: the log-probability / entropy computation of the compact
 * actor path takes the [N, V] logits of the loss-masked rows and returns
 * per-row scalars; the top-p masks it also builds are not covered).  Per row
 * i, z_i = h_i W^T formed tile by tile in fp32 and never written to memory:
 *     logp[i]    = z_i[y_i] - lse(z_i)
 *     entropy[i] = -sum_v p_i(v) log p_i(v) = lse(z_i) - sum_v p_i(v) z_i[v]
 *   h [N, H], W [V, H]   bf16; H a multiple of 64.
 *   y [N] int32 device   sampled token per row, in [0, V) (not checked on
 *                        the device; a row whose y lies outside gets
 *                        logp of about -1e30).
 *   row_mask             as rkl_forward_hidden (rows with 0: all outputs 0).
 *   logp, entropy [N] fp32 out.
 *   stats [N, 4] fp32 out: (lse, entropy, logp, lpmax) -- all the backward
 *                        needs.
 * Workspace: rkl_workspace_bytes(N, V, H, 0).  N = 0 launches nothing.
 */
int rkl_forward_logprob_entropy(int64_t N, int64_t V, int64_t H, const rkl_bf16* h, const rkl_bf16* W,
                                const int32_t* y, const uint8_t* row_mask, float* logp, float* entropy, float* stats,
                                void* workspace, size_t workspace_bytes, rkl_stream_t stream);

/*
 * Backward of sum_i (g_lp,i logp_i + g_H,i entropy_i) (NeMo-RL page,
 * implementation notes: like the entropy kernel there, the log-softmax is
 * recomputed from h and W instead of cached):
 *     dz_i[v] = g_lp,i (1[v = y_i] - p_i(v)) - g_H,i p_i(v) (log p_i(v) + entropy_i)
 *     dh = dz W (overwritten),  dW = sum_i dz_i^T h_i (overwritten, or added
 *     to when accumulate_dW != 0).
 *   grad_logp [N] fp32 (NULL = all ones), grad_entropy [N] fp32 (NULL = all
 *   zeros); stats from rkl_forward_logprob_entropy on the same inputs.
 * Other arguments, limits and the workspace as rkl_backward_hidden with Ht = 0.
 */
int rkl_backward_logprob_entropy(int64_t N, int64_t V, int64_t H, const rkl_bf16* h, const rkl_bf16* W,
                                 const int32_t* y, const uint8_t* row_mask, const float* grad_logp,
                                 const float* grad_entropy, const float* stats, float* dh, float* dW,
                                 int accumulate_dW, void* workspace, size_t workspace_bytes, rkl_stream_t stream);

/*
 * Top-k estimator of the reverse KL (NeMo-RL page, summary: the full
 * objective is the K = V limit of the top-k estimator -- once the support
 * spans the whole vocabulary its score-function tail term vanishes).  Per
 * row i, a support S_i of K vocabulary ids chosen without looking at the
 * sampled token (e.g. the teacher's top K) and a token y_i sampled from the
 * student; with f = log p_s - log p_t,
 *     L_i = sum_{j in S_i} p_s(j) f(j)  +  [y_i not in S_i] f(y_i),
 * an exact part on the support and a one-sample estimate of the rest, so
 * that over y_i ~ p_s its expectation is the reverse KL (K = V: exactly the
 * reverse KL; K = 0: the sampled token's log-probability gap).  Only the
 * student is projected (hidden states h [N, H], weight W [V, H], bf16); the
 * teacher arrives as log-probabilities on the support and at the token:
 *   y              [N] int32 sampled tokens, in [0, V) (not checked on the
 *                  device).
 *   support        [N, K] int32 ids per row (distinct; ids outside [0, V)
 *                  are skipped).  K in [0, V]; NULL when K = 0.
 *   logpt_support  [N, K] fp32 teacher log-probabilities at those ids.
 *   logpt_y        [N] fp32 teacher log-probability at y (read only for rows
 *                  whose y is not in their support).
 *   row_mask       as rkl_forward_hidden (rows with 0: loss and stats 0).
 *   loss           [N] fp32 out: L_i.
 *   stats          [N, 4] fp32 out: (lse, c, sp, bound) -- the student's
 *                  log-sum-exp, c = sum_{j in S} p_j (f_j + 1) + [y not in S]
 *                  sp, sp = [y not in S] (f_y + 1), and a bound on |dz| / |g|;
 *                  all the backward needs besides the inputs.
 *   logps_support  [N, K] fp32 out, optional (NULL: not written): the
 *                  student's log-probabilities log p_s(j) on the support (0
 *                  for ids outside [0, V) and on rows with row_mask 0).
 *                  Passed to rkl_backward_topk, they spare it the K dot
 *                  products per row; its results are the same bit for bit.
 * The student's logits on the support are K dot products per row; the cost
 * beyond the fused log-sum-exp grows as N K H.
 * Workspace: rkl_workspace_bytes(N, V, H, 0).  N = 0 launches nothing.
 */
int rkl_forward_topk(int64_t N, int64_t V, int64_t H, int64_t K, const rkl_bf16* h, const rkl_bf16* W,
                     const int32_t* y, const int32_t* support, const float* logpt_support, const float* logpt_y,
                     const uint8_t* row_mask, float* loss, float* stats, float* logps_support, void* workspace,
                     size_t workspace_bytes, rkl_stream_t stream);

/*
 * Backward of sum_i g_i L_i for rkl_forward_topk: the exact gradient of the
 * support part and the score-function estimate of the tail's,
 *     dz_i[j] = g_i (-p_j c_i + [j in S_i] p_j (f_j + 1) + [j = y_i] sp_i),
 *     dh = dz W (overwritten),  dW = sum_i dz_i^T h_i (overwritten, or added
 *     to when accumulate_dW != 0).
 *   grad_loss [N] fp32 (NULL = all ones); stats from rkl_forward_topk on the
 *   same inputs; logps_support the forward's optional output on the same
 *   inputs, or NULL (the dot products are formed again).  Other arguments,
 *   limits and the workspace as rkl_backward_logprob_entropy.
 */
int rkl_backward_topk(int64_t N, int64_t V, int64_t H, int64_t K, const rkl_bf16* h, const rkl_bf16* W,
                      const int32_t* y, const int32_t* support, const float* logpt_support, const uint8_t* row_mask,
                      const float* grad_loss, const float* stats, const float* logps_support, float* dh, float* dW,
                      int accumulate_dW, void* workspace, size_t workspace_bytes, rkl_stream_t stream);

/*
 * Log-probability / entropy over one vocabulary shard (NeMo-RL page,
 * implementation notes: the reverse-KL functions sit beside a distributed,
 * vocabulary-parallel entropy function).  A rank owns vocabulary rows
 * [v0, v0 + V) of W and passes those rows with V = its row count, and y in
 * the shard's own coordinates (y - v0; a row whose token lies in another
 * shard passes any value outside [0, V), e.g. -1).  Nothing is finalised:
 *   partial [5, N] fp32 out: per row, over the shard's columns,
 *       m = max z, S = sum exp(z - m), B = sum exp(z - m) z,
 *       z_y (the token's logit, or -1e30 when the token is not in the shard), 0
 *   (planes of N, in that order).
 * Workspace: rkl_workspace_bytes(N, V, H, 0) with the shard's V.
 */
int rkl_forward_logprob_entropy_shard(int64_t N, int64_t V, int64_t H, const rkl_bf16* h, const rkl_bf16* W,
                                      const int32_t* y, float* partial, void* workspace, size_t workspace_bytes,
                                      rkl_stream_t stream);

/*
 * Merge G shards' log-probability / entropy partials [G, 5, N] (in shard
 * order): M = max_g m_g, S = sum_g S_g exp(m_g - M), B likewise, z_y the
 * largest of the shards' (the one shard that holds the token); then
 * finalise as rkl_forward_logprob_entropy: logp [N] = z_y - lse, entropy [N]
 * = lse - B / S, stats [N, 4] (lse, entropy, logp, log p_max); rows with
 * row_mask 0 get zeros.  1 <= G <= 2^20.  The backward of a shard is
 * rkl_backward_logprob_entropy on the shard's rows of W with the shard-local
 * y and these merged stats: the shard's dW rows and its term of dh.
 */
int rkl_combine_shards_logprob_entropy(int64_t G, int64_t N, const float* partials, const uint8_t* row_mask,
                                       float* logp, float* entropy, float* stats, rkl_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RKL_H */
