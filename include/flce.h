/*
 * flce.h -- C ABI of liblce03.so: fused linear cross-entropy (FLCE),
 * standalone cross-entropy (CE) and vocabulary-shard statistics on AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (sources: the liger-kernel 0.1.1 README, "Kernels"
 * section, for CrossEntropy and FusedLinearCrossEntropy; the torchtune + Liger
 * blog "Peak performance, minimized memory", text under Figure 1, for the
 * chunked FLCE steps; the DeepSpeed vocab-parallel CE pull request, "Changes"
 * and "Real-device validation", for reductions, ignored targets and shards):
 *
 *   z_n      = x_n W^T (+ b)                        logits of row n, [V]
 *   lse_n    = ln sum_v exp(z_n[v])
 *   loss_n   = lse_n - z_n[y_n]   (0 for ignored rows)
 *   none -> [loss_n];  sum -> sum_n loss_n;  mean -> sum_n loss_n / N_valid
 *   dz_n     = s * (softmax(z_n) - onehot(y_n))    s = 1/N_valid (mean), else 1
 *   grad_X   = dZ W,  grad_W = dZ^T X,  grad_bias = sum_n dz_n
 *
 * FLCE never holds the [N, V] logits: it processes `chunk_rows` rows at a
 * time, turning each chunk's logits in place into dlogits.
 *
 * Conventions shared by every entry point
 *   - Array pointers are DEVICE pointers owned by the caller; arrays are dense
 *     and row-major (the last index is contiguous). Base pointers must be
 *     16-byte aligned. The library never allocates or frees device memory:
 *     scratch space is the caller's `workspace`.
 *   - Element type of X, W, bias and logits: FLCE_F32 (float), FLCE_BF16
 *     (bfloat16 bit patterns, uint16) or FLCE_F16 (IEEE half; the DeepSpeed
 *     vocab-parallel CE page tests FP32/FP16/BF16 logits). All of a call's
 *     floating inputs share one type; 16-bit types need H % 8 == 0 and H,
 *     V below 2^22 (32-bit offsets inside a GEMM tile). Chunk
 *     logits and dlogits are stored in that type; losses, statistics and
 *     FLCE gradients are float32. With FLCE_F16 the dlogits inside the FLCE
 *     calls are stored times a power of two and without the reduction's
 *     scale, which the float32 gradient products apply (so a large
 *     vocabulary's probabilities stay in fp16's normal range); the standalone
 *     CE writes its fp16 gradient with the scale applied, as PyTorch does.
 *   - Targets are int32 class ids. A row is ignored iff its target equals
 *     ignore_index. A target that is not ignore_index and lies outside
 *     [0, V) is a device-detected error: the row is treated as ignored (zero
 *     loss and gradient), and flce_check_device_error() reports FLCE_E_TARGET.
 *   - mean with no valid row returns loss 0 and zero gradients.
 *   - For reduction NONE the gradients are those of the sum of row losses.
 *   - Gradient outputs are overwritten, never accumulated into.
 *   - Every call is asynchronous: work is enqueued on `stream` (a hipStream_t;
 *     NULL = the default stream) and the call returns without waiting. The
 *     library keeps no data between calls (only the row-packing and timing
 *     switches below), so concurrent calls on different
 *     streams are safe as long as their workspaces and outputs do not overlap.
 *   - Errors are returned as flce_status; host-detectable errors are returned
 *     before anything is enqueued. No exception crosses the ABI.
 */
#ifndef LCE03_FLCE_H
#define LCE03_FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLCE_OK = 0,
  FLCE_E_INVALID_ARG = 1, /* null pointer, non-positive size, bad enum, shape mismatch */
  FLCE_E_WORKSPACE = 2,   /* workspace null or smaller than the *_workspace_bytes query */
  FLCE_E_UNSUPPORTED = 3, /* misaligned pointer, bf16 with H % 8 != 0, size over limits */
  FLCE_E_TARGET = 4,      /* (device) a target outside [0, V) that is not ignore_index */
  FLCE_E_HIP = 5          /* a HIP runtime call or kernel launch failed */
} flce_status;

typedef enum { FLCE_F32 = 0, FLCE_BF16 = 1, FLCE_F16 = 2 } flce_dtype;

typedef enum {
  FLCE_REDUCTION_NONE = 0,
  FLCE_REDUCTION_SUM = 1,
  FLCE_REDUCTION_MEAN = 2
} flce_reduction;

/* Human-readable text for a status code (static storage, never NULL). */
const char* flce_status_string(int status);

/*
 * Bytes of workspace flce_forward_backward / flce_shard_stats /
 * flce_shard_backward (with V = V_local for the shard calls) need for this
 * problem and chunk size (chunk_rows 0 = the planner's choice). Pure host
 * computation; returns 0 for invalid sizes.
 */
size_t flce_workspace_bytes(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows);

/*
 * The chunk planner's decision (pure host computation): rows per chunk and the
 * number of K-splits used for the grad_X product. Either output may be NULL.
 * Returns FLCE_OK or FLCE_E_INVALID_ARG.
 */
int flce_plan(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows,
              int64_t* chunk_rows_out, int32_t* dx_splits_out);

/*
 * The workspace of flce_forward_backward split into its regions (pure host
 * computation), in bytes, each rounded up to 256: parts[0] the header and the
 * per-row losses, [1] one chunk of logits / dlogits (chunk x round_up(V, 8)
 * elements), [2] the grad_X K-split partials (float32, S x chunk x H for the
 * largest split S used, at least one for 16-bit inputs; with row packing a
 * chunk's gathered hidden states, chunk x H 16-bit elements, and when they
 * fit their transpose too, share it), [3] the packed-row lists (3 x N int32
 * and the pack kernels' block counts; 0 for float32 inputs). The parts sum
 * to flce_workspace_bytes.
 * parts must hold 4 entries. Returns FLCE_OK or FLCE_E_INVALID_ARG.
 */
int flce_workspace_parts(int64_t N, int64_t H, int64_t V, int dtype, int64_t chunk_rows,
                         size_t* parts);

/*
 * Fused linear cross-entropy, forward and backward in one call (the liger
 * README's FusedLinearCrossEntropy; the steps of the torchtune blog, Figure 1).
 *
 *   X        [N, H]  hidden states (the flattened [batch*seq, H])
 *   W        [V, H]  lm_head weight (nn.Linear(H, V).weight layout)
 *   bias     [V] or NULL
 *   targets  [N] int32
 *   loss     [1] float32, or [N] for FLCE_REDUCTION_NONE
 *   grad_X   [N, H] float32 or NULL (NULL skips the grad_X product)
 *   grad_W   [V, H] float32 or NULL (NULL skips the grad_W product)
 *   grad_bias[V] float32 or NULL (must be NULL when bias is NULL)
 *   workspace of at least flce_workspace_bytes(N, H, V, dtype, chunk_rows)
 *   chunk_rows: rows per chunk, 0 = planner's choice; the workspace is one
 *   chunk of logits (chunk_rows x round_up(V, 8) elements of the input
 *   type), the grad_X K-split partials (float32, a multiple of
 *   chunk_rows x H) and O(N) bytes of per-row data (flce_workspace_parts).
 * Results do not depend on chunk_rows except for the rounding order of grad_W
 * and grad_bias; the loss is bitwise independent of it.
 */
int flce_forward_backward(const void* X, const void* W, const void* bias,
                          const int32_t* targets, int64_t N, int64_t H, int64_t V,
                          int dtype, int32_t ignore_index, int reduction,
                          float* loss, float* grad_X, float* grad_W, float* grad_bias,
                          void* workspace, size_t workspace_bytes, int64_t chunk_rows,
                          void* stream);

/*
 * As flce_forward_backward, with the gradients in the input's 16-bit type
 * when grad_dtype equals dtype (FLCE_BF16 or FLCE_F16): grad_X, grad_W and
 * grad_bias then point to arrays of that type. grad_dtype FLCE_F32 gives
 * float32 gradients (flce_forward_backward). The pages test FP16/BF16 logits
 * and gradients (DeepSpeed vocab-parallel CE page, Real-device validation) but
 * fix no accumulation rule; here products are accumulated in float32 within a
 * chunk and rounded to the output type once per chunk: grad_X rows once,
 * grad_W and grad_bias once per chunk they are added to (read, add in float32,
 * round), so their rounding depends on chunk_rows. It halves the gradient
 * outputs' memory (grad_W of a 128k x 4096 head: 1.05 GB instead of 2.1 GB).
 * FLCE_E_INVALID_ARG for any other grad_dtype (float32 inputs take
 * FLCE_F32 only).
 */
int flce_forward_backward_ex(const void* X, const void* W, const void* bias,
                             const int32_t* targets, int64_t N, int64_t H, int64_t V, int dtype,
                             int32_t ignore_index, int reduction, int grad_dtype, float* loss,
                             void* grad_X, void* grad_W, void* grad_bias, void* workspace,
                             size_t workspace_bytes, int64_t chunk_rows, void* stream);

/*
 * Several LM heads over the same hidden states in one call (the Medusa
 * example the liger README points FusedLinearCrossEntropy users to: extra
 * heads predicting tokens further ahead). Head k has its own weight, bias,
 * targets and loss; the hidden-state gradient is the sum over heads:
 *
 *   W        [K, V, H]  the heads' weights, head-major
 *   bias     [K, V] or NULL
 *   targets  [K, N] int32 (head k's targets, e.g. labels shifted by k + 1)
 *   loss     [K] float32 (head k's loss with its own N_valid for MEAN), or
 *            [K, N] for FLCE_REDUCTION_NONE
 *   grad_X   [N, H] float32 or NULL: sum over heads of dZ_k W_k
 *   grad_W   [K, V, H] float32 or NULL;  grad_bias [K, V] float32 or NULL
 *   workspace of at least flce_multihead_workspace_bytes(N, H, V, K, ...)
 * The gradients are those of the sum of the K heads' losses. Heads run one
 * after another through the same chunk buffer, so peak scratch is that of one
 * head.
 */
size_t flce_multihead_workspace_bytes(int64_t N, int64_t H, int64_t V, int64_t K, int dtype,
                                      int64_t chunk_rows);
int flce_multihead_forward_backward(const void* X, const void* W, const void* bias,
                                    const int32_t* targets, int64_t N, int64_t H, int64_t V,
                                    int64_t K, int dtype, int32_t ignore_index, int reduction,
                                    float* loss, float* grad_X, float* grad_W, float* grad_bias,
                                    void* workspace, size_t workspace_bytes, int64_t chunk_rows,
                                    void* stream);

/*
 * As flce_multihead_forward_backward, with the gradients in the input's
 * 16-bit type when grad_dtype equals dtype (rounding as in
 * flce_forward_backward_ex; grad_X is summed over the heads in that type,
 * rounded once per head). FLCE_E_INVALID_ARG for any other grad_dtype than
 * FLCE_F32 or dtype.
 */
int flce_multihead_forward_backward_ex(const void* X, const void* W, const void* bias,
                                       const int32_t* targets, int64_t N, int64_t H, int64_t V,
                                       int64_t K, int dtype, int32_t ignore_index, int reduction,
                                       int grad_dtype, float* loss, void* grad_X, void* grad_W,
                                       void* grad_bias, void* workspace, size_t workspace_bytes,
                                       int64_t chunk_rows, void* stream);

/* Bytes of workspace ce_forward_backward / ce_shard_stats /
 * ce_combine_shard_stats (V = V_global) need. */
size_t ce_workspace_bytes(int64_t N, int64_t V);

/*
 * Cross-entropy over given logits, loss and gradient together (the liger
 * README's CrossEntropy: the gradient may overwrite the input logits).
 *
 *   logits      [N, V] (dtype)
 *   grad_logits [N, V] (same dtype), or == logits (in place), or NULL (loss only)
 *   targets     [N] int32;  loss [1] or [N] (NONE) float32
 * When grad_logits is neither NULL nor logits, logits is not modified.
 * N is limited to 4194303 rows (one launch covers all rows with one
 * workgroup of up to 1024 lanes each): FLCE_E_UNSUPPORTED beyond.
 */
int ce_forward_backward(const void* logits, void* grad_logits, const int32_t* targets,
                        int64_t N, int64_t V, int dtype, int32_t ignore_index,
                        int reduction, float* loss, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * ce_forward_backward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The call's scratch (the 256-byte header
 * and one float per row) lives in a static device array of 16 MiB + 256 bytes
 * that the library holds on each device it runs on until the process ends;
 * the call itself allocates nothing. N is limited to 4194303 rows, as for
 * ce_forward_backward (FLCE_E_UNSUPPORTED beyond, before anything is
 * launched). All calls on one
 * device share that array: calls that overlap on one device (different
 * streams, or threads) race and must be serialised by the caller. Other
 * arguments, outputs and errors as ce_forward_backward; an out-of-range
 * target is treated as ignored, and is not reported (there is no workspace to
 * pass to flce_check_device_error).
 */
int ce_forward_backward_noalloc(const void* logits, void* grad_logits, const int32_t* targets,
                                int64_t N, int64_t V, int dtype, int32_t ignore_index,
                                int reduction, float* loss, void* stream);

/*
 * Statistics of one vocabulary shard (the per-rank part of vocab-parallel CE in
 * the DeepSpeed and Megatron pages), for logits columns covering global ids
 * [vocab_start, vocab_start + V_local) of V_global. For each row n:
 *   row_max[n]          = max over the shard
 *   row_sumexp[n]       = sum over the shard of exp(z - row_max[n])
 *   row_target_logit[n] = z[n, y_n - vocab_start] when y_n is a valid global
 *                         target inside the shard, else 0
 * Combining shards k: M = max m_k, lse = M + ln sum_k s_k exp(m_k - M),
 * z_y = sum_k t_k. No collective is performed. Targets are global ids checked
 * against [0, V_global). N is limited to 4194303 rows (FLCE_E_UNSUPPORTED).
 */
int ce_shard_stats(const void* logits_shard, const int32_t* targets, int64_t N,
                   int64_t V_local, int64_t vocab_start, int64_t V_global, int dtype,
                   int32_t ignore_index, float* row_max, float* row_sumexp,
                   float* row_target_logit, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * Shard statistics of the logits X W_shard^T (+ bias_shard), computed chunk by
 * chunk without holding [N, V_local]; W_shard is [V_local, H]. Workspace:
 * flce_workspace_bytes(N, H, V_local, dtype, chunk_rows).
 */
int flce_shard_stats(const void* X, const void* W_shard, const void* bias_shard,
                     const int32_t* targets, int64_t N, int64_t H, int64_t V_local,
                     int64_t vocab_start, int64_t V_global, int dtype,
                     int32_t ignore_index, float* row_max, float* row_sumexp,
                     float* row_target_logit, void* workspace, size_t workspace_bytes,
                     int64_t chunk_rows, void* stream);

/*
 * Combine the statistics of P vocabulary shards into the global per-row
 * log-sum-exp and the loss (the exchange step of vocab-parallel CE on the
 * DeepSpeed page, done on one device; the collective that gathers the shards'
 * statistics is the caller's). Shards are combined in index order, in float64:
 * M = max_k m_k, lse = M + ln sum_k s_k exp(m_k - M), z_y = sum_k t_k, so the
 * result does not depend on how the statistics were produced.
 *
 *   shard_max, shard_sumexp, shard_target_logit  [P, N] float32, shard-major
 *     (row k holds shard k's ce_shard_stats / flce_shard_stats outputs)
 *   targets   [N] int32 global ids, validity judged against [0, V_global)
 *   row_lse   [N] float32 global lse per row, or NULL
 *   loss      [1] float32 (SUM / MEAN) or [N] (NONE): loss_n = lse_n - z_y
 *             for valid rows, 0 for ignored or bad ones
 *   workspace of at least ce_workspace_bytes(N, V_global)
 * Bad targets are reported by flce_check_device_error on this workspace.
 */
int ce_combine_shard_stats(const float* shard_max, const float* shard_sumexp,
                           const float* shard_target_logit, int64_t P, int64_t N,
                           const int32_t* targets, int64_t V_global, int32_t ignore_index,
                           int reduction, float* row_lse, float* loss, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * The backward of FLCE for one vocabulary shard (the per-rank gradient step of
 * vocab-parallel CE on the DeepSpeed page): with the global row_lse from
 * ce_combine_shard_stats, for each chunk of rows
 *   dZ = c * (exp(X W_shard^T (+ bias_shard) - lse) - onehot)   (shard columns,
 *        one-hot only where the global target falls in the shard; c = 1/N_valid
 *        for MEAN, 1 otherwise; 0 for ignored or bad rows)
 *   grad_X         [N, H] float32 or NULL: this shard's partial dZ W_shard,
 *                  overwritten; the shards' partials sum to grad_X (the
 *                  caller's all-reduce)
 *   grad_W_shard   [V_local, H] float32 or NULL: dZ^T X, overwritten
 *   grad_bias_shard[V_local] float32 or NULL (NULL when bias_shard is NULL)
 * Workspace: flce_workspace_bytes(N, H, V_local, dtype, chunk_rows). Same
 * layout, alignment and error rules as flce_forward_backward.
 */
int flce_shard_backward(const void* X, const void* W_shard, const void* bias_shard,
                        const int32_t* targets, int64_t N, int64_t H, int64_t V_local,
                        int64_t vocab_start, int64_t V_global, int dtype, int32_t ignore_index,
                        int reduction, const float* row_lse, float* grad_X, float* grad_W_shard,
                        float* grad_bias_shard, void* workspace, size_t workspace_bytes,
                        int64_t chunk_rows, void* stream);
/*
 * As flce_shard_backward, with the gradients in the 16-bit input type when
 * grad_dtype equals dtype (the rounding rules of flce_forward_backward_ex:
 * float32 products rounded once per chunk, grad_W_shard and grad_bias_shard
 * read, added in float32 and rounded at every chunk after the first);
 * FLCE_F32 is flce_shard_backward. FLCE_E_INVALID_ARG for another grad_dtype.
 */
int flce_shard_backward_ex(const void* X, const void* W_shard, const void* bias_shard,
                           const int32_t* targets, int64_t N, int64_t H, int64_t V_local,
                           int64_t vocab_start, int64_t V_global, int dtype, int32_t ignore_index,
                           int reduction, const float* row_lse, int grad_dtype, void* grad_X,
                           void* grad_W_shard, void* grad_bias_shard, void* workspace,
                           size_t workspace_bytes, int64_t chunk_rows, void* stream);

/*
 * Fused linear Jensen-Shannon distillation (the knowledge-distillation loss
 * the Megatron integration page lists among Liger's chunked losses): per
 * chunk of rows, student logits X_s W_s^T and frozen-teacher logits
 * X_t W_t^T over the same vocabulary, then per row
 *   JSD = 1/2 KL(P || M) + 1/2 KL(Q || M),  P = softmax(student / T),
 *   Q = softmax(teacher / T),  M = (P + Q) / 2   (no T^2 factor),
 * reduced over the rows whose target is not ignore_index (targets only mask
 * rows; out-of-range ones are reported like FLCE's). Gradients are the
 * student's only.
 *   X_s [N, H_s], W_s [V, H_s]; X_t [N, H_t], W_t [V, H_t]; one dtype
 *   loss [1] or [N] (NONE); grad_X_s [N, H_s], grad_W_s [V, H_s] float32 or NULL
 *   temperature > 0
 *   workspace of at least flce_jsd_workspace_bytes(N, H_s, V, dtype, chunk_rows)
 *   (two chunk buffers: student and teacher logits)
 */
size_t flce_jsd_workspace_bytes(int64_t N, int64_t H_s, int64_t V, int dtype, int64_t chunk_rows);
int flce_jsd_forward_backward(const void* X_s, const void* W_s, const void* X_t, const void* W_t,
                              const int32_t* targets, int64_t N, int64_t H_s, int64_t H_t,
                              int64_t V, int dtype, int32_t ignore_index, int reduction,
                              float temperature, float* loss, float* grad_X_s, float* grad_W_s,
                              void* workspace, size_t workspace_bytes, int64_t chunk_rows,
                              void* stream);
/* As flce_jsd_forward_backward, with the student's gradients in the 16-bit
 * input type when grad_dtype equals dtype (rounding as flce_forward_backward_ex). */
int flce_jsd_forward_backward_ex(const void* X_s, const void* W_s, const void* X_t, const void* W_t,
                                 const int32_t* targets, int64_t N, int64_t H_s, int64_t H_t,
                                 int64_t V, int dtype, int32_t ignore_index, int reduction,
                                 float temperature, int grad_dtype, float* loss, void* grad_X_s,
                                 void* grad_W_s, void* workspace, size_t workspace_bytes,
                                 int64_t chunk_rows, void* stream);

/*
 * Fused linear DPO (the alignment loss the Megatron integration page lists
 * among Liger's chunked losses and the torchtune blog plans a recipe for):
 * X holds 2 * n_pairs sequences of seq_len token rows, the chosen sequences
 * first, then the rejected ones in the same pair order; targets [N] mark the
 * response tokens (ignore_index elsewhere). A sequence's log-probability is
 * the sum of log softmax(x W^T)[target] over its non-ignored rows; with the
 * reference log-probabilities ref_logps [2 * n_pairs] (same order),
 *   d_b = beta ((logp_w - ref_w) - (logp_l - ref_l)),
 *   loss = mean_b softplus(-d_b) = mean_b -log sigmoid(d_b)
 * Two passes over the chunks: the token log-probabilities, then the logits
 * again (skipped when every row fits one chunk) weighted per row by
 * +-beta sigmoid(-d_b) / n_pairs for the gradient products.
 *   loss [1]; pair_loss [n_pairs] or NULL; grad_X [N, H], grad_W [V, H] or NULL
 *   beta > 0; workspace of at least flce_dpo_workspace_bytes(...)
 */
size_t flce_dpo_workspace_bytes(int64_t n_pairs, int64_t seq_len, int64_t H, int64_t V, int dtype,
                                int64_t chunk_rows);
int flce_dpo_forward_backward(const void* X, const void* W, const int32_t* targets, int64_t n_pairs,
                              int64_t seq_len, int64_t H, int64_t V, int dtype,
                              int32_t ignore_index, const float* ref_logps, float beta,
                              float* loss, float* pair_loss, float* grad_X, float* grad_W,
                              void* workspace, size_t workspace_bytes, int64_t chunk_rows,
                              void* stream);
/* As flce_dpo_forward_backward, with grad_X and grad_W in the 16-bit input
 * type when grad_dtype equals dtype (rounding as flce_forward_backward_ex). */
int flce_dpo_forward_backward_ex(const void* X, const void* W, const int32_t* targets,
                                 int64_t n_pairs, int64_t seq_len, int64_t H, int64_t V, int dtype,
                                 int32_t ignore_index, const float* ref_logps, float beta,
                                 int grad_dtype, float* loss, float* pair_loss, void* grad_X,
                                 void* grad_W, void* workspace, size_t workspace_bytes,
                                 int64_t chunk_rows, void* stream);

/*
 * Causal-LM targets from token labels (the DeepSpeed vocab-parallel CE page
 * keeps the label shift of causal language modelling as part of the loss
 * contract, "Changes"): labels [B, S] int32 row-major,
 * targets [B * S] int32 with targets[b*S + s] = labels[b*S + s + 1] for
 * s < S - 1 and ignore_index at each sequence's last position. The result is
 * the `targets` argument of the other calls for X = hidden states [B*S, H].
 * targets must not alias labels. Asynchronous on `stream`.
 */
int flce_shift_labels(const int32_t* labels, int64_t B, int64_t S, int32_t ignore_index,
                      int32_t* targets, void* stream);

/*
 * Waits for `stream`, then reports whether the last call that used this
 * workspace met an out-of-range target: FLCE_OK, FLCE_E_TARGET or FLCE_E_HIP.
 */
int flce_check_device_error(const void* workspace, void* stream);

/*
 * Row packing in the FLCE calls with 16-bit inputs (flce_forward_backward,
 * its _ex variant, each head of the multi-head calls, flce_shard_backward and
 * both passes of flce_dpo_forward_backward, and flce_jsd_forward_backward
 * when chunk_rows x H_t teacher elements fit the student's split-K buffer;
 * not flce_shard_stats, whose statistics cover every row). A row whose
 * target is ignore_index has zero loss and a zero dlogits row (the definition
 * at the top of this header), so it adds nothing to grad_W or grad_bias and
 * its grad_X row is zero. The chunk loop therefore lists the other rows on
 * the device and runs the logits, grad_X and grad_W products and the
 * row kernel over those only; the results land in the original rows, and
 * grad_X rows of ignored rows are zero. The host never reads the count back:
 * every chunk is launched for the largest possible size and its kernels stop
 * at the count, so the calls stay asynchronous. The last chunk, usually
 * part-full, splits the K of its grad_X product in two. The loss is bitwise
 * the same either way, and so are the grad_X rows outside the last chunk;
 * the rest differ only in rounding order (the last chunk's split, and where
 * the chunk boundaries fall in the grad_W and grad_bias sums). On by default; `enable` 0 turns it
 * off (for comparisons). Returns the previous setting. Process-wide, not
 * thread-safe; the workspace size does not depend on it.
 */
int flce_set_row_packing(int enable);

/*
 * Kernel timing for measurement. While enabled, the library brackets each
 * kernel it launches with HIP events on that kernel's stream. flce_timing_read
 * waits for the recorded events, returns for kernel class `kind` (0 logits
 * GEMM, 1 row CE, 2 grad_X GEMM, 3 grad_W GEMM, 4 other) the summed duration
 * in milliseconds and the number of launches since the last reset, and
 * flce_timing_reset clears the tallies. Not thread-safe; off by default.
 */
int flce_timing_enable(int enable);
int flce_timing_read(int kind, double* total_ms, int64_t* launches);
int flce_timing_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* LCE03_FLCE_H */
