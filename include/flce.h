/*
 * flce.h -- C ABI of the MI355X (gfx950) fused linear + cross-entropy library.
 *
 * What is computed.  For hidden states X [BT, H], an output-projection weight
 * W [V, H] (the nn.Linear(H, V).weight layout, no bias) and integer targets
 * y [BT]:
 *
 *     Z = X W^T,  lse_i = ln sum_v exp(Z_iv),  l_i = lse_i - Z_{i, y_i},
 *     N = #{i : y_i != ignore_index},  loss = sum_{valid i} l_i / N,
 *     G_iv = (exp(Z_iv - lse_i) - [v == y_i]) / N   (0 on ignored rows),
 *     dX = G W,  dW = G^T X.
 *
 * This is the fused Linear+CrossEntropy (FLCE) loss of "[論文レビュー] Liger
 * Kernel: Efficient Triton Kernels for LLM Training" (nubint.ai), section
 * 提案手法: the tokens are taken in chunks so that the BT x V logits are never
 * held whole; within a chunk the softmax statistics come from an online
 * max / sum-of-exponentials and the logits are overwritten by their gradient
 * (section 主な発見).  "Liger-Kernel 項目詳細介紹" (aibars.net), section
 * 技術實現, states that the computation is exact; section 使用方法, item 3,
 * fixes the call shape: loss_fn(weight, input, target), weight first.  The
 * softmax cross-entropy formulas themselves are the textbook definition.
 *
 * Readings of what the pages leave open: the reduction is the mean over the
 * non-ignored tokens of the whole call; N = 0 gives loss 0 and zero
 * gradients; a non-ignored target outside [0, V) is an error.
 *
 * Conventions for every entry point.
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing.  Row-major, densely packed.
 *   - Process-global state: a per-device "is this a gfx950" answer (filled
 *     on first use, safe to fill from several threads), and the optional
 *     kernel-timing switch of flce_profile_begin / flce_profile_end (not
 *     thread-safe; while it is on, every launch from any thread records
 *     events into one shared table).  Nothing else persists between calls.
 *   - Sizes (tokens, hidden size, vocabulary) must be below 2^31; larger
 *     ones return FLCE_ERR_ARG (queries return 0).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Results are valid once the stream has been synchronised.
 *   - Problems detectable on the host are reported by the return value
 *     before anything is launched or written.  A non-ignored target outside
 *     [0, V) is detected on the device: *err_flag is set to FLCE_ERR_TARGET
 *     (and to 0 otherwise) and the numeric outputs are then unspecified.
 *   - Two calls may run concurrently only with distinct workspaces and
 *     outputs.  Inputs are never written (except `logits` in the in-place call).
 */
#ifndef FLCE_H
#define FLCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of X, W (and dX).  Accumulation is always fp32. */
enum flce_dtype { FLCE_F32 = 0, FLCE_BF16 = 1 };

/* Status codes. */
enum flce_status {
  FLCE_OK = 0,
  FLCE_ERR_ARG = 1,       /* null pointer, negative, zero or >= 2^31 size */
  FLCE_ERR_DTYPE = 2,     /* dtype not one of flce_dtype */
  FLCE_ERR_WORKSPACE = 3, /* workspace_bytes below what *_workspace_bytes returns */
  FLCE_ERR_DEVICE = 4,    /* current device is not gfx950 */
  FLCE_ERR_LAUNCH = 5,    /* a kernel launch failed */
  FLCE_ERR_TARGET = 6,    /* (device-side, via *err_flag) target out of range */
  FLCE_ERR_SHAPE = 7,     /* H not a multiple of 8 (bf16) or 4 (fp32), or a 256-row tile too large (below) */
  FLCE_ERR_ALIGN = 8,     /* X, W, dX or dW not 16-byte aligned, workspace not 256, targets not 8 */
  FLCE_ERR_SCRATCH = 9    /* more rows than ce_fwd_bwd_inplace_noalloc's static scratch holds */
};

/* Tokens per chunk that flce_fwd_bwd will use: chunk_tokens if positive
 * (capped at BT); otherwise the fewest chunks whose logits buffer
 * (chunk x round_up(V, 256) elements of the dtype) fits in 1 GiB, made equal
 * and rounded up to a multiple of 256 tokens (never above the 1 GiB bound),
 * capped at BT.  Returns 0 for invalid arguments. */
int64_t flce_chunk_tokens(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype);

/* Bytes of device workspace flce_fwd_bwd needs for these sizes: one logits
 * chunk (chunk x round_up(V, 256) elements of the dtype) plus per-token and
 * per-tile statistics (O(chunk x V / 256) floats; for bf16 the region is at
 * least H x round_up(chunk, 64) x 2 bytes, as it also holds the transposed
 * token chunk for the dW product once the statistics are consumed), the
 * chunk's gathered token rows (chunk x H elements, plus 12 bytes per chunk
 * token and 4 per token of the batch) and, when the dX product is split along
 * the vocabulary, fp32 partials bounded by half the chunk or 128 MiB,
 * whichever is larger.
 * This is the whole extra memory of the call.  Returns 0 for invalid args. */
size_t flce_workspace_bytes(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype);

/* Fused linear + cross-entropy, forward and backward, in one call.
 *   X        [BT, H] dtype, 16-byte aligned        (may be NULL if BT == 0)
 *   W        [V, H]  dtype, 16-byte aligned
 *   targets  [BT]    int64, values in [0, V) or ignore_index
 *   token_scale [BT] float or NULL: NULL gives the gradients of the mean
 *            loss (factor 1/N per token); otherwise token i's gradient rows
 *            are (softmax - onehot) * token_scale[i], the gradients of
 *            sum_i token_scale[i] * l_i (reduction "none" or "sum" with an
 *            upstream gradient; ignored tokens stay 0).  The loss output is
 *            the mean either way.  4-byte aligned.
 *   loss     device float scalar: sum of token losses / N (0 when N == 0)
 *   row_loss [BT] float or NULL: per-token loss l_i (0 on ignored tokens)
 *   dX       [BT, H] dtype: d loss / d X, 16-byte aligned (may be NULL if BT == 0)
 *   dW       [V, H]  float: d loss / d W, fp32 (overwritten, not accumulated into),
 *            16-byte aligned (the products store 4 consecutive h per lane)
 *   workspace, workspace_bytes: >= flce_workspace_bytes(...), 256-byte aligned
 *   err_flag device int32: 0, or FLCE_ERR_TARGET after the call completes
 * With token_scale NULL the gradients are for an upstream gradient of 1 on the
 * mean loss; scale them for another.
 * Only the non-ignored tokens go through the products: they are packed, in
 * their order, into chunks of chunk tokens (the last ones fewer, or none),
 * and the ignored tokens' dX rows and losses are written as zeros.  Every
 * result is the same as with all tokens in the products (ignored rows add
 * exact zeros), except the grouping of dW's sum over chunks.
 * Size limits (status FLCE_ERR_SHAPE): the kernels address a 256-row tile with
 * 32-bit byte offsets, so 256 * H * esize, 256 * H * 4 (the fp32 dW),
 * 256 * round_up(V, 256) * esize and, for bf16, 256 * round_up(chunk, 64) * 2
 * must each be below 2^31 (esize 2 for bf16, 4 for fp32: V up to ~4.19 M for
 * bf16, ~2.09 M for fp32; H up to ~2.09 M).  flce_fwd checks only the first;
 * flce_orpo checks all four. */
int flce_fwd_bwd(const void* X, const void* W, const int64_t* targets, const float* token_scale, int64_t BT,
                 int64_t H, int64_t V, int64_t ignore_index, int64_t chunk_tokens, int dtype, float* loss,
                 float* row_loss, void* dX, float* dW, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                 void* stream);

/* Bytes of device workspace flce_fwd needs: per-token and per-tile softmax
 * statistics only (no logits are stored).  chunk_tokens > 0 sets the tokens
 * per pass (capped at BT); otherwise a pass takes as many tokens as keep its
 * statistics (8 bytes per token and 128-wide vocabulary block) within
 * 256 MiB, capped at BT.  Returns 0 for invalid arguments. */
size_t flce_fwd_workspace_bytes(int64_t BT, int64_t H, int64_t V, int64_t chunk_tokens, int dtype);

/* Fused linear + cross-entropy, forward only (evaluation, no gradients): the
 * loss of flce_fwd_bwd from the same logits and softmax statistics, without
 * the in-place gradient and the two backward products; the logits never
 * leave the GEMM epilogue.  loss and row_loss are bitwise equal to those of
 * flce_fwd_bwd on the same inputs.  Arguments as for flce_fwd_bwd, with
 * workspace_bytes >= flce_fwd_workspace_bytes(...). */
int flce_fwd(const void* X, const void* W, const int64_t* targets, int64_t BT, int64_t H, int64_t V,
             int64_t ignore_index, int64_t chunk_tokens, int dtype, float* loss, float* row_loss, void* workspace,
             size_t workspace_bytes, int32_t* err_flag, void* stream);

/* Bytes of device workspace flce_orpo needs: the larger of the forward-only
 * and the forward+backward workspaces for n_seq * seq_len tokens, plus three
 * floats per token and three doubles per sequence.  0 for invalid args. */
size_t flce_orpo_workspace_bytes(int64_t n_seq, int64_t seq_len, int64_t H, int64_t V, int64_t chunk_tokens,
                                 int dtype);

/* Fused-linear ORPO (odds-ratio preference) loss and its gradients.  The
 * pages name the loss (LigerFusedLinearORPOLoss, "Liger-Kernel 項目詳細介紹",
 * 主要功能) and show the call orpo_loss(lm_head.weight, x, target) (使用方法,
 * item 4); the objective is the published ORPO one:
 *   X [n_seq * seq_len, H]: n_seq = 2B sequences, sequence-major; sequences
 *   0..B-1 are the chosen responses, B..2B-1 the rejected ones (pair p =
 *   (p, B + p)); targets [n_seq * seq_len] with ignore_index.
 *   a_s  = mean over the sequence's valid tokens of log softmax(x_i W^T)[y_i]
 *   r_p  = (a_w - a_l) - (log(1 - e^{a_w}) - log(1 - e^{a_l}))
 *   loss = mean cross-entropy over the chosen sequences' valid tokens
 *          + beta / B * sum_p softplus(-r_p)
 * A pair with a sequence without valid tokens adds nothing to the second
 * term.  Runs the forward-only pass (token losses), one small kernel for the
 * sequence terms and the per-token gradient factors, then the fused
 * forward+backward pass with those factors as token_scale.
 *   seq_logp [n_seq] float or NULL: a_s (0 for a sequence without valid tokens)
 *   dX [n_seq * seq_len, H] dtype, dW [V, H] float: d loss / d X, d loss / d W
 * Other arguments as for flce_fwd_bwd; n_seq must be even and >= 2. */
int flce_orpo(const void* X, const void* W, const int64_t* targets, int64_t n_seq, int64_t seq_len, int64_t H,
              int64_t V, int64_t ignore_index, float beta, int64_t chunk_tokens, int dtype, float* loss,
              float* seq_logp, void* dX, float* dW, void* workspace, size_t workspace_bytes, int32_t* err_flag,
              void* stream);

/* Bytes of device workspace ce_fwd_bwd_inplace needs (a counter, and BT
 * floats of per-token loss when row_loss is NULL). */
size_t ce_workspace_bytes(int64_t BT, int64_t V);

/* Logits-only cross-entropy, forward and backward, in place: the CrossEntropy
 * kernel of the same review page (主な発見): online softmax per row, then the
 * fp32 logits [BT, V] are overwritten by d loss / d logits
 * = (softmax - onehot) / N (rows with ignored targets become 0).
 *   logits   [BT, V] float, 4-byte aligned; 1 <= V < 2^31 (status 1 otherwise)
 *   targets, ignore_index, loss, row_loss, err_flag, stream: as above. */
int ce_fwd_bwd_inplace(float* logits, const int64_t* targets, int64_t BT, int64_t V, int64_t ignore_index,
                       float* loss, float* row_loss, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                       void* stream);

/* ce_fwd_bwd_inplace without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  It allocates nothing: its scratch (the valid-token
 * count and, when row_loss is NULL, one float per row) is a static device
 * array of 256 + 4 * ce_noalloc_max_rows() bytes (8 MiB + 256 B) that each
 * GPU holds for the life of the process.  The first call on a device looks
 * up that array's address there (no allocation, no stream work).
 *   BT <= ce_noalloc_max_rows() (2^21); more rows return FLCE_ERR_SCRATCH
 *   before anything is launched.  Other arguments, results and errors as for
 *   ce_fwd_bwd_inplace.
 * All calls on one GPU share its scratch: calls that overlap on that GPU
 * (several streams or host threads at once) race and give undefined results;
 * serialise them.  Nothing needs clearing between calls: every scratch word
 * a call reads is written earlier in the same call. */
int64_t ce_noalloc_max_rows(void);
int ce_fwd_bwd_inplace_noalloc(float* logits, const int64_t* targets, int64_t BT, int64_t V, int64_t ignore_index,
                               float* loss, float* row_loss, int32_t* err_flag, void* stream);

/* Per-kernel timing, for benchmarks and profilers (process-global, not
 * thread-safe, off by default).  flce_profile_begin(max_launches) creates
 * 2 x max_launches HIP events and turns timing on: from then on every kernel
 * the library launches is bracketed by two event records on its own stream
 * (launches beyond max_launches are not timed).  flce_profile_end waits for
 * the recorded events, turns timing off, frees the events and writes, for
 * each kernel kind p < n, the summed duration in ms and the number of timed
 * launches.  Kinds: 0 target count, 1 logits GEMM + softmax statistics,
 * 2 log-sum-exp, 3 in-place logits gradient, 4 dX and dW GEMMs (one launch,
 * with the bf16 chunk transpose before it), 5 dX split sum, 6 final mean,
 * 7 logits-only cross-entropy rows, 8 zero fill, 9 ORPO sequence statistics,
 * 10 token compaction (ignored tokens' rows zeroed, each chunk's rows
 * gathered). */
#define FLCE_NUM_KERNEL_KINDS 11
int flce_profile_begin(int max_launches);
int flce_profile_end(double* total_ms, int64_t* launches, int n);

/* Static English text for a status code. */
const char* flce_status_str(int status);

/* 1 if device `device` (a HIP ordinal) is a gfx950, 0 if not, -1 on error. */
int flce_device_supported(int device);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H */
