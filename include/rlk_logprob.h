/*
 * rlk_logprob.h -- strict selected-token log-probability and per-token entropy on
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  For every row r of logits x (given directly, or as the
 * LM-head projection x = H W^T of a bf16 hidden state) and a temperature tau:
 *
 *     logprob[r] = x_t/tau - log sum_i exp(x_i/tau)           (t = target_ids[r])
 *     entropy[r] = - sum_i p_i log p_i,  p_i = softmax(x/tau)_i  (natural log, 0 log 0 = 0)
 *
 * over the FULL vocabulary.  This is the "selected logprob" of each response row named
 * by the RL-Kernel issue #342 runbook "Strict R/R trace and operator ablation runbook"
 * (section 2: per-row selected-logprob comparison between training and rollout), the
 * per-token entropy behind the RL-Kernel h100-pcp.json page's train/entropy_loss, and
 * the "linear_logp" operator (LM-head projection fused with the logprob) whose backend
 * id "rlkernel.linear_logp.bitwise.v1" appears in that page's runtime readbacks.
 *
 * Strictness contract (the checks of the RL-Kernel Qwen3-Next logprob prior-art report:
 * tp4_equals_tp1, batch_bitwise, distinct_results_in_repeats):
 *   - results are bitwise identical whatever the number of rows, their order, which
 *     other rows share the call, the repeat, and the vocab split count (1, 2, 4 or 8
 *     contiguous vocabulary shards, each reduced on its own as a vocab-parallel rank
 *     would, then merged in one fixed tree);
 *   - there are no atomics and no data-dependent reduction order;
 *   - there is no fallback path: an unsupported case returns an error.
 *
 * Conventions for every call:
 *   - all tensor pointers are DEVICE pointers owned by the caller, row-major;
 *     inputs are never modified; outputs are fp32;
 *   - every call is asynchronous on `stream` (a hipStream_t passed as void*, NULL =
 *     the default stream); it never allocates, never synchronizes and never reads
 *     device memory on the host; results are valid once the stream has reached the
 *     point of the call; a call only launches kernels (workspace clearing included),
 *     so it can be captured into a HIP graph and replayed;
 *   - arguments are validated on the host before anything is launched; on error
 *     nothing is launched and no output is written;
 *   - n_tokens == 0 returns RLK_OK and launches nothing (two exceptions, which still
 *     write their defined result: rlk_logprob_compare and rlk_linear_logprob_backward);
 *   - a target id outside [0, vocab) gives a NaN logprob for that row (its entropy is
 *     still computed); a NaN or +inf logit anywhere in a row, or a row whose logits are
 *     all -inf, gives NaN for both outputs of that row; -inf logits are tokens of
 *     probability zero;
 *   - the current HIP device must be a gfx950 GPU, otherwise
 *     RLK_ERR_UNSUPPORTED_DEVICE; `stream` and every pointer belong to that device (the
 *     launch shapes, such as one workgroup per compute unit for the persistent tile
 *     kernel, are taken from it);
 *   - calls on different streams may run concurrently if they use distinct workspaces.
 */
#ifndef RLK_LOGPROB_H
#define RLK_LOGPROB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RLK_OK = 0,
  RLK_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad size, bad stride, bad temperature,
                                    vocab_splits not in {1,2,4,8}, bad op code           */
  RLK_ERR_UNSUPPORTED_DEVICE = 2,/* no HIP device, or the current device is not gfx950  */
  RLK_ERR_WORKSPACE_TOO_SMALL = 3,/* workspace_bytes below rlk_workspace_bytes()        */
  RLK_ERR_HIP = 4                /* a HIP runtime call or kernel launch failed          */
} rlk_status;

/* Operation codes for rlk_workspace_bytes. */
#define RLK_OP_FROM_LOGITS 0
#define RLK_OP_LINEAR 1
#define RLK_OP_ENTROPY 2
#define RLK_OP_COMPARE 3
#define RLK_OP_BACKWARD_FROM_LOGITS 4
#define RLK_OP_LINEAR_BACKWARD 5

/*
 * A row's reduction state, as the forward calls can save it for the backward calls (the
 * analogue of saving the log-sum-exp): 24 bytes, 8-byte aligned.  Its contents are the
 * canonical state the forward reduced to (a reference logit m within 8 ln(2) temperature of
 * the row's max, and in fp64 s = sum 2^a, u = sum 2^a a with
 * a = log2(e) (x - m) / temperature) plus the target's logit; callers treat it as opaque.
 * It depends on the logits and the temperature, not on vocab_splits.
 */
typedef struct {
  float m;
  float target_logit;
  double s;
  double u;
} rlk_row_state;

/* rlk_workspace_bytes's answer for a request it cannot size (bad op code, negative or
   oversized sizes, vocab_splits not in {1,2,4,8}): no allocation can satisfy it. */
#define RLK_WORKSPACE_INVALID ((size_t)-1)

/*
 * Device workspace, in bytes, that the call `op` needs for these sizes.  Pure host
 * arithmetic (no device access, no allocation).  `hidden` is ignored unless op is
 * RLK_OP_LINEAR or RLK_OP_LINEAR_BACKWARD; for RLK_OP_COMPARE only n_tokens is used.
 * The workspace itself belongs to the caller, must be 256-byte aligned, and its contents
 * on entry do not matter.  Returns RLK_WORKSPACE_INVALID for a request no call accepts.
 * What needs the space: the vocab-split exchange of the RL-Kernel Qwen3-Next logprob
 * prior-art report's tp4_equals_tp1 check (each shard's partial state, merged in a fixed
 * order, S x 24 bytes per row), the fused path's per-tile states (24 bytes per row and
 * 256-column vocabulary tile), and the backward's saved rows and logit gradients.
 */
size_t rlk_workspace_bytes(int op, int64_t n_tokens, int64_t vocab, int64_t hidden,
                           int32_t vocab_splits);

/*
 * Selected-token logprob (and optionally entropy) from precomputed fp32 logits: the
 * "selected logprob" of each response row that the RL-Kernel issue #342 runbook compares
 * between training and rollout (section 2, strict R/R step), scored in the RL-Kernel
 * Qwen3-Next logprob prior-art report against the same shared logits in fp64
 * (reference "shared_logits_fp64"), with the report's tp4_equals_tp1, batch_bitwise and
 * distinct_results_in_repeats properties.
 *   logits        [n_tokens, ld_logits] fp32, first `vocab` columns used, ld_logits >= vocab
 *   target_ids    [n_tokens] int64
 *   temperature   finite, > 0 (the softmax is of logits / temperature; the h100-pcp.json
 *                 evidence page's rollout runs at temperature .7)
 *   vocab_splits  1, 2, 4 or 8: number of contiguous vocabulary shards reduced separately
 *                 and merged (the result bits do not depend on it)
 *   logprob_out   [n_tokens] fp32
 *   entropy_out   [n_tokens] fp32, may be NULL
 *   workspace     rlk_workspace_bytes(RLK_OP_FROM_LOGITS, ...) bytes (may be NULL if 0)
 * Sizes: 1 <= vocab < 2^31, 0 <= n_tokens < 2^31.
 * Errors: RLK_ERR_INVALID_ARGUMENT (null pointer where one is required, sizes, stride,
 * temperature, split count, misaligned workspace), RLK_ERR_WORKSPACE_TOO_SMALL,
 * RLK_ERR_UNSUPPORTED_DEVICE, RLK_ERR_HIP (a launch failed); on error no output is written.
 */
rlk_status rlk_logprob_from_logits(const float* logits, int64_t ld_logits, int64_t n_tokens,
                                   int64_t vocab, const int64_t* target_ids, float temperature,
                                   int32_t vocab_splits, float* logprob_out, float* entropy_out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * rlk_logprob_from_logits that also saves each row's reduction state for the backward
 * calls (the analogue of saving the log-sum-exp for training, whose records on the
 * h100-pcp.json evidence page consume the logprob and the entropy): outputs and their
 * bits are those of rlk_logprob_from_logits.
 *   row_states_out  [n_tokens] rlk_row_state, 8-byte aligned, may be NULL
 * Other arguments, sizes and errors as rlk_logprob_from_logits.
 */
rlk_status rlk_logprob_from_logits_with_states(const float* logits, int64_t ld_logits,
                                               int64_t n_tokens, int64_t vocab,
                                               const int64_t* target_ids, float temperature,
                                               int32_t vocab_splits, float* logprob_out,
                                               float* entropy_out,
                                               rlk_row_state* row_states_out, void* workspace,
                                               size_t workspace_bytes, void* stream);

/*
 * The same two calls on bf16 logits (16-bit patterns, [n_tokens, ld_logits] row-major):
 * each value is widened exactly to fp32 and reduced in the canonical order of the fp32
 * calls, so the outputs are bitwise equal to rlk_logprob_from_logits / rlk_entropy on the
 * widened logits.  Half the HBM bytes per token.  The RL-Kernel runbook's model is BF16
 * (issue #342, "Source and environment"), so LM-head logits can arrive in bf16.
 * Workspace: rlk_workspace_bytes with RLK_OP_FROM_LOGITS / RLK_OP_ENTROPY (same sizes).
 */
rlk_status rlk_logprob_from_logits_bf16(const uint16_t* logits, int64_t ld_logits,
                                        int64_t n_tokens, int64_t vocab,
                                        const int64_t* target_ids, float temperature,
                                        int32_t vocab_splits, float* logprob_out,
                                        float* entropy_out, void* workspace,
                                        size_t workspace_bytes, void* stream);

rlk_status rlk_entropy_bf16(const uint16_t* logits, int64_t ld_logits, int64_t n_tokens,
                            int64_t vocab, float temperature, int32_t vocab_splits,
                            float* entropy_out, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * LM-head projection fused with the selected-token logprob ("linear-logp"): the operator
 * whose backend id "rlkernel.linear_logp.bitwise.v1" the RL-Kernel h100-pcp.json evidence
 * page's runtime readbacks record for both training and rollout, and whose strict symbols
 * the RL-Kernel issue #342 runbook's preflight requires (section 1).
 * logits = hidden * weight^T are formed tile by tile in fp32 (bf16 x bf16 products,
 * fp32 accumulation in a fixed order over the hidden dimension, no split over it) and
 * never written to memory.
 *   hidden_bf16   [n_tokens, ld_hidden] bf16 bits, first hidden_dim columns used
 *   weight_bf16   [vocab, ld_weight] bf16 bits (nn.Linear / lm_head layout)
 *   hidden_dim    a positive multiple of 64, at most 2^20; ld_hidden, ld_weight >=
 *                 hidden_dim, multiples of 8 and at most 2^22; both base pointers
 *                 16-byte aligned; vocab at most 2^26
 *   other arguments as rlk_logprob_from_logits; entropy_out may be NULL (the tiles then
 *                 skip the entropy terms: the logprob bits are the same as with them)
 *   workspace     rlk_workspace_bytes(RLK_OP_LINEAR, n_tokens, vocab, hidden_dim, splits)
 * Errors as rlk_logprob_from_logits.
 */
rlk_status rlk_linear_logprob(const uint16_t* hidden_bf16, int64_t ld_hidden,
                              const uint16_t* weight_bf16, int64_t ld_weight, int64_t n_tokens,
                              int64_t hidden_dim, int64_t vocab, const int64_t* target_ids,
                              float temperature, int32_t vocab_splits, float* logprob_out,
                              float* entropy_out, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * rlk_linear_logprob that also saves each token's reduction state for
 * rlk_linear_logprob_backward (as rlk_logprob_from_logits_with_states does for the logits
 * path); outputs and their bits are those of rlk_linear_logprob.
 *   row_states_out  [n_tokens] rlk_row_state, 8-byte aligned, may be NULL
 */
rlk_status rlk_linear_logprob_with_states(const uint16_t* hidden_bf16, int64_t ld_hidden,
                                          const uint16_t* weight_bf16, int64_t ld_weight,
                                          int64_t n_tokens, int64_t hidden_dim, int64_t vocab,
                                          const int64_t* target_ids, float temperature,
                                          int32_t vocab_splits, float* logprob_out,
                                          float* entropy_out, rlk_row_state* row_states_out,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * rlk_linear_logprob for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It takes no workspace argument and
 * allocates nothing (no hipMalloc, hipFree or allocating library routine): its workspace is
 * one static device array of RLK_NOALLOC_SCRATCH_BYTES, which each GPU the library runs on
 * holds from the first call on it until the process ends.  Same kernels as
 * rlk_linear_logprob, so the outputs are bitwise those of rlk_linear_logprob.
 *   arguments     as rlk_linear_logprob, without workspace and workspace_bytes
 *   limit         rlk_workspace_bytes(RLK_OP_LINEAR, n_tokens, vocab, hidden_dim,
 *                 vocab_splits) <= RLK_NOALLOC_SCRATCH_BYTES, else
 *                 RLK_ERR_WORKSPACE_TOO_SMALL (nothing launched); at vocab 151936 that is
 *                 up to 4659 tokens with vocab_splits 1 (24 bytes per token and 256-column
 *                 vocabulary tile, plus the split exchange)
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU (other streams
 * or threads) race and must be serialised by the caller.  No call needs the array cleared.
 */
#define RLK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

rlk_status rlk_linear_logprob_noalloc(const uint16_t* hidden_bf16, int64_t ld_hidden,
                                      const uint16_t* weight_bf16, int64_t ld_weight,
                                      int64_t n_tokens, int64_t hidden_dim, int64_t vocab,
                                      const int64_t* target_ids, float temperature,
                                      int32_t vocab_splits, float* logprob_out,
                                      float* entropy_out, void* stream);

/*
 * Per-token entropy only (no targets): the per-token Shannon entropy (nats) of the
 * tempered full-vocabulary softmax, the quantity behind the h100-pcp.json evidence page's
 * train/entropy_loss records (the mean over tokens is the caller's).  Bitwise equal to the
 * entropy output of rlk_logprob_from_logits with the same logits, temperature and any
 * split count.  Arguments, workspace (RLK_OP_ENTROPY) and errors as rlk_logprob_from_logits.
 */
rlk_status rlk_entropy(const float* logits, int64_t ld_logits, int64_t n_tokens, int64_t vocab,
                       float temperature, int32_t vocab_splits, float* entropy_out,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of the logits path: the gradient of  sum_r g_lp[r] logprob[r] + g_ent[r] entropy[r]
 * with respect to the fp32 logits, for the logprob and entropy rlk_logprob_from_logits
 * computes.  Training consumes both (the RL-Kernel h100-pcp.json evidence page's train/loss,
 * entropy_loss and grad_norm records; its comparison block finds the trained weights and
 * norms equal across parallel configurations, so the gradient must be deterministic):
 *     grad[r, i] = ( g_lp[r] (delta(i, t_r) - p_i) - g_ent[r] p_i (log p_i + H_r) ) / tau
 * with p = softmax(logits[r] / tau) and H_r the row's entropy (p log p taken as 0 at p = 0).
 *   logits, ld_logits, n_tokens, vocab, target_ids, temperature, vocab_splits: as for
 *                   rlk_logprob_from_logits (target_ids may be NULL if grad_logprob is NULL)
 *   grad_logprob    [n_tokens] fp32 upstream gradient of each row's logprob, or NULL (= 0)
 *   grad_entropy    [n_tokens] fp32 upstream gradient of each row's entropy, or NULL (= 0)
 *   row_states      [n_tokens] rlk_row_state saved by rlk_logprob_from_logits on the same
 *                   logits and temperature, or NULL: then they are recomputed (one more read
 *                   of the logits)
 *   grad_logits     [n_tokens, ld_grad] fp32 output, ld_grad >= vocab; it may be the logits
 *                   array itself (in place) when ld_grad == ld_logits, and must not
 *                   otherwise overlap it
 *   workspace       rlk_workspace_bytes(RLK_OP_BACKWARD_FROM_LOGITS, ...) bytes, 256-aligned
 * Row rules: a row whose two upstream gradients are both 0 gets all zeros; otherwise a row
 * whose forward outputs are NaN (NaN or +inf logit, all logits -inf), or whose target lies
 * outside [0, vocab) while grad_logprob is non-zero, gets NaN.  The gradient is bitwise
 * independent of the batch, the row order and vocab_splits: every element depends only on
 * its own logit and the row's canonical state.
 */
rlk_status rlk_logprob_backward_from_logits(const float* logits, int64_t ld_logits,
                                            int64_t n_tokens, int64_t vocab,
                                            const int64_t* target_ids, float temperature,
                                            int32_t vocab_splits, const float* grad_logprob,
                                            const float* grad_entropy,
                                            const rlk_row_state* row_states, float* grad_logits,
                                            int64_t ld_grad, void* workspace,
                                            size_t workspace_bytes, void* stream);

/*
 * Backward of the fused path: gradients of  sum_r g_lp[r] logprob[r] + g_ent[r] entropy[r]
 * with respect to the hidden states and the LM-head weight, for the quantities
 * rlk_linear_logprob computes (logits x = hidden . weight^T).  With dX the logit gradient of
 * rlk_logprob_backward_from_logits:   grad_hidden = dX . weight,   grad_weight = dX^T . hidden.
 * The RL-Kernel h100-pcp.json evidence page's training records consume both outputs and
 * find the trained weights equal across parallel configurations: the reductions here have
 * fixed orders (the vocabulary in 4 fixed ranges summed in a fixed tree for grad_hidden,
 * the tokens in increasing order for grad_weight), with no atomics, so results repeat
 * bitwise, and each row of grad_hidden is independent of the other rows of the batch.
 *   hidden, ld_hidden, weight, ld_weight, n_tokens, hidden_dim, vocab, target_ids,
 *   temperature, vocab_splits: as for rlk_linear_logprob (target_ids may be NULL if
 *                   grad_logprob is NULL)
 *   grad_logprob, grad_entropy: [n_tokens] fp32 upstream gradients, or NULL (= 0)
 *   row_states      [n_tokens] rlk_row_state saved by rlk_linear_logprob on the same
 *                   inputs and temperature, or NULL: then the forward is recomputed
 *   grad_hidden     [n_tokens, ld_grad_hidden] fp32 output, or NULL (not computed)
 *   grad_weight     [vocab, ld_grad_weight] fp32 output, or NULL (not computed)
 *   workspace       rlk_workspace_bytes(RLK_OP_LINEAR_BACKWARD, ...) bytes, 256-aligned
 * The logit gradient is formed in fp32 and rounded to bf16 for the two bf16 MFMA products
 * (fp32 accumulation).  Row rules as for rlk_logprob_backward_from_logits; a NaN row of the
 * logit gradient makes the corresponding grad_hidden row, and every grad_weight entry, NaN.
 * With n_tokens == 0 the gradient is that of an empty sum: grad_weight, when non-NULL, is
 * filled with zeros (one small launch; no workspace is needed).
 */
rlk_status rlk_linear_logprob_backward(const uint16_t* hidden_bf16, int64_t ld_hidden,
                                       const uint16_t* weight_bf16, int64_t ld_weight,
                                       int64_t n_tokens, int64_t hidden_dim, int64_t vocab,
                                       const int64_t* target_ids, float temperature,
                                       int32_t vocab_splits, const float* grad_logprob,
                                       const float* grad_entropy,
                                       const rlk_row_state* row_states, float* grad_hidden,
                                       int64_t ld_grad_hidden, float* grad_weight,
                                       int64_t ld_grad_weight, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Train-vs-rollout selected-logprob comparison over the active tokens: the figures the
 * RL-Kernel h100-pcp.json evidence page reports in its train_rollout_logprob block and
 * runtime_scalar_logprob rows, and that the RL-Kernel issue #342 runbook requires of the
 * per-row selected-logprob comparison (section 2: mismatch count 0, max abs diff 0.0).
 * With d = train - rollout evaluated in fp64 (exact for fp32 inputs):
 *   active_tokens           number of tokens with active_mask != 0 (all if mask is NULL)
 *   mismatch_count          active tokens with train != rollout as IEEE values
 *                           (NaN on either side counts; -0 equals +0)
 *   bitwise_mismatch_count  active tokens whose 32-bit patterns differ
 *   max_abs_diff            max |d|  (NaN if any active d is NaN)
 *   mean_abs_diff           sum |d| / n
 *   mismatch_kl             sum(-d) / n                 k1 estimate of KL(rollout || train)
 *   mismatch_k3_kl          sum(expm1(d) - d) / n       k3 estimate of KL(rollout || train)
 * with n = active_tokens; when n = 0 every figure is 0.  The rollout engine sampled the
 * tokens, which is why the log-ratio d estimates KL(rollout || train) this way.
 *   train_logprob, rollout_logprob  [n_tokens] fp32 device arrays
 *   active_mask     [n_tokens] uint8 device array or NULL
 *   result          one rlk_compare_result in DEVICE memory (8-byte aligned), written by the
 *                   call; unlike the other calls, n_tokens == 0 still launches one small
 *                   kernel, to write the all-zero result
 *   workspace       rlk_workspace_bytes(RLK_OP_COMPARE, n_tokens, ...) bytes, 256-aligned
 * Sizes: 0 <= n_tokens <= 2^40.
 * Deterministic: fixed token-to-thread mapping and a fixed combination tree, no atomics;
 * the same inputs give the same bits on every call.
 */
typedef struct {
  int64_t active_tokens;
  int64_t mismatch_count;
  int64_t bitwise_mismatch_count;
  int64_t reserved;          /* written as 0 */
  double max_abs_diff;
  double mean_abs_diff;
  double mismatch_kl;
  double mismatch_k3_kl;
} rlk_compare_result;       /* 64 bytes */

rlk_status rlk_logprob_compare(const float* train_logprob, const float* rollout_logprob,
                               const uint8_t* active_mask, int64_t n_tokens,
                               rlk_compare_result* result, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code (never NULL; "unknown status" for a
   value outside the enum).  The runbook's preflight (issue #342, section 1) fails closed
   with a reason instead of falling back; this is the reason's text. */
const char* rlk_status_string(rlk_status status);

/* Static identifier of the implementation that runs, "rlk.logprob.strict.gfx950.v1",
   recorded next to results as the h100-pcp.json evidence page's runtime readbacks record
   each operator's backend id (e.g. "rlkernel.linear_logp.bitwise.v1") with no fallback. */
const char* rlk_backend_id(void);

#ifdef __cplusplus
}
#endif

#endif /* RLK_LOGPROB_H */
