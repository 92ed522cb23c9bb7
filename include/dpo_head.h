/* dpo_head.h - C ABI of the DPO LM-head log-probability / loss / gradient path
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  "DPO Training on GPU, in depth" (aicassindra.com),
 * section "What one DPO step computes": each preference pair is a prompt with
 * a chosen and a rejected completion; a completion's score is the sum of its
 * token log-probabilities over completion tokens only; the loss is minus the
 * log-sigmoid of beta times the chosen-minus-rejected difference of
 * policy-minus-reference scores; chosen and rejected rows are concatenated
 * into one batch of 2B rows.  Section "A training configuration that fits"
 * gives the per-token step as a full-vocabulary log-softmax, a gather of the
 * target token, and a masked fp32-or-better sum per row; its memory section
 * ("Where the memory goes for an 8B model") is why the fused entry points
 * never build the [rows x T x V] logits.
 *
 * Conventions for every entry point:
 *  - Array arguments are DEVICE pointers owned by the caller.  The library
 *    never allocates or frees device memory and keeps no pointer after a call
 *    returns.  Scratch space is the caller's `workspace`, sized by
 *    dpo_workspace_bytes().
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the legacy default
 *    stream) and is asynchronous: outputs are valid once the stream has
 *    reached the end of the call.
 *  - Arguments are validated on the host before anything is enqueued; on
 *    error nothing is enqueued and a negative DPO_ERR_* code is returned.
 *  - bf16 arrays hold raw bfloat16 bit patterns (uint16_t).
 *  - "Aligned" targets: targets[r*T+t] is the token whose probability is read
 *    from the logits computed at (r, t); the caller applies the one-position
 *    shift of the page's hand-written loss by slicing.  mask[r*T+t] != 0
 *    marks a completion position.  Targets at mask-0 positions are never
 *    read as indices (they may hold the ignore value -100).
 *  - Shape rules: rows even and > 0; T, H, V > 0; H % 64 == 0; V % 8 == 0;
 *    rows*T < 2^31; the hidden tensor under 4 GiB (rows*T*H < 2^31).
 *    Pointers to bf16 and float arrays must be 16-byte aligned.
 *  - Target ids outside [0, V) at completion positions are detected on the
 *    device: the call's outputs for that position are NaN and
 *    dpo_device_status() reports DPO_ERR_TARGET_RANGE.
 *  - Results are deterministic run to run: no floating-point atomics.
 *  - Calls that share a workspace must not overlap in time (same stream, or
 *    ordered by events).
 */
#ifndef DPO_HEAD_H
#define DPO_HEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t dpo_bf16; /* raw bfloat16 bits */

enum {
  DPO_OK = 0,
  DPO_ERR_NULL = -1,         /* a required pointer is NULL */
  DPO_ERR_SHAPE = -2,        /* a size breaks the shape rules */
  DPO_ERR_ALIGN = -3,        /* a pointer is not 16-byte aligned */
  DPO_ERR_BETA = -4,         /* beta is not finite and > 0 */
  DPO_ERR_LAYOUT = -5,       /* unknown pair layout / flag value */
  DPO_ERR_WORKSPACE = -6,    /* workspace smaller than dpo_workspace_bytes() */
  DPO_ERR_TARGET_RANGE = -7, /* device-detected target id outside [0, V) */
  DPO_ERR_HIP = -8,          /* a HIP runtime call failed */
  DPO_ERR_ALPHA = -9,        /* sft_alpha is not finite and >= 0 */
  DPO_ERR_SCRATCH = -10      /* sizes beyond the no-allocation entry point's static scratch */
};

/* Pair layouts of the concatenated batch.
 * ADJACENT: rows 2i (chosen) and 2i+1 (rejected) - the Megatron-Bridge DPO
 *   change ("feat(training): add DPO training with offline-scored reference
 *   model", changelog) keeps a pair's rows next to each other.
 * HALVES: rows i (chosen) and B+i (rejected) - the torchtune recipe
 *   ("Run Distributed Full-Model DPO with PyTorch FSDP", step 4) and the
 *   hand-written loss on "DPO Training on GPU, in depth" split the batch in
 *   halves. */
enum { DPO_PAIRS_ADJACENT = 0, DPO_PAIRS_HALVES = 1 };

/* Operations for dpo_workspace_bytes(). */
enum {
  DPO_OP_SEQ_LOGPS = 0,
  DPO_OP_REF_SCORE = 1,
  DPO_OP_HEAD_BACKWARD = 2,
  DPO_OP_LOGITS_SEQ_LOGPS = 3, /* also the fp32-logits forward */
  DPO_OP_LOGITS_BACKWARD = 4,  /* also the fp32-logits backward */
  DPO_OP_SHARD_COMBINE = 5,    /* dpo_shard_combine; V = the whole vocabulary */
  DPO_OP_SEQ_LOGPS_METRICS = 6 /* dpo_seq_logps_metrics */
};
/* The vocabulary-shard entry points take the workspace of the unsharded
 * operation at the shard's size: dpo_workspace_bytes(DPO_OP_SEQ_LOGPS, ...,
 * V_shard) for dpo_seq_logps_shard and (DPO_OP_HEAD_BACKWARD, ..., V_shard)
 * for dpo_head_backward_shard. */

/* Flags of dpo_loss_ex. */
enum { DPO_LOSS_LENGTH_NORM = 1, DPO_LOSS_REFERENCE_FREE = 2 };

/* Bytes of device workspace `op` needs for these sizes (H is ignored by the
 * logits operations).  Returns 0 if the sizes break the shape rules or `op`
 * is unknown.  Pure host arithmetic; touches no device. */
size_t dpo_workspace_bytes(int op, int rows, int T, int H, int V);

/* Sequence scores of the policy: for each row r,
 *   logp_sum[r] = sum over completion positions t of log softmax(W h_{r,t})[y_{r,t}]
 * ("DPO Training on GPU, in depth": "What one DPO step computes" and the
 * hand-written loss in "A training configuration that fits"; sums, not
 * averages, as the torchtune recipe's concatenated forward returns).
 *   hidden   [rows, T, H] bf16  final hidden states
 *   w_vocab  [V, H] bf16        LM-head weight (row v = token v)
 *   targets  [rows, T] int32, mask [rows, T] uint8  (aligned, see above)
 *   logp_sum [rows] float       the row scores (fp32)
 *   logp_sum64 [rows] double    the same sums in fp64 (nullable); feed these
 *                               to dpo_loss for a loss accurate to 1e-4
 *   lse      [rows, T] float    per-position log-sum-exp over V, kept for the
 *                               backward; 0 at mask-0 positions (nullable)
 *   n_tokens [rows] int32       completion positions per row (nullable)
 * The [rows, T, V] logits are never formed: the contraction runs on MFMA
 * tiles and each tile keeps only a per-position running max and sum of
 * exponentials plus the target logit. */
int dpo_seq_logps(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                  const uint8_t* mask, int rows, int T, int H, int V, float* logp_sum,
                  double* logp_sum64, float* lse, int32_t* n_tokens, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Offline reference scoring: per-row completion log-prob sums, no beta applied
 * ("feat(training): add DPO training with offline-scored reference model",
 * section "Why the reference is scored offline"; "DPO Training on GPU, in
 * depth", section "Four ways to host the reference model", item 3).  Same
 * inputs as dpo_seq_logps; output ref_sum [rows] float. */
int dpo_ref_score(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                  const uint8_t* mask, int rows, int T, int H, int V, float* ref_sum,
                  void* workspace, size_t workspace_bytes, void* stream);

/* The sigmoid DPO loss ("DPO Training on GPU, in depth", sections "What one
 * DPO step computes" and "A worked example of the numbers"), in fp64:
 *   reward_r = beta (policy_r - ref_r);  margin_i = reward_chosen - reward_rejected
 *   loss = mean over the num_pairs pairs of -log sigmoid(margin_i)
 *   weight_r = -d loss / d policy_r = +beta sigmoid(-margin_i) / num_pairs on the
 *              chosen row, the negative on the rejected row (the page's
 *              per-pair gradient scale sigmoid(-margin))
 *   accuracy = fraction of pairs with margin_i > 0 (strict)
 *   policy_sum64 [2B] double, ref_sum [2B] float, layout DPO_PAIRS_*
 *   loss [1] float; weight [2B] float; reward [2B], margin [B], accuracy [1]
 *   float, each nullable.
 * A caller that accumulates gradients over k micro-batches scales `weight`
 * by 1/k before dpo_head_backward. */
int dpo_loss(const double* policy_sum64, const float* ref_sum, int num_pairs, double beta,
             int layout, float* loss, float* weight, float* reward, float* margin,
             float* accuracy, void* stream);

/* The loss variants the pages name, on the same scores and weights; the
 * backward entry points take the resulting `weight` unchanged.
 *  - DPO_LOSS_REFERENCE_FREE: reference scores are 0 and ref_sum may be NULL
 *    ("Run Distributed Full-Model DPO with PyTorch FSDP", "Where to Go
 *    Next": a reference-free objective drops the reference model).
 *  - DPO_LOSS_LENGTH_NORM: every row's policy and reference score is divided
 *    by its completion token count n_tokens[r] before the margin ("DPO
 *    Training on GPU, in depth", "Failure modes you will see on real runs":
 *    length-normalised variants such as sigmoid_norm); a row without tokens
 *    averages to 0 and gets weight 0.
 *  - sft_alpha > 0: loss += sft_alpha * NLL with NLL = -sum(policy of chosen
 *    rows) / sum(n_tokens of chosen rows), the mean negative log-probability
 *    per chosen completion token of the batch ("Direct Preference
 *    Optimization (DPO): End-to-End Implementation": DPO loss plus RPO alpha
 *    times the NLL on the chosen responses; the Megatron-Bridge change's
 *    optional SFT term).  Every chosen row's weight grows by
 *    sft_alpha / sum(n_tokens of chosen rows).
 *   n_tokens [2B] int32: required for LENGTH_NORM, sft_alpha > 0 or a
 *     non-NULL nll; the counts dpo_seq_logps wrote.
 *   nll [1] float, nullable: the NLL value (also when sft_alpha == 0).
 *   loss = preference loss + sft_alpha * NLL; other outputs as dpo_loss.
 * Errors: unknown flag bits -> DPO_ERR_LAYOUT; bad sft_alpha -> DPO_ERR_ALPHA. */
int dpo_loss_ex(const double* policy_sum64, const float* ref_sum, const int32_t* n_tokens,
                int num_pairs, double beta, int layout, int flags, double sft_alpha, float* loss,
                float* weight, float* reward, float* margin, float* accuracy, float* nll,
                void* stream);

/* Head gradients of the loss through the row scores:
 *   D_{r,t} = weight_r (softmax(W h_{r,t}) - onehot(y_{r,t}))   at completion positions
 *   d_hidden[r,t,:] = D_{r,t} W      (exactly 0 at mask-0 positions)
 *   d_w_vocab       = sum_{r,t} D_{r,t}^T h_{r,t}   (overwrite if accumulate_dw == 0,
 *                                                    add to the existing values if 1)
 * lse is the array dpo_seq_logps wrote; weight the array dpo_loss wrote.
 * The logits are recomputed tile by tile (the page's chunked loss recomputes
 * its log-softmax in backward the same way); D exists only as a bf16 operand
 * in the workspace.  d_hidden [rows, T, H] and d_w_vocab [V, H] are fp32. */
int dpo_head_backward(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                      const uint8_t* mask, int rows, int T, int H, int V, const float* lse,
                      const float* weight, float* d_hidden, float* d_w_vocab, int accumulate_dw,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Bandwidth-bound variant over pre-materialised logits: the per-token step
 * of the hand-written chunked loss on "DPO Training on GPU, in depth",
 * section "A training configuration that fits" (it takes logits and labels,
 * applies a full-vocabulary log-softmax, gathers the label's entry and sums
 * over the completion mask), for a caller that already holds the logits
 * whose size that page's section "Where the memory goes for an 8B model"
 * works out (0.49 GiB per 2,048-token sequence in bf16 at V = 128,256).
 *   logits   [rows, T, V] bf16  row-major, 16-byte aligned; read once per
 *                               completion position, never at mask-0 ones
 *   targets, mask, rows, T, V, workspace: as dpo_seq_logps (H does not exist
 *     here; workspace DPO_OP_LOGITS_SEQ_LOGPS)
 *   logp_sum, logp_sum64, lse, n_tokens: as dpo_seq_logps.
 * Logits may hold -inf (a caller's vocabulary masking); those entries add
 * nothing to the log-sum-exp.  A position whose logits are all -inf, or whose
 * target's logit is -inf, has no finite log-probability. */
int dpo_logits_seq_logps(const dpo_bf16* logits, const int32_t* targets, const uint8_t* mask,
                         int rows, int T, int V, float* logp_sum, double* logp_sum64, float* lse,
                         int32_t* n_tokens, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Backward of that loss over the given logits (the gradient the page's
 * chunked loss produces by autograd in "A training configuration that fits";
 * its section "Where the memory goes for an 8B model" counts this tensor next
 * to the logits):
 *   d_logits[r,t,:] = weight_r (softmax(logits[r,t,:]) - onehot(y_{r,t}))
 * at completion positions, exactly 0 at mask-0 positions, rounded to bf16
 * (nearest even).
 *   logits [rows, T, V] bf16; lse [rows, T] float from dpo_logits_seq_logps;
 *   weight [rows] float from dpo_loss; d_logits [rows, T, V] bf16, written in
 *   full (16-byte aligned, must not overlap logits).
 *   workspace: DPO_OP_LOGITS_BACKWARD (a status word only); a target outside
 *   [0, V) at a completion position is reported by dpo_device_status. */
int dpo_logits_backward(const dpo_bf16* logits, const int32_t* targets, const uint8_t* mask,
                        int rows, int T, int V, const float* lse, const float* weight,
                        dpo_bf16* d_logits, void* workspace, size_t workspace_bytes,
                        void* stream);

/* The same two streaming passes over fp32 logits ("DPO Training on GPU, in
 * depth", "Where the memory goes for an 8B model": fp32 logits of a
 * 2,048-token sequence take 0.98 GiB).  logits [rows, T, V] float; the
 * backward writes d_logits [rows, T, V] float (no rounding), 0 at mask-0
 * positions.  Workspaces: DPO_OP_LOGITS_SEQ_LOGPS / DPO_OP_LOGITS_BACKWARD. */
int dpo_logits_f32_seq_logps(const float* logits, const int32_t* targets, const uint8_t* mask,
                             int rows, int T, int V, float* logp_sum, double* logp_sum64,
                             float* lse, int32_t* n_tokens, void* workspace,
                             size_t workspace_bytes, void* stream);
int dpo_logits_f32_backward(const float* logits, const int32_t* targets, const uint8_t* mask,
                            int rows, int T, int V, const float* lse, const float* weight,
                            float* d_logits, void* workspace, size_t workspace_bytes,
                            void* stream);

/* One GPU's share of a head whose vocabulary is split over GPUs (tensor
 * parallelism over W_vocab rows; the Megatron-Bridge change scores and trains
 * with TP=4 and notes that the sums change with the shard count).  This GPU
 * holds W rows [v_begin, v_begin + V_shard) of a V_total vocabulary as
 * w_shard [V_shard, H] (V_shard % 8 == 0, v_begin >= 0,
 * v_begin + V_shard <= V_total).  Targets are global ids in [0, V_total).
 *
 * dpo_seq_logps_shard writes, for every position (layout [rows, T], float):
 *   part_max     max over the shard's logits   (-inf at mask-0 positions)
 *   part_sumexp  sum over the shard of exp(z - part_max)   (0 at mask-0)
 *   part_tgt     the target's logit if this shard holds the target, else -inf
 * A caller gathers the S shards' arrays into [S, rows, T] (one all-gather of
 * 12 bytes per position) and calls dpo_shard_combine, which forms
 *   lse = M + log(sum_s part_sumexp_s exp(part_max_s - M)),  M = max_s part_max_s
 *   log p = (the one finite part_tgt) - lse
 * in fp64 and writes the same outputs as dpo_seq_logps.  A completion
 * position that no shard holds the target of is reported through
 * dpo_device_status as DPO_ERR_TARGET_RANGE.
 *
 * dpo_head_backward_shard takes the combined lse and the loss weights and
 * writes this shard's share: d_hidden [rows, T, H] fp32 is the shard's term
 * D_shard W_shard (the shards' terms add up to the whole dHidden: one
 * all-reduce), d_w_shard [V_shard, H] fp32 the shard's rows of dW_vocab.
 * The one-hot part of D applies only where this shard holds the target. */
int dpo_seq_logps_shard(const dpo_bf16* hidden, const dpo_bf16* w_shard, const int32_t* targets,
                        const uint8_t* mask, int rows, int T, int H, int V_shard, int v_begin,
                        int V_total, float* part_max, float* part_sumexp, float* part_tgt,
                        void* workspace, size_t workspace_bytes, void* stream);
int dpo_shard_combine(const float* part_max, const float* part_sumexp, const float* part_tgt,
                      int num_shards, const int32_t* targets, const uint8_t* mask, int rows, int T,
                      int V_total, float* logp_sum, double* logp_sum64, float* lse,
                      int32_t* n_tokens, void* workspace, size_t workspace_bytes, void* stream);
int dpo_head_backward_shard(const dpo_bf16* hidden, const dpo_bf16* w_shard,
                            const int32_t* targets, const uint8_t* mask, int rows, int T, int H,
                            int V_shard, int v_begin, int V_total, const float* lse,
                            const float* weight, float* d_hidden, float* d_w_shard,
                            int accumulate_dw, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Forward by-products for the logits-mean metrics ("Run Distributed
 * Full-Model DPO with PyTorch FSDP", "What to Watch Out For": the loop logs the
 * mean chosen and rejected logits and then frees the logits).  Here the
 * logits never exist, so the forward epilogue sums them on the way:
 * dpo_seq_logps_metrics is dpo_seq_logps plus
 *   logit_sum [rows] double = sum over the row's completion positions and all
 *                             V vocabulary entries of the logits
 * (workspace DPO_OP_SEQ_LOGPS_METRICS).  dpo_logits_mean turns the sums into
 *   means[0] = mean logit of the chosen rows, means[1] = of the rejected rows,
 * each over (completion positions x V); 0 for a half without tokens.  The
 * pages average over the whole logits tensor; this library has logits only at
 * completion positions, so the means cover those. */
int dpo_seq_logps_metrics(const dpo_bf16* hidden, const dpo_bf16* w_vocab, const int32_t* targets,
                          const uint8_t* mask, int rows, int T, int H, int V, float* logp_sum,
                          double* logp_sum64, float* lse, int32_t* n_tokens, double* logit_sum,
                          void* workspace, size_t workspace_bytes, void* stream);
int dpo_logits_mean(const double* logit_sum, const int32_t* n_tokens, int num_pairs, int V,
                    int layout, float* means, void* stream);

/* dpo_logits_seq_logps without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  It allocates nothing and calls no allocating
 * routine: its scratch (a 256-byte status header, fp64 log p and a target
 * flag per position) is a static device array of 12 MiB + 256 bytes that each
 * GPU the library runs on holds until the process ends.
 *   Same inputs and outputs as dpo_logits_seq_logps, without workspace, plus
 *   status [1] int32 (device): DPO_OK, or DPO_ERR_TARGET_RANGE if a target at
 *   a completion position lies outside [0, V); written on `stream` at the end
 *   of the call (dpo_device_status does not apply: there is no workspace).
 * Limit: rows * T <= 2^20 positions, else DPO_ERR_SCRATCH before any launch.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents: calls that overlap in time on one GPU (different streams
 * without ordering, or different host threads) race and give wrong results.
 * Calls ordered on one stream are safe. */
int dpo_logits_seq_logps_noalloc(const dpo_bf16* logits, const int32_t* targets, const uint8_t* mask,
                                 int rows, int T, int V, float* logp_sum, double* logp_sum64, float* lse,
                                 int32_t* n_tokens, int32_t* status, void* stream);

/* Waits for `stream`, then returns DPO_ERR_TARGET_RANGE if the most recent
 * call that used `workspace` met a target id outside [0, V) at a completion
 * position, DPO_OK otherwise (or DPO_ERR_HIP). */
int dpo_device_status(void* workspace, void* stream);

/* Static description of a status code. */
const char* dpo_strerror(int status);

/* Kernel timing.  While enabled, every kernel the library enqueues is
 * bracketed by a pair of HIP events on its stream.  dpo_profile_count()
 * waits for the recorded events and returns the number of distinct kernels
 * seen; dpo_profile_entry() returns, for entry i, the kernel name, the summed
 * duration in milliseconds and the number of launches.  Enabling (on=1) or
 * disabling (on=0) clears what was collected.  dpo_profile_select() limits the
 * timing to the kernels named `name` (the names dpo_profile_entry() reports;
 * NULL or "" restores all kernels); the string is copied, and the choice holds
 * until the next call, across enable/disable.  Host-only: it touches no
 * device and never fails. */
int dpo_profile_enable(int on);
int dpo_profile_select(const char* name);
int dpo_profile_count(void);
int dpo_profile_entry(int i, const char** name, double* total_ms, int* launches);

#ifdef __cplusplus
}
#endif

#endif /* DPO_HEAD_H */
