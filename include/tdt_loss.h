/*
 * tdt_loss.h — C ABI of the MI355X (gfx950) Token-and-Duration Transducer loss.
 *
 * One call computes the TDT loss and its gradient with respect to the token logits and
 * the duration logits of a joint network output, as described on the page
 * "tdt-loss: add TDT loss kernel" (huggingface/kernels-community PR #882, comment
 * "What's in it"): a log-softmax over the vocabulary of every lattice node, float64
 * alpha/beta passes over the lattice with no limit of 1024 labels, one fused gradient
 * pass for token and duration logits, fp32/fp16/bf16 logits read in place (slices of
 * the joint output such as logits[..., :V] are not copied), and the reductions
 * mean_volume, mean_batch, mean, sum and none.  Labels are padded with -100 (page
 * "Add TDT loss kernel", huggingface/transformers PR #46048, commit summary on label
 * padding).  sigma is the logit under-normalisation discussed in that page's review
 * thread on sigma.
 *
 * Definitions, for utterance b with T = logit_lengths[b] frames, U = label_lengths[b]
 * labels y_1..y_U and lattice nodes n = (t, u), 0 <= t < T, 0 <= u <= U:
 *   - a blank with duration d > 0 moves (t,u) -> (t+d,u) when t+d < T, and ends the
 *     alignment when u == U and t+d == T;
 *   - label y_{u+1} with any duration d (0 allowed) moves (t,u) -> (t+d,u+1) when
 *     u < U and t+d < T;
 *   - each move weighs log_softmax(h(n))[token] - sigma + log_softmax(g(n))[d's index],
 *     where h(n) are the V token logits (blank included) and g(n) the D duration logits;
 *   - loss_b = -log of the sum over alignments of exp(sum of move weights).
 * Reductions with per-utterance gradient weights w_b:
 *   none -> loss[b] = loss_b (w_b = 1);  sum -> sum_b loss_b (w_b = 1);
 *   mean_batch -> sum_b loss_b / B;  mean -> (1/B) sum_b loss_b / max(U_b, 1);
 *   mean_volume -> sum_b loss_b / max(sum_b U_b, 1).
 * The gradient written is d(reduced loss)/d(logits) (for 'none': of sum_b loss_b),
 * exactly 0 at padded nodes (t >= T or u > U), in the dtype of the logits, rounded to
 * nearest even.
 */
#ifndef TDT_LOSS_H
#define TDT_LOSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the logits (and of the gradients, which use the same type). */
typedef enum { TDT_DTYPE_F32 = 0, TDT_DTYPE_F16 = 1, TDT_DTYPE_BF16 = 2 } tdt_dtype_t;

typedef enum {
  TDT_REDUCTION_NONE = 0,
  TDT_REDUCTION_SUM = 1,
  TDT_REDUCTION_MEAN = 2,
  TDT_REDUCTION_MEAN_BATCH = 3,
  TDT_REDUCTION_MEAN_VOLUME = 4
} tdt_reduction_t;

/* Return codes (host-detectable errors; nothing is launched when one is returned). */
#define TDT_OK 0
#define TDT_ERR_INVALID_ARGUMENT (-1)  /* null pointer, bad size, bad enum, bad durations, bad blank, non-finite sigma */
#define TDT_ERR_UNSUPPORTED_DTYPE (-2) /* dtype not one of tdt_dtype_t */
#define TDT_ERR_BAD_STRIDE (-3)        /* pointer not aligned to the element size */
#define TDT_ERR_WORKSPACE_TOO_SMALL (-4)
#define TDT_ERR_UNSUPPORTED (-5)       /* a size beyond this library's limits (see below) */
#define TDT_ERR_HIP (-6)               /* a HIP launch failed */

/* Per-utterance status bits written to utt_status[b] (device memory, may be NULL).
 * A data error makes that utterance's loss NaN and its gradient 0; other utterances
 * are unaffected (the reduced loss becomes NaN).  An utterance with no alignment
 * (e.g. T == 0, or durations {2} and odd T) gets loss +inf, gradient 0. */
#define TDT_UTT_BAD_LOGIT_LENGTH 1 /* logit_lengths[b] outside [0, T_max] */
#define TDT_UTT_BAD_LABEL_LENGTH 2 /* label_lengths[b] outside [0, U1_max - 1] */
#define TDT_UTT_BAD_LABEL 4        /* a label y_1..y_U outside [0, V) */
#define TDT_UTT_INFEASIBLE 8       /* no alignment exists */

/* Limits of the library: 1 <= num_durations <= 16, duration values in [0, 16] with at
 * least one > 0, T_max and U1_max below 2^24 with T_max * U1_max below 2^27, and fewer
 * than 2^31 (node, row segment) pairs per call, a row segment being up to 512 16-byte
 * chunks of a logits row (beyond these: TDT_ERR_UNSUPPORTED).  There is no other limit on
 * the label count: long label sequences are swept as bands of tiles.  bf16 logits whose
 * row maximum exceeds about 2.3e38 in magnitude give their utterance a NaN loss; a move
 * whose log-weight is below about -9.3e7 (e.g. a logit masked with -1e10) is impossible. */
#define TDT_MAX_DURATIONS 16
#define TDT_MAX_DURATION_VALUE 16

/*
 * Workspace bytes needed by tdt_loss_fwd_bwd for these sizes.
 *   dtype: tdt_dtype_t of the logits.  B, T_max, U1_max: padded batch shape of the
 *   logits [B, T_max, U1_max, *].  V: token classes.  durations[num_durations]: host
 *   array of the duration values.
 * Writes the size to *bytes and returns TDT_OK, or a negative code for invalid sizes.
 */
int tdt_loss_workspace_size(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                            const int32_t* durations, int32_t num_durations, size_t* bytes);

/*
 * TDT loss forward and backward, stream-ordered on `stream` (a hipStream_t; NULL =
 * the default stream): results are ready when work enqueued after the call on `stream`
 * runs.  The call only validates arguments on the host and enqueues kernels (see the
 * launch sequence below): it never synchronises, never allocates device memory and
 * keeps no pointer after it returns.  All pointers except `durations` and the three stride arrays are device
 * pointers owned by the caller.
 *
 *   dtype            element type of logits, dur_logits, grad_logits, grad_dur_logits.
 *   B, T_max, U1_max padded shape; U1_max = (maximum label count) + 1.
 *   V                number of token classes, blank included.
 *   logits           token logits [B, T_max, U1_max, V], element strides
 *                    logits_strides[0..2] for the first three dims, unit stride in the
 *                    last one (e.g. joint[..., :V] of a [B, T_max, U1_max, V + D] joint).
 *   dur_logits       duration logits [B, T_max, U1_max, D], strides dur_strides[0..2],
 *                    unit last stride (e.g. joint[..., V:]).  May alias `logits`' buffer.
 *   labels           int64 [B, >= U1_max - 1], row stride labels_stride elements;
 *                    entries at index >= label_lengths[b] (-100 padding) are never read.
 *   logit_lengths    int64 [B] frames per utterance.
 *   label_lengths    int64 [B] labels per utterance.
 *   durations        host int32 [num_durations]: distinct duration values (see limits).
 *   blank            blank id in [0, V).
 *   sigma            logit under-normalisation, subtracted once per emission (finite).
 *   reduction        tdt_reduction_t.
 *   loss_out         float [B] for TDT_REDUCTION_NONE, else float [1].
 *   grad_logits      gradient w.r.t. logits, same shape, strides grad_strides[0..2];
 *                    NULL together with grad_dur_logits for a forward-only call.  Every
 *                    element of the [B, T_max, U1_max, V] view is written (zeros in
 *                    padding), so it may start uninitialised.  May share a buffer with
 *                    grad_dur_logits (e.g. two slices of one joint gradient).  In place:
 *                    grad_logits may be the logits view itself (same pointer and
 *                    strides); the logits are then overwritten by their gradient, which
 *                    saves a logits-sized buffer (the memory saving the page "tdt-loss:
 *                    add TDT loss kernel" reports for fine-tuning, comment "What's in
 *                    it").  Any other overlap of a gradient view with a logits view
 *                    returns TDT_ERR_INVALID_ARGUMENT.
 *   grad_dur_logits  gradient w.r.t. dur_logits [B, T_max, U1_max, D], strides
 *                    grad_dur_strides[0..2]; may likewise be the dur_logits view itself.
 *   utt_status       int32 [B] status bits, or NULL.
 *   workspace        device scratch of at least tdt_loss_workspace_size() bytes,
 *                    256-byte aligned; its contents need no initialisation and are
 *                    overwritten.  Calls that share a workspace must not overlap.
 * Returns TDT_OK or a negative TDT_ERR_* code.
 *
 * Long label sequences run as label columns in work-groups that wait on each other; they
 * are launched only when the GPU holds all of them at once, and every wait is bounded
 * (about 0.1 s), after which the utterance is recomputed by the extended-range sweeps, so
 * work on other streams can slow a call down but not stop it.  The environment variable
 * TDT_LINK_SPIN_LIMIT (read at each call; for tests) lowers that bound to the given
 * number of polls, forcing that recomputation.
 */
int tdt_loss_fwd_bwd(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                     const void* logits, const int64_t* logits_strides, const void* dur_logits,
                     const int64_t* dur_strides, int32_t num_durations, const int64_t* labels,
                     int64_t labels_stride, const int64_t* logit_lengths, const int64_t* label_lengths,
                     const int32_t* durations, int32_t blank, double sigma, int32_t reduction, float* loss_out,
                     void* grad_logits, const int64_t* grad_strides, void* grad_dur_logits,
                     const int64_t* grad_dur_strides, int32_t* utt_status, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Launch sequence, all on `stream`, in order: row partials (log-sum-exp partials of the
 * token-logit rows), node weights, lattice (alpha and beta sweeps), coefficients (which
 * also reduce the loss), gradient pass.  For rows of at most 256 16-byte chunks whose
 * logits and gradient rows share their address modulo 16 bytes, the gradient pass
 * computes the coefficients itself and reduces the loss (no coefficient kernel).  A
 * forward-only call runs a loss-reduction kernel in place of the coefficients and the
 * gradient pass.
 *
 * Same as tdt_loss_fwd_bwd, and additionally records caller-created events (hipEvent_t
 * handles on the device of `stream`; NULL entries are skipped) on `stream`, for tools
 * that attribute time per kernel:
 *   num_events == 4: events[0] before the first kernel, [1] after the last one, [2]
 *     right before the gradient pass and [3] right after it;
 *   num_events == 7: events[0] before the row partials, [1] after them, [2] after the
 *     node weights, [3] after the lattice, [4] after the coefficients (directly after [3]
 *     when the gradient pass computes them), [5] after the gradient pass, [6] after the
 *     loss reduction kernel (forward only; with gradients [6] directly follows [5]).
 * Any other count (or events == NULL) returns TDT_ERR_INVALID_ARGUMENT.
 */
int tdt_loss_fwd_bwd_timed(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                           const void* logits, const int64_t* logits_strides, const void* dur_logits,
                           const int64_t* dur_strides, int32_t num_durations, const int64_t* labels,
                           int64_t labels_stride, const int64_t* logit_lengths, const int64_t* label_lengths,
                           const int32_t* durations, int32_t blank, double sigma, int32_t reduction,
                           float* loss_out, void* grad_logits, const int64_t* grad_strides, void* grad_dur_logits,
                           const int64_t* grad_dur_strides, int32_t* utt_status, void* workspace,
                           size_t workspace_bytes, void* stream, void* const* events, int32_t num_events);

/*
 * Gradient of a loss computed earlier by a forward-only tdt_loss_fwd_bwd call (both
 * gradient pointers NULL), for autograd-style use where the upstream gradient is known
 * only later.  Stream-ordered on `stream`; runs the coefficient kernel (when the launch
 * sequence above has one) and the gradient pass on the state the forward call
 * left in `workspace`, so between the two calls the workspace must be untouched, and
 * logits, dur_logits, labels, the two length arrays and every size, durations, blank,
 * sigma and reduction must be the same (contents included).  Nothing is checked on the
 * device against the forward call: other values give meaningless gradients.
 *
 *   grad_loss        device float, the upstream gradient d(objective)/d(loss_out): [B]
 *                    for TDT_REDUCTION_NONE (utterance b's gradient is scaled by
 *                    grad_loss[b]), else [1]; NULL means 1.  It multiplies the
 *                    per-utterance weights w_b in float64, so grad_loss = 1 gives the
 *                    bits of tdt_loss_fwd_bwd's gradients.
 *   grad_logits, grad_dur_logits  required; the same rules as in tdt_loss_fwd_bwd
 *                    (in place allowed).
 * The loss and the status array are not written.  Returns TDT_OK or a negative
 * TDT_ERR_* code (nothing is launched then).
 */
int tdt_loss_backward(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V, const void* logits,
                      const int64_t* logits_strides, const void* dur_logits, const int64_t* dur_strides,
                      int32_t num_durations, const int64_t* labels, int64_t labels_stride,
                      const int64_t* logit_lengths, const int64_t* label_lengths, const int32_t* durations,
                      int32_t blank, double sigma, int32_t reduction, const float* grad_loss, void* grad_logits,
                      const int64_t* grad_strides, void* grad_dur_logits, const int64_t* grad_dur_strides,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): tdt_loss_fwd_bwd without the
 * workspace arguments.  The workspace is a library-owned device array of
 * TDT_NOALLOC_SCRATCH_BYTES on each GPU the library runs on (held until the process
 * ends); this call allocates nothing and frees nothing.  Arguments, launch sequence,
 * results and return codes are those of tdt_loss_fwd_bwd (the same kernels), except that
 * sizes whose tdt_loss_workspace_size() exceeds TDT_NOALLOC_SCRATCH_BYTES return
 * TDT_ERR_WORKSPACE_TOO_SMALL before anything is launched, and a failure to obtain the
 * array's device address returns TDT_ERR_HIP.  The array of a GPU is found from
 * `stream`'s device (the current device for the NULL stream).  Every call on one GPU
 * shares that GPU's array and overwrites its contents: calls that may overlap in time on
 * one GPU (other streams, other threads) race and must not be issued.
 */
#define TDT_NOALLOC_SCRATCH_BYTES (64u << 20)
int tdt_loss_fwd_bwd_noalloc(int32_t dtype, int64_t B, int64_t T_max, int64_t U1_max, int64_t V,
                             const void* logits, const int64_t* logits_strides, const void* dur_logits,
                             const int64_t* dur_strides, int32_t num_durations, const int64_t* labels,
                             int64_t labels_stride, const int64_t* logit_lengths, const int64_t* label_lengths,
                             const int32_t* durations, int32_t blank, double sigma, int32_t reduction,
                             float* loss_out, void* grad_logits, const int64_t* grad_strides, void* grad_dur_logits,
                             const int64_t* grad_dur_strides, int32_t* utt_status, void* stream);

/* Static string naming a return code. */
const char* tdt_loss_status_string(int status);

/* ABI version of this library (incremented on incompatible changes). */
int tdt_loss_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TDT_LOSS_H */
