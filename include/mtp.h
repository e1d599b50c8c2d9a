/*
 * mtp.h -- C ABI of libmtp: MTP rejection-sampling verification and the
 * end-to-end multi-step TV loss on AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the pages about "Breaking Entropy Bounds:
 * Accelerating RL Training via MTP with Rejection Sampling" (Bebop, arXiv
 * 2606.12370): paperlayer.ai summary Sec. 2 "Acceptance methods", Sec. 3
 * "Rejection Sampling", Sec. 4 "End-to-end TV loss", App. A "Derivation of TV
 * Loss Gradient", App. F "Fused TV Loss Kernel", App. G.1 "Multinomial Draft
 * Sampling (SGLang)"; paper.rainbus.top summary, prerequisites "Rejection
 * Sampling", "Total Variation Distance", "Entropy", and "Method steps".
 *
 * Conventions for every entry point:
 *  - Pointers named as device pointers refer to GPU memory owned by the caller.
 *    The library never allocates, frees or keeps a pointer past the call.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream)
 *    and the call returns without synchronising.  Faults inside kernels surface
 *    at the caller's next synchronisation.
 *  - Argument errors are detected before any HIP call; the call then returns a
 *    non-zero mtp_status, writes nothing and launches nothing.  mtp_last_error()
 *    gives a thread-local description of the last failure.
 *  - Logit rows are contiguous in the vocabulary dimension.  Row base addresses
 *    must be 16-byte aligned (the pointer and stride * element size multiples of
 *    16).  V need not be a multiple of anything.
 *  - Logits may contain -inf (masked tokens).  Rows whose log-sum-exp is not
 *    finite (all -inf, NaN, +inf) are reported through row_status, not as a
 *    call failure.
 *  - Workspaces: query the size, allocate it (256-byte aligned), and zero it
 *    once before its first use.  Each call leaves its workspace zeroed again when
 *    it completes, so one workspace can serve any sequence of calls on one
 *    stream.  Calls that use the same workspace concurrently race.  A workspace
 *    size depends on the device (how many workgroups it holds at once): size it on
 *    the device that runs the calls.
 *  - Co-residency: the verify calls and the single-read TV forward run persistent
 *    grids whose workgroups exchange row statistics, so every workgroup of a grid
 *    must be resident on the GPU at the same time.  The grid is sized from the
 *    device's occupancy for an otherwise idle GPU; work from other streams or
 *    processes that holds compute units can keep some workgroups waiting.  Every
 *    such wait is bounded (one second by default, mtp_set_wait_limit): a wait
 *    that gives up sets the workspace's error word (mtp_workspace_error) and the
 *    affected rows report it -- verify rows get MTP_ROW_SYNC_TIMEOUT, NaN overlap
 *    and TV, token -1 and a rejection; TV-loss positions get NaN alpha, S and
 *    loss.  The call itself still returns MTP_OK (it has returned before the
 *    kernels run).  The verify calls finish each sequence in the same grid, in a
 *    workgroup whose own share is done; its wait for the sequence's rows is bounded
 *    by the larger of that limit and one second.  If that wait gives up (some
 *    workgroup of the grid could not run for that long), workspace words written
 *    after it may stay set: zero the workspace again before reusing it.
 */
#ifndef MTP_H
#define MTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status and dtype codes are plain 32-bit integers (any value may be passed in:
 * unknown dtype codes are rejected with MTP_ERR_DTYPE, unknown status codes have
 * a status string), named by the constants below. */
typedef int32_t mtp_status;
enum {
  MTP_OK = 0,
  MTP_ERR_NULL = 1,       /* a required pointer is NULL                          */
  MTP_ERR_SHAPE = 2,      /* a size or stride is out of range                    */
  MTP_ERR_DTYPE = 3,      /* unknown dtype code                                  */
  MTP_ERR_ALIGN = 4,      /* a row base address is not 16-byte aligned           */
  MTP_ERR_WORKSPACE = 5,  /* workspace NULL, misaligned or smaller than required */
  MTP_ERR_DEVICE = 6,     /* a HIP device query failed                           */
  MTP_ERR_LAUNCH = 7      /* a kernel launch failed                              */
};

typedef int32_t mtp_dtype;
enum { MTP_F32 = 0, MTP_BF16 = 1 };

/* row_status bits (per verify row) */
#define MTP_ROW_BAD_TOKEN 1       /* draft token outside [0, V): counted as a rejection    */
#define MTP_ROW_BAD_TARGET 2      /* target row has no finite log-sum-exp                 */
#define MTP_ROW_BAD_DRAFT 4       /* draft row has no finite log-sum-exp                  */
#define MTP_ROW_RESIDUAL_EMPTY 8  /* max(0, p - q) has no mass: the row sampled from p    */
#define MTP_ROW_SYNC_TIMEOUT 16   /* a bounded wait for the row's statistics gave up      */

#define MTP_MAX_GAMMA 8

/* ------------------------------------------------------------------------ */
/* Verification (paperlayer Sec. 2 "Acceptance methods", App. G.1; rainbus
 * "Rejection Sampling"; the EntMTP page, Related Work "Speculative Decoding").
 *
 * For sequence b and draft position k < gamma, with p = softmax(target row
 * (b, k)) and q = softmax(draft row (b, k)):
 *   accept[b, k]   = u < min(1, p(y) / q(y)),  y = draft_tokens[b, k]
 *   overlap[b, k]  = sum_v min(p_v, q_v)
 *   tv[b, k]       = sum_v max(0, p_v - q_v)        (= 1 - overlap)
 *   entropy[b, k]  = -sum_v p_v ln p_v,  also for the bonus row k = gamma
 *   row_token[b,k] = inverse-CDF sample in vocabulary order of
 *                    r = max(0, p - q)  (k < gamma)  or  r = p  (k = gamma):
 *                    the smallest v whose running sum of r exceeds u' * sum r
 *   accepted_len[b] = n = number of leading accepts (0..gamma)
 *   next_token[b]   = row_token[b, n]
 * u and u' are Philox4x32-10 outputs (words 0 and 1, each (w >> 8) * 2^-24) with
 * key = seed and 64-bit counter = offset + b * (gamma + 1) + k.  Advance `offset`
 * by batch * (gamma + 1) between calls for fresh uniforms.
 *
 * target: device, dtype, rows (b, k) at target + (b*(gamma+1) + k) * target_row_stride
 *         elements, k = 0..gamma.
 * draft:  device, dtype, rows (b, k) at draft + (b*gamma + k) * draft_row_stride, k < gamma.
 * draft_tokens: device int32 [batch, gamma].
 * Required outputs (device): accept uint8 [batch, gamma], accepted_len int32 [batch],
 *   next_token int32 [batch].
 * Optional outputs (device, NULL to skip): row_token int32 [batch, gamma+1],
 *   overlap, tv float [batch, gamma], entropy float [batch, gamma+1],
 *   row_status int32 [batch, gamma+1] (MTP_ROW_* bits).
 * Rows with MTP_ROW_BAD_TARGET / MTP_ROW_BAD_DRAFT give NaN statistics, token -1
 * and a rejection; MTP_ROW_SYNC_TIMEOUT rows (see Co-residency above) give NaN
 * overlap and TV, token -1 and a rejection (their entropy needs no exchange and
 * stays valid).  The acceptance ratio is formed in float64 from the float32 row
 * sums, and the inverse CDF's cumulative sums run in float64.
 * batch == 0 is a no-op.
 * Limits: 1 <= gamma <= MTP_MAX_GAMMA, 1 <= vocab <= 2^30, strides >= vocab.
 */
mtp_status mtp_verify_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                     size_t* bytes);

mtp_status mtp_verify(const void* target, int64_t target_row_stride,
                      const void* draft, int64_t draft_row_stride, mtp_dtype dtype,
                      int32_t batch, int32_t gamma, int32_t vocab,
                      const int32_t* draft_tokens, uint64_t seed, uint64_t offset,
                      uint8_t* accept, int32_t* accepted_len, int32_t* next_token,
                      int32_t* row_token, float* overlap, float* tv, float* entropy,
                      int32_t* row_status,
                      void* workspace, size_t workspace_bytes, void* stream);

/* mtp_verify without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Arguments, outputs and results are those of mtp_verify.  The
 * workspace is a file-scope device array of MTP_VERIFY_NOALLOC_SCRATCH_BYTES that
 * each GPU holds from the first call on it until the process ends; calls whose
 * workspace (mtp_verify_workspace_size) would be larger return MTP_ERR_WORKSPACE
 * and write nothing.  The call allocates and frees nothing.  The first call on a
 * device zeroes that device's array with a kernel on `stream` (it must not be
 * captured in a graph: MTP_ERR_DEVICE); every call leaves the array zeroed again.
 * All calls on one GPU share its array: calls that overlap on one GPU (other
 * streams, other host threads) race.
 */
#define MTP_VERIFY_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

mtp_status mtp_verify_noalloc(const void* target, int64_t target_row_stride,
                              const void* draft, int64_t draft_row_stride, mtp_dtype dtype,
                              int32_t batch, int32_t gamma, int32_t vocab,
                              const int32_t* draft_tokens, uint64_t seed, uint64_t offset,
                              uint8_t* accept, int32_t* accepted_len, int32_t* next_token,
                              int32_t* row_token, float* overlap, float* tv, float* entropy,
                              int32_t* row_status, void* stream);

/* The largest vocab that the verify entry points (all three) accept for dtype on
 * the current device: every row is cut into chunks of 4096 (bfloat16) or 3072
 * (float32) logits, one workgroup each, and all workgroups of a row must be
 * resident on the GPU at once.  Larger vocabularies return MTP_ERR_SHAPE from the
 * verify calls.  Queries the device (MTP_ERR_DEVICE without one).
 */
mtp_status mtp_verify_max_vocab(mtp_dtype dtype, int32_t* vocab);

/* ------------------------------------------------------------------------ */
/* Target-only verification with the rejection-sampling / target-only diagnostic
 * (paperlayer Sec. 2 "Preliminaries", acceptance methods; Sec. 7 "Discussion",
 * robustness of acceptance methods; App. D.2 "Target-Only Sampling").
 *
 * Each draft position proposes its greedy token instead of a sampled one:
 *   draft_token[b, k] = yhat = argmax_v q_v   (the smallest index among equal maxima)
 *   accept[b, k]      = u < p(yhat)
 *   p_yhat[b, k]      = p(yhat)
 *   rs_better[b, k]   = tv[b, k] < 1 - p(yhat): rejection sampling (acceptance
 *                       1 - TV) would accept more often than target-only sampling
 *   row_token[b, k]   = inverse-CDF sample of r = p with r_yhat = 0 (the residual of
 *                       the point-mass draft at yhat, so the emitted token's law is
 *                       p); if that has no mass (p(yhat) = 1), a sample of p with
 *                       MTP_ROW_RESIDUAL_EMPTY set; the bonus row samples p
 * and overlap, tv, entropy, accepted_len, next_token, row_status, u, u' exactly as
 * for mtp_verify.  Arguments as for mtp_verify without draft_tokens; draft_token
 * (device int32 [batch, gamma]) is a required output, p_yhat (float) and
 * rs_better (uint8) [batch, gamma] are optional.  Bad rows give draft_token -1, NaN
 * p_yhat, rs_better 0 and a rejection.  The workspace size differs from mtp_verify's.
 */
mtp_status mtp_verify_target_only_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                                 size_t* bytes);

mtp_status mtp_verify_target_only(const void* target, int64_t target_row_stride,
                                  const void* draft, int64_t draft_row_stride, mtp_dtype dtype,
                                  int32_t batch, int32_t gamma, int32_t vocab,
                                  uint64_t seed, uint64_t offset,
                                  uint8_t* accept, int32_t* accepted_len, int32_t* next_token,
                                  int32_t* draft_token, float* p_yhat, uint8_t* rs_better,
                                  int32_t* row_token, float* overlap, float* tv, float* entropy,
                                  int32_t* row_status,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Verification at a temperature with Gumbel-max sampling (paperlayer App. G.2
 * "Gumbel-Max Trick (vLLM)"; Sec. 2 acceptance methods).
 *
 * As mtp_verify with p = softmax(target row / T) and q = softmax(draft row / T)
 * (the temperature scales both), except for the row samples:
 *   row_token[b, k] = argmax_v (log r_v + g_v), r as for mtp_verify (an empty
 *                     residual samples p, MTP_ROW_RESIDUAL_EMPTY set), the smallest
 *                     index among equal keys;
 *   g_v = -log(-log U_v), U_v = ((w >> 8) + 1/2) * 2^-24 with w word v % 4 of the
 *         Philox4x32-10 block at key = seed, counter words (lo(c), hi(c),
 *         v / 4 + 1, 0), c = offset + b * (gamma + 1) + k.
 * u keeps mtp_verify's counter (third word 0), so acceptance uses the same
 * uniforms.  temperature must be positive and finite (else MTP_ERR_SHAPE);
 * T = 1 gives mtp_verify's accept flags and statistics.  Other arguments as for
 * mtp_verify; its own workspace size.
 */
mtp_status mtp_verify_gumbel_workspace_size(int32_t batch, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                            size_t* bytes);

mtp_status mtp_verify_gumbel(const void* target, int64_t target_row_stride,
                             const void* draft, int64_t draft_row_stride, mtp_dtype dtype,
                             int32_t batch, int32_t gamma, int32_t vocab,
                             const int32_t* draft_tokens, float temperature, uint64_t seed, uint64_t offset,
                             uint8_t* accept, int32_t* accepted_len, int32_t* next_token,
                             int32_t* row_token, float* overlap, float* tv, float* entropy,
                             int32_t* row_status,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Gumbel-max draft sampling (paperlayer App. G.2): for each of `rows` logit rows x
 * (device, dtype, row r at logits + r * row_stride elements),
 *   tokens[r] = argmax_v (x_v / T + g_v)   (a sample of softmax(x / T)),
 * g_v as for mtp_verify_gumbel with c = offset + r; the smallest index among
 * equal keys, -1 for a row with no finite key (all -inf or NaN logits).  tokens:
 * device int32 [rows].  workspace: device, 256-byte aligned, at least
 * mtp_gumbel_sample_workspace_size bytes (per-chunk partial maxima), left zeroed
 * on return like the verify workspaces, so one zeroed buffer serves both.
 * rows == 0 is a no-op.
 * Sampling draft rows (b, k) in row-major order with offset o and verifying with
 * an offset whose counters do not overlap [o, o + batch * gamma) keeps the two
 * noises independent.  rows * ceil(vocab / 8192) (bfloat16; / 4096 for float32)
 * must stay below 2^24.
 */
mtp_status mtp_gumbel_sample_workspace_size(int32_t rows, int32_t vocab, mtp_dtype dtype, size_t* bytes);

mtp_status mtp_gumbel_sample(const void* logits, int64_t row_stride, mtp_dtype dtype, int32_t rows,
                             int32_t vocab, float temperature, uint64_t seed, uint64_t offset,
                             int32_t* tokens, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* End-to-end TV loss, forward (paperlayer Sec. 4 "End-to-end TV loss", App. F;
 * rainbus "Method steps").  For position t and head k (1-based in the formula):
 *   alpha_{t,k} = clamp(sum_v min(p_v, q_v), 0, 1)
 *   S_{t,k}     = sum_v 1[q_v <= p_v] q_v
 *   pos_loss[t] = -sum_k prod_{j<=k} alpha_{t,j}
 *   loss[0]     = mean_t pos_loss[t]
 * with q = softmax(draft row (t, k)) and p = softmax(target row (t, k)).
 *
 * Row (t, k) of draft  starts at draft  + t*draft_pos_stride  + k*draft_head_stride.
 * Row (t, k) of target starts at target + t*target_pos_stride + k*target_head_stride;
 * target_head_stride = 0 shares one target row across the heads of a position.
 * Outputs (device float): loss [1] (required), pos_loss [T] (optional),
 *   saved [T, gamma, 4] = (ln-sum-exp of p, of q, alpha, S) (required; the
 *   backward consumes it).
 * Limits: T >= 1, 1 <= gamma <= MTP_MAX_GAMMA, 1 <= vocab <= 2^30.
 * -inf logits are allowed (masking).  A head whose target or draft row has no
 * finite normaliser (all -inf, or a NaN) is a data error: its alpha and S are NaN,
 * and so are its position's loss and the mean.
 * Each logit is read once when a position has at most 5 rows (a shared target with
 * gamma <= 4, or per-head targets with gamma <= 2) and the GPU can hold every chunk
 * of a row at once (vocab up to ~2M bf16 logits on MI355X); otherwise twice (two
 * streaming passes).  The results agree within the statistic tolerances either way;
 * the indicator of S is then taken on float32 probabilities rather than logits.
 * Workspace: mtp_tv_loss_workspace_size bytes for the same T, gamma, vocab, dtype
 * and sharing (it covers both forms), zeroed once and left zeroed by every call.
 */
mtp_status mtp_tv_loss_workspace_size(int32_t T, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                      int32_t shared_target, size_t* bytes);

mtp_status mtp_tv_loss_fwd(const void* target, int64_t target_pos_stride, int64_t target_head_stride,
                           const void* draft, int64_t draft_pos_stride, int64_t draft_head_stride,
                           mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab,
                           float* loss, float* pos_loss, float* saved,
                           void* workspace, size_t workspace_bytes, void* stream);

/* End-to-end TV loss, backward (paperlayer App. A; rainbus "Technical novelty").
 * p is detached: only the draft logits get a gradient.
 *   grad[t, k, v] = w_{t,k} q_v (1[q_v <= p_v] - S_{t,k}),
 *   w_{t,k} = -(g / T) sum_{m>=k} prod_{i<=m, i!=k} alpha_{t,i},   g = grad_loss[0].
 * The indicator is evaluated as z_v - x_v <= lnZ_q - lnZ_p on the logits, with
 * the forward's saved statistics.  grad_dtype MTP_BF16 rounds to nearest even;
 * MTP_F32 keeps the float32 value.
 * saved: device float [T, gamma, 4] from mtp_tv_loss_fwd on the same inputs.
 * grad_loss: device float [1].
 * grad: device, grad_dtype, row (t, k) at grad + t*grad_pos_stride + k*grad_head_stride,
 *   16-byte aligned rows.  Needs no workspace.
 */
mtp_status mtp_tv_loss_bwd(const void* target, int64_t target_pos_stride, int64_t target_head_stride,
                           const void* draft, int64_t draft_pos_stride, int64_t draft_head_stride,
                           mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab,
                           const float* saved, const float* grad_loss,
                           void* grad, int64_t grad_pos_stride, int64_t grad_head_stride,
                           mtp_dtype grad_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* End-to-end TV loss, forward and backward in one sweep (paperlayer App. F "Fused
 * TV Loss Kernel": the backward reuses what the forward computed; rainbus "Method
 * steps": the fused kernel keeps the memory peak down), for when the upstream
 * gradient g = grad_loss[0] (device float [1]) is known before the call.
 * Outputs: loss, pos_loss, saved as mtp_tv_loss_fwd; grad as mtp_tv_loss_bwd with
 * the same g.  Each logit is read once and each gradient element written once;
 * the indicator of the gradient is the one S uses (on float32 probabilities), so
 * the saved statistics are exactly those the gradient was formed with.  Shapes
 * the one-sweep kernel does not take (more than 5 rows per position, gamma > 4, a
 * vocabulary whose chunks cannot all be resident, or gamma = 1 with bfloat16
 * logits and gradient, where the two calls are faster) run mtp_tv_loss_fwd then
 * mtp_tv_loss_bwd on the same workspace.  Arguments and limits as for those calls;
 * workspace: mtp_tv_loss_fwd_bwd_workspace_size bytes, zeroed once, left zeroed.
 */
mtp_status mtp_tv_loss_fwd_bwd_workspace_size(int32_t T, int32_t gamma, int32_t vocab, mtp_dtype dtype,
                                              int32_t shared_target, size_t* bytes);

mtp_status mtp_tv_loss_fwd_bwd(const void* target, int64_t target_pos_stride, int64_t target_head_stride,
                               const void* draft, int64_t draft_pos_stride, int64_t draft_head_stride,
                               mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab, const float* grad_loss,
                               float* loss, float* pos_loss, float* saved,
                               void* grad, int64_t grad_pos_stride, int64_t grad_head_stride,
                               mtp_dtype grad_dtype, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* End-to-end TV loss with top-K targets (paperlayer App. F "Fused TV Loss
 * Kernel": an optional top-K path keeps O(K) of the target instead of O(V)).
 *
 * The target of head k at position t is given by K entries, vocabulary indices
 * I_j = target_idx[t*topk_pos_stride + k*topk_head_stride + j] and logits
 * A_j = target_val[same] (topk_head_stride = 0: one set shared by all heads).  It
 * stands for the target truncated to those entries and renormalised,
 * p_j = exp(A_j - lse_A); q = softmax(draft row (t, k)) over all V.  Then
 *   alpha = clamp(sum_j min(p_j, q(I_j)), 0, 1),  S = sum_j 1[q(I_j) <= p_j] q(I_j),
 * and the loss, per-position losses and the gradient are those of
 * mtp_tv_loss_fwd / mtp_tv_loss_bwd with these alpha and S:
 *   dL/dz_v = w_{t,k} q_v (c_v - S),  c_v = #{j : I_j = v, q_v <= p_j}.
 * For distinct indices this is the full-vocabulary TV loss against the truncated
 * target.  An index outside [0, V) carries no mass; repeated indices count entry
 * by entry (each its own point mass).  saved[t, k, :] = (lse_A, lse_q, alpha, S).
 * A row with no finite normaliser (no entry in range, or a NaN / all -inf draft
 * row) gives NaN alpha and S.
 *
 * target_idx: device int32, target_val: device float32, both 4-byte aligned;
 * strides in entries.  Draft, dtype, T, gamma, vocab, strides, loss, pos_loss,
 * saved, grad and grad_dtype as for mtp_tv_loss_fwd / _bwd; 1 <= K <= 2^20.  The
 * forward needs a workspace of mtp_tv_topk_workspace_size bytes (zeroed once,
 * left zeroed); the backward needs none.  The forward reads the draft once
 * (plus the K entries); the backward reads it once and writes the gradient.
 */
mtp_status mtp_tv_topk_workspace_size(int32_t T, int32_t gamma, int32_t vocab, mtp_dtype dtype, size_t* bytes);

mtp_status mtp_tv_topk_fwd(const int32_t* target_idx, const float* target_val, int64_t topk_pos_stride,
                           int64_t topk_head_stride, int32_t K,
                           const void* draft, int64_t draft_pos_stride, int64_t draft_head_stride,
                           mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab,
                           float* loss, float* pos_loss, float* saved,
                           void* workspace, size_t workspace_bytes, void* stream);

mtp_status mtp_tv_topk_bwd(const int32_t* target_idx, const float* target_val, int64_t topk_pos_stride,
                           int64_t topk_head_stride, int32_t K,
                           const void* draft, int64_t draft_pos_stride, int64_t draft_head_stride,
                           mtp_dtype dtype, int32_t T, int32_t gamma, int32_t vocab,
                           const float* saved, const float* grad_loss,
                           void* grad, int64_t grad_pos_stride, int64_t grad_head_stride,
                           mtp_dtype grad_dtype, void* stream);

/* ------------------------------------------------------------------------ */
/* Error word of a workspace: non-zero if a kernel that used it hit its bounded
 * wait limit (the exchange of row statistics between workgroups did not complete
 * in time).  Copies the 32-bit word to host memory, synchronising `stream`.  The
 * word stays set until the caller clears it. */
mtp_status mtp_workspace_error(const void* workspace, uint32_t* host_word, void* stream);

/* Diagnostics: the bound on every wait for row statistics exchanged between
 * workgroups, in ticks of the GPU's 100 MHz constant clock (default 100000000 =
 * one second), for the calls launched after it is set (process-wide).  0 makes a
 * wait give up as soon as a record is missing, which exercises the failure
 * reporting described under Co-residency without stalling any kernel.  Returns
 * the previous bound. */
uint64_t mtp_set_wait_limit(uint64_t ticks);

/* Diagnostics: the number of 16-byte vectors per chunk of the persistent grids
 * (the verify calls, the single-read TV forward and mtp_tv_loss_fwd_bwd), for the
 * calls and workspace-size queries made after it is set (process-wide).  A chunk
 * is one workgroup's share of a row; by default it is the workgroup's full reach
 * (4096 bfloat16 or 3072 float32 logits for verify).  A smaller count, down to one
 * vector, spreads a short row over many workgroups, so that their exchange of row
 * statistics (records past the first 64 per row, many super-groups of few items,
 * workgroups covering their chunk in part) runs at small vocabularies; results
 * are the same up to rounding.  The co-residency bound applies to the chunk count,
 * so the largest vocabulary shrinks with the chunk (mtp_verify_max_vocab reports
 * it).  0 or a negative count restores the default.  Size workspaces after setting
 * it.  Returns the previous count (0 for the default). */
int32_t mtp_set_chunk_vectors(int32_t vectors);

const char* mtp_status_string(mtp_status s);
const char* mtp_last_error(void);
const char* mtp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTP_H */
