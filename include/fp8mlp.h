/* fp8mlp.h -- C ABI of libfp8mlp, the fused FP8 ReLU^2 MLP path for AMD
 * Instinct MI355X (gfx950 / CDNA4).
 *
 * What it computes (page titles and sections of the speedrun write-ups):
 *  - "A Retrospective on Our World Records" (Paradigma), Modded-NanoGPT Main
 *    Track: the MLP down-projection runs in FP8; the fused up-projection
 *    epilogue writes the BF16 post-activation for backward, an FP8 copy and a
 *    tiny partial-amax tensor, so the activation is never reread; the FP8
 *    scale at step t comes from amax(t-1) times a safety margin (delayed
 *    scaling); a transposed FP8 cache of W2 is refreshed after each optimizer
 *    update (an exact, non-delayed refresh is viable per its implementation
 *    notes); the BF16 backward is unchanged.
 *  - "NanoGPT Speedrun (Track 1)" (Recursive), "Changes vs Record #83": item 1,
 *    QKV / output projections in float8_e4m3 on the forward pass with weights
 *    stored transposed; item 4, the ReLU^2 MLP stores only post = relu(pre)^2
 *    and the backward rebuilds relu(pre) = sqrt(post).
 *
 * Conventions for every entry point:
 *  - Tensors are caller-owned DEVICE memory, row-major and contiguous.
 *    bf16 tensors are passed as uint16_t bit patterns, e4m3 tensors as uint8_t
 *    codes of the OCP E4M3FN format (largest finite 448, no infinities).
 *    Weights use the [out, in] layout: W1 [h, d], W2 [d, h].
 *  - Every tensor pointer must be 16-byte aligned.  Feature sizes must be
 *    positive multiples of 64 (the contraction sizes of the e4m3 GEMMs,
 *    multiples of 128); the token count M may be any value >= 0 (ragged
 *    tails are masked, M = 0 is a valid empty call).  The GEMM entry points
 *    also take feature sizes of at most 2^22 and weights of fewer than 2^31
 *    elements (the kernels address memory with 32-bit byte offsets); larger
 *    sizes return FP8MLP_E_SHAPE.
 *  - Scalars that change from step to step (amax, scales) live in device
 *    memory as fp32 so a training step never synchronises with the host.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and runs asynchronously.  The library never synchronises, never
 *    allocates or frees memory, and keeps no pointer after the call returns;
 *    buffers must stay alive until the stream has passed the enqueued work.
 *  - Every call returns FP8MLP_OK (0) or a negative status.  Arguments are
 *    validated on the host before anything is enqueued, so a call that
 *    returns an error has launched nothing (FP8MLP_E_HIP, a failed launch, is
 *    the exception: earlier kernels of the same call may have been enqueued).
 *  - Calls are stateless and may be issued from several threads; calls that
 *    share output or workspace buffers must be ordered by the caller.
 */
#ifndef FP8MLP_H
#define FP8MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8MLP_ABI_VERSION 1

enum {
  FP8MLP_OK = 0,
  FP8MLP_E_NULL = -1,      /* a required pointer is NULL */
  FP8MLP_E_SHAPE = -2,     /* a size is negative, zero where not allowed, not a multiple of 64, or too large */
  FP8MLP_E_ALIGN = -3,     /* a tensor pointer is not 16-byte aligned */
  FP8MLP_E_WORKSPACE = -4, /* workspace missing or smaller than the *_workspace() size */
  FP8MLP_E_ARCH = -5,      /* the current device is not gfx950 */
  FP8MLP_E_HIP = -6,       /* a HIP call failed; see fp8mlp_last_hip_error() */
  FP8MLP_E_ARG = -7        /* any other invalid argument (mode, dtype, margin) */
};
enum { FP8MLP_TRAIN_FP8 = 0, FP8MLP_EVAL_BF16 = 1 }; /* mlp_relu2_fwd mode */
enum { FP8MLP_F32 = 0, FP8MLP_BF16 = 1 };            /* amax_reduce dtype */

int fp8mlp_abi_version(void);
const char* fp8mlp_status_str(int status);
/* hipError_t value behind the last FP8MLP_E_HIP returned on this thread. */
int fp8mlp_last_hip_error(void);
/* Debug mode: with the environment variable FP8MLP_SYNC_CHECK=1, every launch
 * of the library waits for its stream (not under graph capture) and a kernel
 * that failed is reported as FP8MLP_E_HIP by the call that launched it;
 * fp8mlp_last_failed_kernel() then names that kernel (NULL if none failed on
 * this thread).  The name is a static string owned by the library. */
const char* fp8mlp_last_failed_kernel(void);

/* ------------------------------------------------------------------------
 * mlp_relu2_fwd -- one forward of the MLP block.
 *
 * TRAIN (mode FP8MLP_TRAIN_FP8), per "A Retrospective on Our World Records",
 * Main Track:
 *   pre    = X W1^T                      (bf16 MFMA, fp32 accumulate; never stored)
 *   post   = bf16(relu(pre)^2)           -> post [M, h]
 *   scale  = fp32(448 / fp32(margin * amax_prev))   (1 if that is not a
 *            positive finite number)     -> scale_out (if not NULL)
 *   post_q = e4m3(fp32(post * scale))    -> post_q [M, h]; round to nearest
 *            even, saturate to +-448
 *   partial[tile] = max(post over the tile), then amax_out = max(partial)
 *   Y      = bf16((post_q . W2t_q) * fp32(1/scale) * w2_inv_scale)   [M, d]
 *   The scale depends only on amax_prev (the previous step's amax_out), so
 *   quantisation happens inside the up-projection epilogue and the forward
 *   never waits for the current amax.
 * In TRAIN mode post may be NULL: then only post_q is written (the backward
 * is mlp_relu2_bwd_fp8post).
 * EVAL (mode FP8MLP_EVAL_BF16), per "NanoGPT Speedrun (Track 1)", "Approach"
 *   item 5 (bf16 at eval): post as above, Y = bf16(post W2^T) with the bf16 W2;
 *   post_q, W2t_q, w2_inv_scale and amax_prev are not read (may be NULL);
 *   amax_out is still produced.
 *
 * Arguments:
 *   X [M, d] bf16, W1 [h, d] bf16; d a multiple of 64, h a multiple of 64
 *   (EVAL) or 128 (TRAIN).
 *   W2t_q [h, d] e4m3: the transposed W2 cache (fp8_cast_transpose_w2);
 *   w2_inv_scale: device fp32, its dequantisation multiplier.
 *   W2 [d, h] bf16: read in EVAL mode only (may be NULL in TRAIN).
 *   amax_prev: device fp32, amax_out of the previous step.  margin: the
 *   safety margin (> 0, finite; 2 in the speedrun workload).
 *   amax_out: device fp32, required.  scale_out: device fp32 or NULL.
 *   In TRAIN mode amax_prev, amax_out and scale_out must be three distinct
 *   words (E_ARG otherwise): the launch writes amax_out and scale_out while
 *   it still reads amax_prev, so amax_t and amax_{t-1} need two buffers
 *   (swap them between steps).
 *   workspace: device memory of mlp_relu2_fwd_workspace(M, d, h) bytes.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ARCH, E_ARG, E_HIP.
 * ---------------------------------------------------------------------- */
size_t mlp_relu2_fwd_workspace(int64_t M, int64_t d, int64_t h);
int mlp_relu2_fwd(int mode, const uint16_t* X, const uint16_t* W1, const uint8_t* W2t_q,
                  const float* w2_inv_scale, const uint16_t* W2, const float* amax_prev, float margin,
                  uint16_t* post, uint8_t* post_q, float* amax_out, float* scale_out, uint16_t* Y,
                  int64_t M, int64_t d, int64_t h, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * mlp_relu2_fwd_noalloc -- mlp_relu2_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, kernels and
 * results as mlp_relu2_fwd, with no workspace argument.  The partial-amax
 * tensor lives in a scratch array inside the library, one per GPU, kept
 * until the process ends and shared by every call on that GPU; it needs
 * mlp_relu2_fwd_workspace(M, d, h) bytes, at most
 * mlp_relu2_fwd_noalloc_max_bytes() (256 KB: M * h up to about 4.3e9 with
 * 256 x 256 tiles), else FP8MLP_E_WORKSPACE.  Nothing in the scratch array
 * needs to start at zero (every entry a call reads, the same call writes
 * first).  The call allocates and frees nothing; its first call on a device
 * looks up the array's device address once.  Calls that overlap on one GPU
 * (on different streams, without ordering) race on the array.
 * Arguments and errors otherwise as mlp_relu2_fwd.
 * ---------------------------------------------------------------------- */
size_t mlp_relu2_fwd_noalloc_max_bytes(void);
int mlp_relu2_fwd_noalloc(int mode, const uint16_t* X, const uint16_t* W1, const uint8_t* W2t_q,
                          const float* w2_inv_scale, const uint16_t* W2, const float* amax_prev, float margin,
                          uint16_t* post, uint8_t* post_q, float* amax_out, float* scale_out, uint16_t* Y,
                          int64_t M, int64_t d, int64_t h, void* stream);

/* ------------------------------------------------------------------------
 * mlp_relu2_bwd -- the bf16 backward of the block, straight through the FP8
 * forward ("A Retrospective on Our World Records", Main Track: the BF16
 * backward path is left unchanged; "NanoGPT Speedrun (Track 1)", "Changes vs
 * Record #83" item 4: relu(pre) is rebuilt in-kernel as sqrt(post)).
 *   dpost = dY W2                         (never stored)
 *   dpre  = bf16(2 * sqrt(post) * dpost)  (kept in the workspace)
 *   dX    = bf16(dpre W1)                 -> dX [M, d] bf16
 *   dW1   = dpre^T X                      -> dW1 [h, d] fp32
 *   dW2   = dY^T post                     -> dW2 [d, h] fp32
 * accumulate = 0 overwrites dW1 / dW2, 1 adds into them.  The weight
 * gradients are summed over M in a fixed order (split-k partials reduced in
 * split order), so repeated calls give identical bits.
 * Arguments: dY [M, d] bf16, X [M, d] bf16, W1 [h, d] bf16, W2 [d, h] bf16,
 * post [M, h] bf16 (from mlp_relu2_fwd); workspace of
 * mlp_relu2_bwd_workspace(M, d, h) bytes.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ARCH, E_ARG, E_HIP.
 * ---------------------------------------------------------------------- */
size_t mlp_relu2_bwd_workspace(int64_t M, int64_t d, int64_t h);
int mlp_relu2_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* W1, const uint16_t* W2,
                  const uint16_t* post, uint16_t* dX, float* dW1, float* dW2, int accumulate, int64_t M,
                  int64_t d, int64_t h, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * mlp_relu2_bwd_fp8post -- the backward when the forward kept only the e4m3
 * copy of post (mlp_relu2_fwd / mlp_relu2_fwd_fp8up in TRAIN mode with post
 * = NULL).  "A Retrospective on Our World Records", Main Track: the BF16 post
 * stays materialised there by choice; dropping it, and rebuilding what the
 * backward needs from the FP8 copy, is the orthogonal variant the page
 * points to.  post's place is taken by
 *   post_hat = fp32(dec(post_q) * fp32(1 / *post_scale))
 *   dpre = bf16(2 * sqrt(post_hat) * dpost),  dpost = dY W2
 *   dW2  = (dY^T dec(post_q)) * fp32(1 / *post_scale)   (fp32 accumulate)
 *   dX, dW1 as in mlp_relu2_bwd.
 * post_q [M, h] e4m3 and post_scale (device fp32: the scale_out of that
 * forward) replace post; everything else, including the workspace
 * (mlp_relu2_bwd_workspace), is as in mlp_relu2_bwd.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ARCH, E_ARG, E_HIP.
 * ---------------------------------------------------------------------- */
int mlp_relu2_bwd_fp8post(const uint16_t* dY, const uint16_t* X, const uint16_t* W1, const uint16_t* W2,
                          const uint8_t* post_q, const float* post_scale, uint16_t* dX, float* dW1, float* dW2,
                          int accumulate, int64_t M, int64_t d, int64_t h, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * fp8_cast_transpose -- bf16 weight W [N, K] -> e4m3 Wt_q [K, N] (the
 * transposed FP8 weight cache of "A Retrospective on Our World Records",
 * Main Track, and of "NanoGPT Speedrun (Track 1)", "Changes vs Record #83"
 * item 1) with one per-tensor scale:
 *   amax  = max |W|                        -> amax_out (if not NULL)
 *   scale = *scale_in if scale_in is not NULL, else fp32(448 / amax)
 *           (the exact, non-delayed refresh; 1 if amax is 0 or not finite)
 *   Wt_q[k, n] = e4m3(fp32(W[n, k] * scale))   RNE, saturating, sign kept
 *   scale -> scale_out, fp32(1 / scale) -> inv_scale_out (each if not NULL)
 * N and K: positive multiples of 16.  workspace: fp8_cast_transpose_workspace
 * (N, K) bytes (used for the amax reduction).
 * fp8_cast_transpose_w2 is the same call on W2 [d, h] -> W2t_q [h, d] with the
 * exact scale, to be run after every update of W2.
 * ---------------------------------------------------------------------- */
size_t fp8_cast_transpose_workspace(int64_t N, int64_t K);
int fp8_cast_transpose(const uint16_t* W, int64_t N, int64_t K, uint8_t* Wt_q, const float* scale_in,
                       float* scale_out, float* inv_scale_out, float* amax_out, void* workspace,
                       size_t workspace_bytes, void* stream);
int fp8_cast_transpose_w2(const uint16_t* W2, int64_t d, int64_t h, uint8_t* W2t_q, float* scale_out,
                          float* inv_scale_out, float* amax_out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------
 * amax_reduce -- amax_out = max |x[i]| over n elements of fp32 (dtype
 * FP8MLP_F32) or bf16 (FP8MLP_BF16) data; 0 for n = 0; NaN if any element is
 * NaN.  The per-tensor amax that sets an FP8 scale ("A Retrospective on Our
 * World Records", Main Track: the partial-amax values are reduced later).
 * The maximum is taken on the bit patterns of |x|, so it is exact and
 * independent of the reduction order.  workspace: amax_reduce_workspace(n).
 * ---------------------------------------------------------------------- */
size_t amax_reduce_workspace(int64_t n);
int amax_reduce(int dtype, const void* x, int64_t n, float* amax_out, void* workspace, size_t workspace_bytes,
                void* stream);

/* ------------------------------------------------------------------------
 * fp8_scale_from_amax -- device-side scale for an FP8 tensor:
 *   scale = fp32(448 / fp32(margin * *amax)), 1 if that is not a positive
 *   finite number; inv_scale = fp32(1 / scale).
 * margin 1 gives the exact per-tensor scale, margin > 1 with the previous
 * step's amax the delayed scale ("A Retrospective on Our World Records",
 * Main Track).  scale_out / inv_scale_out: device fp32 (either may be NULL).
 * ---------------------------------------------------------------------- */
int fp8_scale_from_amax(const float* amax, float margin, float* scale_out, float* inv_scale_out, void* stream);

/* ------------------------------------------------------------------------
 * fp8_saturation_count -- clip-rate telemetry for a delayed scale ("A
 * Retrospective on Our World Records", Main Track: the scale from amax(t-1)
 * times a safety margin; the margin bounds how far the activation may grow
 * in one step before the e4m3 copy clips):
 *   count_out = number of codes among q[0 .. n) of magnitude 448 (0x7E, 0xFE)
 * 448 is the top e4m3 code: every scaled value from 432 up receives it, and
 * values above 464 would not fit at all (saturated), so the count bounds the
 * clipped share from above and is 0 whenever nothing came near the limit.
 * q: device e4m3 codes, n a multiple of 16 (0 gives 0).  count_out: device
 * uint64, 8-byte aligned.  workspace: fp8_saturation_count_workspace(n) bytes.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ARCH, E_HIP.
 * ---------------------------------------------------------------------- */
size_t fp8_saturation_count_workspace(int64_t n);
int fp8_saturation_count(const uint8_t* q, int64_t n, uint64_t* count_out, void* workspace, size_t workspace_bytes,
                         void* stream);

/* ------------------------------------------------------------------------
 * fp8_linear -- forward of an FP8 projection ("NanoGPT Speedrun (Track 1)",
 * "Changes vs Record #83" item 1: QKV and output projections in e4m3 on the
 * forward pass, weights stored transposed):
 *   Xq = e4m3(fp32(X * *x_scale))        (RNE, saturating; kept in the workspace)
 *   Y  = bf16((Xq . Wt_q) * fp32(1 / *x_scale) * *w_inv_scale)
 * X [M, K] bf16, Wt_q [K, N] e4m3 (from fp8_cast_transpose), Y [M, N] bf16.
 * x_scale, w_inv_scale: device fp32.  x_amax_out: device fp32 or NULL; if
 * given it receives max |X| (for the next step's delayed scale); it must not
 * be x_scale or w_inv_scale (E_ARG), which the same launch still reads.
 * K and N: positive multiples of 64; M >= 0.  For K <= 768 one launch
 * converts each row of X inside the GEMM and keeps the codes on chip; for
 * larger K a conversion pass writes the e4m3 copy of X to the workspace
 * first.  Both give the same Y.
 * workspace: fp8_linear_workspace(M, K) bytes (room for the e4m3 copy of X,
 * its rows padded with zero codes to a multiple of 128, used when K > 768,
 * and for the per-block maxima of |X|).
 * ---------------------------------------------------------------------- */
size_t fp8_linear_workspace(int64_t M, int64_t K);
int fp8_linear(const uint16_t* X, const float* x_scale, const uint8_t* Wt_q, const float* w_inv_scale,
               uint16_t* Y, float* x_amax_out, int64_t M, int64_t K, int64_t N, void* workspace,
               size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * mlp_relu2_fwd_fp8up -- the TRAIN forward of mlp_relu2_fwd with the
 * up-projection in e4m3 as well ("NanoGPT Speedrun (Track 1)", "From
 * Unoptimized", "Approach" item 5: both MLP GEMMs in e4m3 on the training
 * forward; bf16 backward, bf16 at eval):
 *   Xq     = e4m3(fp32(X * *x_scale))          (RNE, saturating; in the workspace)
 *   pre    = fp32(fp32(acc * fp32(1 / *x_scale)) * *w1_inv_scale),
 *            acc = Xq . W1t_q in fp32           (never stored)
 *   post, post_q, partial amax, amax_out, scale_out and Y exactly as in
 *   mlp_relu2_fwd TRAIN (the delayed scale of post from amax_prev, margin).
 * The pages do not say how X is scaled; x_scale is a per-tensor multiplier the
 * caller supplies on the device (e.g. fp8_scale_from_amax of the previous
 * step's x_amax_out with a margin, as for post).
 * Arguments: X [M, d] bf16; W1t_q [d, h] e4m3, the transposed W1 cache
 * (fp8_cast_transpose of W1 [h, d]) with its dequantisation multiplier
 * w1_inv_scale; W2t_q / w2_inv_scale as in mlp_relu2_fwd.  x_amax_out:
 * device fp32 or NULL; if given it receives max |X|.  amax_prev, amax_out,
 * scale_out and x_amax_out must be distinct words, and x_amax_out must not
 * be x_scale (E_ARG otherwise; see mlp_relu2_fwd).  d and h: multiples of
 * 128; M >= 0.  workspace: mlp_relu2_fwd_fp8up_workspace(M, d, h) bytes
 * (the partial amax tensor, per-block maxima of |X| and the e4m3 copy of X;
 * 0 for M = 0).  The backward is
 * mlp_relu2_bwd with the bf16 W1 / W2 and the post written here (post may be
 * NULL: then mlp_relu2_bwd_fp8post on post_q).
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ARCH, E_ARG, E_HIP.
 * ---------------------------------------------------------------------- */
size_t mlp_relu2_fwd_fp8up_workspace(int64_t M, int64_t d, int64_t h);
int mlp_relu2_fwd_fp8up(const uint16_t* X, const float* x_scale, const uint8_t* W1t_q, const float* w1_inv_scale,
                        const uint8_t* W2t_q, const float* w2_inv_scale, const float* amax_prev, float margin,
                        uint16_t* post, uint8_t* post_q, float* amax_out, float* scale_out, uint16_t* Y,
                        float* x_amax_out, int64_t M, int64_t d, int64_t h, void* workspace, size_t workspace_bytes,
                        void* stream);

/* ------------------------------------------------------------------------
 * softcap_ce_fwd_bwd -- fused softcapped cross-entropy over a language-model
 * head, forward and backward ("NanoGPT Speedrun (Track 1)", "From
 * Unoptimized", "Approach" item 5: a fused softcapped cross-entropy that never
 * materialises the [M, V] logits in fp32; "A Retrospective on Our World
 * Records", SlowRun part: one head trained against several successive
 * targets per position).  The pages give no formula; this computes
 *   z = X W^T (fp32 accumulate, never stored), z' = c tanh(z / c) (z if c = 0)
 *   lse_m = log sum_v exp(z'[m, v])
 *   loss = (1/M) sum_m sum_j w_j (lse_m - z'[m, t[m, j]])   -> loss_out
 *   G = bf16((dloss/M) (wsum_m softmax(z')[m, v] - sum_j w_j [v == t[m, j]])
 *            (1 - (z'/c)^2)),   wsum_m = sum of w_j over the row's targets
 *   dX = bf16(G W)                                          -> dX [M, d]
 *   dW = G^T X (fp32)                                       -> dW [V, d]
 * in two passes over the head GEMM (row statistics, then G) and two GEMMs.
 * Arguments: X [M, d] bf16, W [V, d] bf16; targets [M, T] int32, T in 1..4
 * (a target < 0 or >= V is no target); weights [T] fp32 (device); softcap c
 * >= 0 (0: none); dloss: device fp32 scalar or NULL (1).  loss_out: device
 * fp32; lse_out: device fp32 [M] or NULL.  accumulate = 1 adds into dW.
 * V and d: multiples of 64; M >= 0 (M = 0: loss 0, dW zeroed unless
 * accumulating).  workspace: softcap_ce_workspace(M, V, d, T) bytes; on
 * return it begins with G ([M, V] bf16, row-major).
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ARCH, E_ARG, E_HIP.
 * ---------------------------------------------------------------------- */
size_t softcap_ce_workspace(int64_t M, int64_t V, int64_t d, int T);
int softcap_ce_fwd_bwd(const uint16_t* X, const uint16_t* W, const int32_t* targets, int T, const float* weights,
                       float softcap, const float* dloss, float* loss_out, float* lse_out, uint16_t* dX, float* dW,
                       int accumulate, int64_t M, int64_t V, int64_t d, void* workspace, size_t workspace_bytes,
                       void* stream);

/* ------------------------------------------------------------------------
 * softcap_ce_fwd_bwd_fp8 -- the same loss and gradients with the head in e4m3
 * ("A Retrospective on Our World Records", SlowRun part: the fused FP8
 * soft-capped cross-entropy):
 *   z = (e4m3(fp32(X * *x_scale)) . Wt_q) * fp32(1 / *x_scale) * *w_inv_scale
 * (fp32 accumulate), then everything as in softcap_ce_fwd_bwd; dX = bf16(G W)
 * and dW = G^T X use the bf16 X and W.  Wt_q [d, V] e4m3 is the transposed
 * cache of W (fp8_cast_transpose of W [V, d]) with its dequantisation
 * multiplier w_inv_scale; x_scale: device fp32.  d: a multiple of 128.
 * workspace: softcap_ce_fp8_workspace(M, V, d, T) bytes (it begins with G).
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_WORKSPACE, E_ARCH, E_ARG, E_HIP.
 * ---------------------------------------------------------------------- */
size_t softcap_ce_fp8_workspace(int64_t M, int64_t V, int64_t d, int T);
int softcap_ce_fwd_bwd_fp8(const uint16_t* X, const float* x_scale, const uint8_t* Wt_q, const float* w_inv_scale,
                           const uint16_t* W, const int32_t* targets, int T, const float* weights, float softcap,
                           const float* dloss, float* loss_out, float* lse_out, uint16_t* dX, float* dW,
                           int accumulate, int64_t M, int64_t V, int64_t d, void* workspace, size_t workspace_bytes,
                           void* stream);

/* ------------------------------------------------------------------------
 * Layer-stack helpers.  The speedrun pages train the MLP block inside a
 * pre-norm transformer and carry its FP8 state per layer from step to step
 * ("A Retrospective on Our World Records", Main Track: delayed scaling from
 * amax(t-1); the transposed FP8 W2 cache refreshed after each optimizer
 * update).  These calls let the block be trained as a stack
 * x <- x + MLP(rmsnorm(x)); the pages give no formulas for them, so they
 * follow the plain textbook definitions (weightless RMSNorm, SGD):
 *
 * rmsnorm_fwd:  per row of x [M, d] bf16:
 *     r = 1 / sqrt(sum_j(x_j^2) / d + eps)   (fp32; -> inv_rms [M] fp32)
 *     xn = bf16(x * r)                       (-> xn [M, d] bf16)
 * rmsnorm_bwd:  per row, given dxn = dL/dxn [M, d] bf16 and the stream
 *   gradient g_in [M, d] bf16 of the residual that bypasses the block:
 *     xh = x * r;  dx = r * (dxn - xh * sum_j(dxn_j xh_j) / d)
 *     g_out = bf16(g_in + dx)                (g_out may alias g_in)
 * add_bf16:     out[i] = bf16(a[i] + b[i])   (the residual add; out may
 *   alias a or b)
 * sgd_update_bf16:  W[i] = bf16(fp32(W[i] - fp32(lr * dW[i]))), in place,
 *   W bf16, dW fp32 (the weight gradients of mlp_relu2_bwd)
 * Sizes: d and n multiples of 8; M >= 0 and n >= 0 (0 launches nothing).
 * Pointers 16-byte aligned (inv_rms 4-byte aligned).  eps >= 0.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_ARCH, E_ARG, E_HIP.
 * ---------------------------------------------------------------------- */
int rmsnorm_fwd(const uint16_t* x, uint16_t* xn, float* inv_rms, int64_t M, int64_t d, float eps, void* stream);
int rmsnorm_bwd(const uint16_t* x, const float* inv_rms, const uint16_t* dxn, const uint16_t* g_in, uint16_t* g_out,
                int64_t M, int64_t d, void* stream);
int add_bf16(const uint16_t* a, const uint16_t* b, uint16_t* out, int64_t n, void* stream);
int sgd_update_bf16(uint16_t* W, const float* dW, int64_t n, float lr, void* stream);

/* ------------------------------------------------------------------------
 * fp8mlp_mfma_probe -- matrix-core rate probe (a measurement aid, not part of
 * the method).  The published MI355X peaks assume the boost clock; under a
 * dense MFMA load the clock falls with the switching activity of the
 * operands, so the benchmark measures the rate the chip sustains on its own
 * data.  Launches FP8MLP_PROBE_BLOCKS blocks of 4 waves; every wave loads 4 + 4
 * operand fragments from a and b (read modulo a_bytes / b_bytes) and issues
 * iters rounds of 16 independent 32x32 MFMAs:
 *   FP8MLP_MFMA_BF16: v_mfma_f32_32x32x16_bf16, 32768 flop each;
 *   FP8MLP_MFMA_E4M3: v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, unit scales),
 *                     131072 flop each.
 * Flop per call = FP8MLP_PROBE_BLOCKS * 4 * 16 * iters * (flop per MFMA).
 * sink: device fp32 [FP8MLP_PROBE_BLOCKS * 256], overwritten.  a, b: device,
 * 16-byte aligned, at least 16 bytes.  1 <= iters <= 2^24.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_ARCH, E_ARG, E_HIP.
 * ---------------------------------------------------------------------- */
enum { FP8MLP_MFMA_BF16 = 0, FP8MLP_MFMA_E4M3 = 1 };
#define FP8MLP_PROBE_BLOCKS 256
int fp8mlp_mfma_probe(int dtype, const void* a, int64_t a_bytes, const void* b, int64_t b_bytes, int64_t iters,
                      float* sink, void* stream);

/* ------------------------------------------------------------------------
 * Per-kernel timing (benchmarking / profiling aid, not part of the method).
 * fp8mlp_timing_start(capacity) creates up to `capacity` hipEvent pairs
 * (driver objects, no device memory) and, until fp8mlp_timing_stop(), brackets
 * every kernel this library launches from the calling thread with
 * hipEventRecord on that kernel's stream.  fp8mlp_timing_stop() returns the
 * number of kernels recorded; launches beyond `capacity` are not recorded
 * and are counted by fp8mlp_timing_dropped().  After the streams have been
 * synchronised, fp8mlp_timing_get(i, &name, &ms) returns the i-th kernel's
 * name (a static string) and duration in milliseconds.  State is per thread;
 * a new fp8mlp_timing_start() discards the previous records.
 * ---------------------------------------------------------------------- */
int fp8mlp_timing_start(int capacity);
int fp8mlp_timing_stop(void);
int fp8mlp_timing_get(int i, const char** name, float* ms);
int fp8mlp_timing_dropped(void);

#ifdef __cplusplus
}
#endif
#endif /* FP8MLP_H */
