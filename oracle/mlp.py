"""The fused FP8 ReLU^2 MLP path, step by step, in float64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
imports this module.

Sources (cited by page title and section):
  [R]  "A Retrospective on Our World Records" (Paradigma), Modded-NanoGPT Main
       Track part: the FP8 down-projection, the fused up-projection epilogue
       (bf16 post for backward + fp8 copy + tiny partial-amax tensor), delayed
       scaling from amax(t-1) times a safety margin, the transposed fp8 W2
       cache refreshed after optimizer updates, the unchanged bf16 backward,
       and the implementation-notes bullets (exact W2 refresh is viable;
       bf16 post stays materialised; amax(t-1) instead of a rolling window).
  [S]  "NanoGPT Speedrun (Track 1)" (Recursive), "Changes vs Record #83":
       item 1, FP8 e4m3 QKV / output projections on the forward pass with
       bf16 backward; item 4, the ReLU^2 MLP kernel that stores only
       post = relu(pre)^2 and rebuilds relu(pre) = sqrt(post) in backward.

Conventions: tensors are row-major; weights use the [out, in] layout
(W1 [h, d], W2 [d, h]); bf16 tensors are passed as uint16 bit patterns,
e4m3 tensors as uint8 codes, fp32 scalars as Python floats.  ``rnd`` arguments
default to the bf16 rounding the method applies; passing ``exact`` removes
every rounding so the same code can be checked against plain calculus.
"""
import numpy as np

from .formats import (E4M3_MAX, bf16, bf16_round, bf16_to_f64, e4m3_decode,
                      e4m3_encode, fl32)


def exact(x):
    """No rounding at all (used to pin the algebra against calculus)."""
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# amax and scales
# --------------------------------------------------------------------------
def amax(x):
    """max |x| over all elements, exact.  NaN if any element is NaN, 0 if empty.

    [R]: the per-tensor amax that sets the fp8 scale.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return 0.0
    a = np.abs(x)
    if np.isnan(a).any():
        return float("nan")
    return float(a.max())


def delayed_scale(amax_prev, margin):
    """Quantisation multiplier at step t from the amax measured at step t-1.

    [R] delayed-scaling paragraph: the scale at step t comes from amax(t-1)
    multiplied by a safety margin.  Reading: scale = 448 / (margin * amax_prev)
    with both the product and the quotient rounded to fp32 (the kernel's
    arithmetic).  The product of two fp32 values is exact in float64, so
    ``fl32`` rounds it once; the float64 quotient followed by ``fl32`` equals
    the correctly rounded fp32 quotient (53 >= 2*24 + 2).
    Guard: a non-positive or non-finite denominator, or a quotient that
    overflows fp32, gives scale 1.
    """
    denom = float(fl32(np.float64(np.float32(margin)) * np.float64(np.float32(amax_prev))))
    if not (np.isfinite(denom) and denom > 0.0):
        return 1.0
    s = float(fl32(E4M3_MAX / denom))
    if not np.isfinite(s):
        return 1.0
    return s


def exact_scale(amax_w):
    """Non-delayed per-tensor weight scale: 448 / max|W| in fp32, guard -> 1.

    [R] implementation notes: an exact, non-delayed refresh of the W2 cache is
    viable because W2 is small; margin 1.
    """
    return delayed_scale(amax_w, 1.0)


def inv_scale(scale):
    """Dequantisation multiplier fl32(1 / scale)."""
    return float(fl32(1.0 / np.float64(np.float32(scale))))


def window_scale(amax_history, margin):
    """Rolling-window variant of the delayed scale: the scale of the largest
    amax among the last L steps ([R] delayed-scaling paragraph names the
    rolling window as the alternative to amax(t-1); L = 1 is amax(t-1)).
    NaN anywhere in the window propagates, as in ``amax``."""
    return delayed_scale(amax(np.asarray(amax_history, dtype=np.float64)), margin)


def saturation_count(codes):
    """Number of e4m3 codes whose value has magnitude 448 (the top code):
    the clip-rate telemetry of a delayed scale."""
    v = e4m3_decode(np.asarray(codes, dtype=np.uint8))
    return int(np.count_nonzero(np.abs(v) == E4M3_MAX))


# --------------------------------------------------------------------------
# weight cache: cast + transpose
# --------------------------------------------------------------------------
def cast_transpose(W_bits, scale_in=None):
    """bf16 W [N, K] -> e4m3 W^T [K, N] with a per-tensor scale.

    [R]: the transposed FP8 cache of W2 refreshed after each optimizer
    update; [S] item 1: QKV / O weights stored transposed in e4m3.
    With ``scale_in`` None the scale is exact (448 / max|W|).
    Returns (codes [K, N] uint8, scale, inv_scale, amax_w).
    """
    W = bf16_to_f64(W_bits)
    a = amax(W)
    s = exact_scale(a) if scale_in is None else float(np.float32(scale_in))
    codes = e4m3_encode(fl32(W * s))
    return np.ascontiguousarray(codes.T), s, inv_scale(s), a


def delayed_cast_transpose(W_bits, amax_w_prev, margin):
    """Delayed-scale variant of the weight-cache refresh: the scale comes from
    the previous refresh's max|W| times a margin instead of the exact max|W|
    of the weights being cast ([R] implementation notes: the exact refresh is
    the viable choice because W2 is small; this is the alternative).
    Returns (codes, scale, inv_scale, amax of the new W)."""
    return cast_transpose(W_bits, scale_in=delayed_scale(amax_w_prev, margin))


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def up_relu2(X_bits, W1_bits, rnd=bf16):
    """post = relu(X W1^T)^2, rounded once to bf16.  [S] item 4; [R]."""
    X = bf16_to_f64(X_bits)
    W1 = bf16_to_f64(W1_bits)
    pre = X @ W1.T
    r = np.maximum(pre, 0.0)
    return rnd(r * r)


def quantize(post, scale):
    """e4m3 copy of the stored bf16 post: e4m3(fl32(post * scale)).

    [R] fused epilogue: the fp8 version is emitted from the values the kernel
    holds.  Reading: the quantiser sees the bf16-rounded post (the tensor the
    backward also reads); bf16 * fp32 is exact in float64, so fl32 rounds once.
    """
    return e4m3_encode(fl32(np.asarray(post, dtype=np.float64) * scale))


def tile_amax(post, bm, bn):
    """Per-tile maxima of post over a (bm x bn) tiling: the partial-amax
    tensor of [R] ("a tiny partial-amax tensor"), shape [ceil(M/bm), ceil(N/bn)]."""
    post = np.asarray(post, dtype=np.float64)
    M, N = post.shape
    tm, tn = -(-M // bm), -(-N // bn)
    out = np.zeros((tm, tn))
    for i in range(tm):
        for j in range(tn):
            out[i, j] = amax(post[i * bm:(i + 1) * bm, j * bn:(j + 1) * bn])
    return out


def down_fp8(q_codes, Wt_codes, inv_sx, inv_sw, rnd=bf16):
    """FP8 x FP8 scaled matmul: y = (dec(q) dec(Wt)) * inv_sx * inv_sw.

    [R]: the down-projection runs as an FP8 scaled matmul on both operands.
    Every e4m3 value is a multiple of 2^-9 with 4 significant bits, so each
    product is a multiple of 2^-18 below 2^18 and a sum of fewer than 2^17 of
    them is exact in float64 in any order: ``acc`` is the exact dot product.
    """
    acc = e4m3_decode(q_codes) @ e4m3_decode(Wt_codes)
    return rnd(acc * inv_sx * inv_sw)


def mlp_fwd(X_bits, W1_bits, W2t_codes, w2_inv_scale, amax_prev, margin,
            mode="train", W2_bits=None, post_bits=None):
    """One forward of the MLP block for one step.

    train: post (bf16) -> amax(post) -> q = e4m3 with the delayed scale ->
           y = fp8 GEMM against the transposed W2 cache.
    eval:  post (bf16) -> y = bf16(post W2^T) in bf16, no fp8
           ([S] item 1 and "Approach" item 5: bf16 at eval).
    ``post_bits`` lets a test feed the GPU's own bf16 post to the quantiser.
    Returns a dict of uint16 / uint8 arrays and float scalars.
    """
    if post_bits is None:
        post_bits = bf16_round(up_relu2(X_bits, W1_bits))
    post = bf16_to_f64(post_bits)
    out = {"post": post_bits, "amax": amax(post)}
    if mode == "train":
        s = delayed_scale(amax_prev, margin)
        q = quantize(post, s)
        y = down_fp8(q, W2t_codes, inv_scale(s), w2_inv_scale)
        out.update(post_q=q, scale=s, y=bf16_round(y))
    else:
        W2 = bf16_to_f64(W2_bits)
        out.update(y=bf16_round(post @ W2.T))
    return out


def up_relu2_fp8(X_bits, x_scale, W1t_codes, w1_inv_scale, rnd=bf16):
    """post = relu(pre)^2 with the up-projection in e4m3 as well.

    [S] "From Unoptimized", "Approach" item 5: both MLP GEMMs run in e4m3 on
    the training forward.  The pages do not say how X is scaled; reading: a
    per-tensor multiplier sx supplied by the caller, as for the attention
    projections ([S] item 1), with W1 held transposed in e4m3 like W2:
      Xq  = e4m3(fl32(X * sx))
      acc = dec(Xq) dec(W1t)        (exact in float64, as in ``down_fp8``)
      pre = acc * fl32(1/sx) * w1_inv_scale
      post = rnd(relu(pre)^2)
    Returns (post, Xq codes, pre), post rounded by ``rnd``, pre unrounded.
    """
    X = bf16_to_f64(X_bits)
    sx = float(np.float32(x_scale))
    xq = e4m3_encode(fl32(X * sx))
    acc = e4m3_decode(xq) @ e4m3_decode(W1t_codes)
    pre = acc * inv_scale(sx) * float(np.float32(w1_inv_scale))
    r = np.maximum(pre, 0.0)
    return rnd(r * r), xq, pre


def mlp_fwd_fp8up(X_bits, x_scale, W1t_codes, w1_inv_scale, W2t_codes, w2_inv_scale, amax_prev, margin,
                  post_bits=None):
    """The training forward with both GEMMs in e4m3 ([S] "Approach" item 5):
    ``up_relu2_fp8``, then the same delayed-scale quantisation, partial amax
    and FP8 down-projection as ``mlp_fwd`` in train mode.  ``post_bits``
    lets a test feed the GPU's own bf16 post to the later steps."""
    xq = None
    if post_bits is None:
        post, xq, _ = up_relu2_fp8(X_bits, x_scale, W1t_codes, w1_inv_scale)
        post_bits = bf16_round(post)
    out = mlp_fwd(X_bits, None, W2t_codes, w2_inv_scale, amax_prev, margin, post_bits=post_bits)
    out.update(xq=xq, x_amax=amax(bf16_to_f64(X_bits)))
    return out


# --------------------------------------------------------------------------
# backward (bf16 path, straight through the fp8 forward)
# --------------------------------------------------------------------------
def mlp_bwd(dY_bits, X_bits, W1_bits, W2_bits, post, rnd=bf16):
    """Backward of y = relu(X W1^T)^2 W2^T with the bf16 master weights.

    [R]: the existing bf16 backward is left unchanged (the fp8 copies are
    forward-only).  [S] item 4: relu(pre) is rebuilt as sqrt(post), so
    d post / d pre = 2 relu(pre) = 2 sqrt(post).

      dpost = dY W2                 [M, h]
      dpre  = rnd(2 sqrt(post) dpost)
      dW2   = dY^T post             [d, h]
      dW1   = dpre^T X              [h, d]
      dX    = rnd(dpre W1)          [M, d]
    ``post`` is a float64 array (the stored bf16 post, decoded).
    Returns float64 arrays (dX, dpre rounded by ``rnd``; dW1, dW2 unrounded).
    """
    dY = bf16_to_f64(dY_bits)
    X = bf16_to_f64(X_bits)
    W1 = bf16_to_f64(W1_bits)
    W2 = bf16_to_f64(W2_bits)
    post = np.asarray(post, dtype=np.float64)
    dpost = dY @ W2
    dpre = rnd(2.0 * np.sqrt(post) * dpost)
    dW2 = dY.T @ post
    dW1 = dpre.T @ X
    dX = rnd(dpre @ W1)
    return {"dX": dX, "dW1": dW1, "dW2": dW2, "dpre": dpre}


def post_from_q(q_codes, scale):
    """The backward's stand-in for post when only its e4m3 copy was kept:
    post_hat = fl32(dec(q) * fl32(1/scale)).

    [R] implementation notes: the BF16 post stays materialised by choice;
    rebuilding what the backward needs from the FP8 copy is the orthogonal
    variant.  Reading: post_hat replaces post everywhere in ``mlp_bwd``
    (sqrt(post_hat) in dpre, post_hat in dW2).  dec(q) (<= 4 significant
    bits) times an fp32 value is exact in float64, so ``fl32`` rounds once.
    """
    return fl32(e4m3_decode(np.asarray(q_codes, dtype=np.uint8)) * inv_scale(scale))


def mlp_bwd_sampled(dY_bits, X_bits, W1_bits, W2_bits, post, rows, dw1_rows,
                    dw2_cols, rnd=bf16):
    """The same formulas as ``mlp_bwd`` evaluated only on sampled outputs.

    rows:     rows of dX (and dpre) to produce
    dw1_rows: rows i of dW1 = dpre[:, i]^T X   (needs dpre column i, all M)
    dw2_cols: columns j of dW2 = dY^T post[:, j]
    """
    dY = bf16_to_f64(dY_bits)
    X = bf16_to_f64(X_bits)
    W1 = bf16_to_f64(W1_bits)
    W2 = bf16_to_f64(W2_bits)
    post = np.asarray(post, dtype=np.float64)
    dpre_rows = rnd(2.0 * np.sqrt(post[rows]) * (dY[rows] @ W2))
    dX_rows = rnd(dpre_rows @ W1)
    dpre_cols = rnd(2.0 * np.sqrt(post[:, dw1_rows]) * (dY @ W2[:, dw1_rows]))
    dW1_rows = dpre_cols.T @ X
    dW2_cols = dY.T @ post[:, dw2_cols]
    return {"dX_rows": dX_rows, "dpre_rows": dpre_rows, "dW1_rows": dW1_rows,
            "dW2_cols": dW2_cols}


# --------------------------------------------------------------------------
# FP8 linear for the attention projections
# --------------------------------------------------------------------------
def fp8_linear(X_bits, x_scale, Wt_codes, w_inv_scale):
    """Y = (dec(e4m3(fl32(X * sx))) dec(Wt)) * fl32(1/sx) * w_inv_scale.

    [S] item 1: QKV and output projections in e4m3 on the forward pass with
    weights stored transposed; the activation is quantised with the
    per-tensor multiplier ``x_scale`` supplied by the caller.
    Returns uint16 bf16 bits of Y.
    """
    X = bf16_to_f64(X_bits)
    sx = float(np.float32(x_scale))
    codes = e4m3_encode(fl32(X * sx))
    acc = e4m3_decode(codes) @ e4m3_decode(Wt_codes)
    return bf16_round(acc * inv_scale(sx) * w_inv_scale)
