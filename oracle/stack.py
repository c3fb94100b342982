"""The layer stack around the MLP block: the normalised residual stream, the
plain SGD step and the per-layer delayed-scale state.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
imports this module.

The pages train the MLP block inside a pre-norm transformer: the block reads
an RMS-normalised copy of the residual stream and adds its output back, and
after every optimizer update the transposed fp8 W2 cache is refreshed while
each layer keeps its own amax(t-1) ("A Retrospective on Our World Records",
Main Track: the delayed-scaling and W2-cache paragraphs).  The pages give no
formulas for the normalisation, the residual arithmetic or the optimizer; the
weightless RMSNorm, the residual add and the SGD step below are harness pieces
with these readings:

  rmsnorm:   r = 1 / sqrt(mean_j(x_j^2) + eps), eps = 1e-6;  xn = bf16(x r)
  backward:  dx = r (dxn - xh mean_j(dxn_j xh_j)),  xh = x r
  residual:  x_{l+1} = bf16(x_l + y_l)
  gradient:  g_l = bf16(g_{l+1} + dx_l)      (the stream gradient stays bf16)
  SGD:       W <- bf16(fp32(W - fp32(lr dW)))

Everything is float64 with the stated roundings written out; ``rnd`` defaults
to bf16 and ``exact`` turns the roundings off so the algebra can be checked
against calculus.
"""
import numpy as np

from .formats import bf16, bf16_round, bf16_to_f64, fl32

EPS = 1e-6


def rmsnorm(x_bits, eps=EPS, rnd=bf16):
    """Weightless RMSNorm of each row.  Returns (xn, r): xn rounded by ``rnd``
    (float64 values), r = 1 / sqrt(mean(x^2) + eps) per row (float64)."""
    x = bf16_to_f64(x_bits)
    ms = np.mean(x * x, axis=1)
    r = 1.0 / np.sqrt(ms + eps)
    return rnd(x * r[:, None]), r


def rmsnorm_bwd(x_bits, r, dxn):
    """Gradient of xn = x r(x) with respect to x, given dL/dxn (float64).

    With xh = x r and D the row width: d xh_i / d x_j = r (delta_ij -
    xh_i xh_j / D), so dx = r (dxn - xh mean(dxn xh)).  Unrounded."""
    x = bf16_to_f64(x_bits)
    r = np.asarray(r, dtype=np.float64)[:, None]
    xh = x * r
    dxn = np.asarray(dxn, dtype=np.float64)
    c = np.mean(dxn * xh, axis=1, keepdims=True)
    return r * (dxn - xh * c)


def residual_add(a_bits, b_bits):
    """bf16(a + b): the sum of two bf16 values is exact in float64, so this is
    one round-to-nearest-even."""
    return bf16_round(bf16_to_f64(a_bits) + bf16_to_f64(b_bits))


def grad_add(g_bits, dx):
    """Stream gradient of the layer below: bf16(g + dx), dx float64."""
    return bf16_round(bf16_to_f64(g_bits) + np.asarray(dx, dtype=np.float64))


def sgd(W_bits, dW, lr):
    """W <- bf16(fp32(W - fp32(lr dW))) with lr and dW taken as fp32.

    lr * dW is a product of two fp32 values, exact in float64, so ``fl32``
    rounds it once; W (bf16) minus an fp32 value is exact in float64 for the
    magnitudes of a training step, so the second ``fl32`` is one rounding too."""
    W = bf16_to_f64(W_bits)
    step = fl32(np.float64(np.float32(lr)) * np.asarray(dW, dtype=np.float32).astype(np.float64))
    return bf16_round(fl32(W - step))


def stack_forward_exact(x, layers, eps=EPS):
    """Plain fp64 forward of x += relu(rmsnorm(x) W1^T)^2 W2^T over the layers
    (no bf16 or fp8 at all); ``layers`` is a list of (W1, W2) float64 arrays.
    Used to pin the stack's composition against finite differences."""
    x = np.asarray(x, dtype=np.float64)
    for W1, W2 in layers:
        ms = np.mean(x * x, axis=1, keepdims=True)
        xn = x / np.sqrt(ms + eps)
        pre = xn @ W1.T
        x = x + (np.maximum(pre, 0.0) ** 2) @ W2.T
    return x


def stack_backward_exact(x, layers, g_top, eps=EPS):
    """Gradients of L = sum(g_top * stack_forward_exact(x)) with respect to x
    and every W1, W2, by the chain rule in the order the harness runs it
    (MLP backward with relu(pre) = sqrt(post), then the RMSNorm backward, then
    the residual).  Returns (dx, [(dW1, dW2), ...])."""
    x = np.asarray(x, dtype=np.float64)
    acts = []
    for W1, W2 in layers:
        ms = np.mean(x * x, axis=1)
        r = 1.0 / np.sqrt(ms + eps)
        xn = x * r[:, None]
        post = np.maximum(xn @ W1.T, 0.0) ** 2
        acts.append((x, r, xn, post))
        x = x + post @ W2.T
    g = np.asarray(g_top, dtype=np.float64)
    grads = [None] * len(layers)
    for i in range(len(layers) - 1, -1, -1):
        W1, W2 = layers[i]
        xi, r, xn, post = acts[i]
        dpre = 2.0 * np.sqrt(post) * (g @ W2)
        grads[i] = (dpre.T @ xn, g.T @ post)
        dxn = dpre @ W1
        xh = xi * r[:, None]
        g = g + r[:, None] * (dxn - xh * np.mean(dxn * xh, axis=1, keepdims=True))
    return g, grads
