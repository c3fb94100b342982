"""Fused softcapped cross-entropy over a language-model head, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
imports this module.

Sources: "NanoGPT Speedrun (Track 1)", "From Unoptimized", "Approach" item 5
(a fused softcapped cross-entropy kernel that never materialises the [M, V]
logits in fp32) and "A Retrospective on Our World Records", the SlowRun part
(one language-model head trained against three successive targets at each
position through a fused FP8 soft-capped cross-entropy).  The pages give no
formula, constant or weighting; the readings are:

  z    = X W^T                          [M, V]  (the head; never stored)
  z'   = c tanh(z / c)                  the softcap, c > 0 (c = inf: none)
  lse  = log sum_v exp(z'[m, v])
  L    = (1/M) sum_m sum_j w_j (lse_m - z'[m, t[m, j]])   over targets t >= 0
  dz'  = (dL/M) (wsum_m softmax(z')[m, v] - sum_j w_j [v == t[m, j]]),
         wsum_m = sum of w_j over the row's valid targets
  dz   = dz' (1 - (z'/c)^2)             (d tanh)
  G    = bf16(dz)                       the gradient of the logits, bf16 [M, V]
  dX   = bf16(G W)                      [M, d]
  dW   = G^T X                          [V, d] (fp32 on the device)

``rnd`` (default bf16) is applied where the device rounds to bf16 (G, dX);
``exact`` removes it so the algebra can be checked against calculus.
"""
import numpy as np

from .formats import bf16, bf16_to_f64, e4m3_decode, e4m3_encode, fl32


def exact(x):
    return np.asarray(x, dtype=np.float64)


def softcap(z, c):
    """c tanh(z / c); c = inf is the identity."""
    z = np.asarray(z, dtype=np.float64)
    return z if np.isinf(c) else c * np.tanh(z / c)


def logsumexp_rows(zc):
    mx = zc.max(axis=1, keepdims=True)
    return (mx + np.log(np.exp(zc - mx).sum(axis=1, keepdims=True)))[:, 0]


def softcap_ce(X_bits, W_bits, targets, weights, c, dloss=1.0, rnd=bf16, Z=None):
    """Loss and gradients of the softcapped cross-entropy (readings above).

    X_bits [M, d] and W_bits [V, d]: bf16 bit patterns; targets [M, T] int
    (negative = no target); weights [T]; c: the softcap; dloss: the incoming
    gradient of L.  ``Z`` lets a test pass precomputed logits z (float64).
    Returns a dict: loss, lse [M], zt [M, T] (the target logits z', NaN for
    no target), G (the rounded logit gradient, float64 values), dX, dW.
    """
    X = bf16_to_f64(X_bits)
    W = bf16_to_f64(W_bits)
    t = np.asarray(targets, dtype=np.int64)
    if t.ndim == 1:
        t = t[:, None]
    w = np.asarray(weights, dtype=np.float64).reshape(-1)
    M, T = t.shape
    V = W.shape[0]
    z = X @ W.T if Z is None else np.asarray(Z, dtype=np.float64)
    zc = softcap(z, c)
    lse = logsumexp_rows(zc)
    valid = t >= 0
    rows = np.arange(M)[:, None]
    zt = np.where(valid, zc[rows, np.clip(t, 0, V - 1)], np.nan)
    per_row = np.where(valid, w[None, :] * (lse[:, None] - np.nan_to_num(zt)), 0.0).sum(axis=1)
    loss = per_row.sum() / M
    wsum = np.where(valid, w[None, :], 0.0).sum(axis=1)
    p = np.exp(zc - lse[:, None])
    dzc = wsum[:, None] * p
    for j in range(T):
        m = np.nonzero(valid[:, j])[0]
        np.add.at(dzc, (m, t[m, j]), -w[j])
    dzc *= dloss / M
    dz = dzc if np.isinf(c) else dzc * (1.0 - (zc / c) ** 2)
    G = rnd(dz)
    return {"loss": float(loss), "lse": lse, "zt": zt, "G": G, "dX": rnd(G @ W), "dW": G.T @ X,
            "per_row": per_row}


def fp8_logits(X_bits, x_scale, Wt_codes, w_inv_scale):
    """The head's logits with both operands in e4m3 (the FP8 form of the
    fused cross-entropy, "A Retrospective on Our World Records", SlowRun
    part): z = (dec(e4m3(fl32(X sx))) dec(Wt)) * fl32(1/sx) * w_inv, the
    product sums exact in float64 (every e4m3 product is a multiple of 2^-18
    below 2^18).  Wt_codes [d, V] is the transposed e4m3 cache of W [V, d].
    Pass the result as ``Z`` to ``softcap_ce`` (whose dX and dW stay on the
    bf16 X and W)."""
    X = bf16_to_f64(X_bits)
    sx = float(np.float32(x_scale))
    xq = e4m3_decode(e4m3_encode(fl32(X * sx)))
    inv_sx = float(fl32(1.0 / np.float64(np.float32(sx))))
    return (xq @ e4m3_decode(Wt_codes)) * inv_sx * float(np.float32(w_inv_scale))
