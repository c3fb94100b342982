"""Pins for the oracle's softcapped cross-entropy (CPU only): torch's own
cross-entropy for the uncapped case, closed forms, central finite
differences of the loss, brute-force loops, and the handling of missing
targets."""
import math

import numpy as np
import torch

from fp8_relu_mlp_amd import synth
from oracle import ce as C
from oracle import formats as F


def _case(M=6, d=8, V=11, T=2, seed=3):
    ins = synth.ce_inputs(M, d, V, T, seed)
    return ins["X"], ins["W"], ins["targets"]


def test_uncapped_single_target_is_torch_cross_entropy():
    X, W, t = _case(T=1)
    out = C.softcap_ce(X, W, t, [1.0], float("inf"))
    z = torch.from_numpy(F.bf16_to_f64(X) @ F.bf16_to_f64(W).T)
    M = t.shape[0]
    assert (t[:, 0] < 0).sum() == 1                 # the last position has no next token
    tt = torch.from_numpy(t[:, 0])
    ref = torch.nn.functional.cross_entropy(z, tt, ignore_index=-1, reduction="sum") / M
    assert abs(out["loss"] - float(ref)) < 1e-12
    zg = z.clone().requires_grad_(True)
    (torch.nn.functional.cross_entropy(zg, tt, ignore_index=-1, reduction="sum") / M).backward()
    g = C.softcap_ce(X, W, t, [1.0], float("inf"), rnd=C.exact)["G"]
    assert np.allclose(g, zg.grad.numpy(), rtol=0, atol=1e-14)


def test_zero_head_closed_form():
    X, _, t = _case()
    W = np.zeros((11, 8), dtype=np.uint16)          # bf16 +0
    w = [0.5, 0.25]
    out = C.softcap_ce(X, W, t, w, 15.0, rnd=C.exact)
    assert np.allclose(out["lse"], math.log(11))
    valid = t >= 0
    expect = (np.where(valid, np.array(w)[None, :], 0.0).sum() * math.log(11)) / t.shape[0]
    assert abs(out["loss"] - expect) < 1e-12
    # G = (wsum / V - sum_j w_j onehot) / M, and (1 - 0) for the softcap
    M, V = t.shape[0], 11
    G = np.zeros((M, V))
    for m in range(M):
        ws = sum(w[j] for j in range(2) if t[m, j] >= 0)
        G[m] += ws / V
        for j in range(2):
            if t[m, j] >= 0:
                G[m, t[m, j]] -= w[j]
    assert np.allclose(out["G"], G / M, rtol=0, atol=1e-15)


def test_softcap_bounds_and_limit():
    z = np.array([-1e4, -30.0, -1.0, 0.0, 2.0, 50.0, 1e4])
    zc = C.softcap(z, 15.0)
    assert (np.abs(zc) < 15.0 + 1e-12).all() and zc[3] == 0.0
    assert np.allclose(C.softcap(z[2:5], 1e8), z[2:5], rtol=1e-12)


def test_loss_gradients_match_finite_differences():
    X, W, t = _case(M=4, d=5, V=7, T=2, seed=9)
    w, c = [1.0, 0.5], 3.0
    Xf, Wf = F.bf16_to_f64(X), F.bf16_to_f64(W)

    def loss(Xv, Wv):
        return C.softcap_ce(X, W, t, w, c, rnd=C.exact, Z=Xv @ Wv.T)["loss"]

    out = C.softcap_ce(X, W, t, w, c, rnd=C.exact)
    # dX and dW from the oracle use the bf16 X / W values; the loss is a
    # function of those, so differentiate around them
    dX = out["G"] @ Wf
    eps = 1e-6
    for (i, j) in [(0, 0), (1, 3), (3, 4)]:
        Xp, Xm = Xf.copy(), Xf.copy()
        Xp[i, j] += eps
        Xm[i, j] -= eps
        fd = (loss(Xp, Wf) - loss(Xm, Wf)) / (2 * eps)
        assert abs(fd - dX[i, j]) < 1e-7 * max(1.0, abs(fd))
        assert abs(out["dX"][i, j] - dX[i, j]) < 1e-15
    for (i, j) in [(0, 0), (2, 1), (6, 4)]:
        Wp, Wm = Wf.copy(), Wf.copy()
        Wp[i, j] += eps
        Wm[i, j] -= eps
        fd = (loss(Xf, Wp) - loss(Xf, Wm)) / (2 * eps)
        assert abs(fd - out["dW"][i, j]) < 1e-7 * max(1.0, abs(fd))


def test_loops_and_missing_targets():
    X, W, t = _case(M=5, d=6, V=9, T=3, seed=12)
    t[1, 2] = -1
    t[4, :] = -1
    w, c = [0.6, 0.3, 0.1], 7.5
    out = C.softcap_ce(X, W, t, w, c, rnd=C.exact)
    Xf, Wf = F.bf16_to_f64(X), F.bf16_to_f64(W)
    total = 0.0
    for m in range(5):
        zc = [c * math.tanh(sum(Xf[m, k] * Wf[v, k] for k in range(6)) / c) for v in range(9)]
        lse = math.log(math.fsum(math.exp(x) for x in zc))
        assert abs(lse - out["lse"][m]) < 1e-12
        total += sum(w[j] * (lse - zc[t[m, j]]) for j in range(3) if t[m, j] >= 0)
    assert abs(total / 5 - out["loss"]) < 1e-12
    assert out["per_row"][4] == 0.0 and np.isnan(out["zt"][4]).all()
    assert (out["G"][4] == 0).all()


def test_fp8_logits_lossless_and_against_torch_cast():
    """Power-of-two scales with e4m3-exact operands: the FP8 logits equal the
    bf16 ones exactly; random data: torch's own e4m3 cast and an exact dot
    product over the untransposed W."""
    from oracle import mlp as O
    g = np.random.default_rng(44)
    X = synth.to_bf16_bits(g.integers(-7, 8, size=(5, 16)) / 4.0)
    Wv = g.integers(-7, 8, size=(9, 16)) / 8.0
    Wv[0, 0] = 7 / 8
    W = synth.to_bf16_bits(Wv)
    Wt, s, inv, _ = O.cast_transpose(W)
    assert s == 512.0
    z = C.fp8_logits(X, 16.0, Wt, inv)
    assert (z == F.bf16_to_f64(X) @ F.bf16_to_f64(W).T).all()
    ins = synth.ce_inputs(4, 32, 64, 1, 45)
    Wt, s, inv, _ = O.cast_transpose(ins["W"])
    Xf = F.bf16_to_f64(ins["X"])
    sx = O.exact_scale(O.amax(Xf))
    z = C.fp8_logits(ins["X"], sx, Wt, inv)

    def cast(v):
        return torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()

    xd, wd = cast(Xf * sx), cast(F.bf16_to_f64(ins["W"]) * s)
    inv_sx = float(np.float32(1.0 / np.float32(sx)))
    for m in range(4):
        for v in range(64):
            acc = math.fsum(xd[m, k] * wd[v, k] for k in range(32))
            assert z[m, v] == acc * inv_sx * inv
