"""Pins for the oracle's layer-stack pieces (CPU only): brute-force loops,
closed forms, central finite differences and torch's independent CPU fp32 /
bf16 arithmetic."""
import math

import numpy as np
import torch

from fp8_relu_mlp_amd import synth
from oracle import formats as F
from oracle import stack as S


def _bits(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float64))


def test_rmsnorm_brute_force():
    g = np.random.default_rng(0)
    xb = _bits(g.standard_normal((5, 24)) * np.array([1e-3, 0.1, 1.0, 10.0, 300.0])[:, None])
    xn, r = S.rmsnorm(xb)
    x = F.bf16_to_f64(xb)
    for i in range(5):
        ms = math.fsum(float(v) * float(v) for v in x[i]) / 24
        ri = 1.0 / math.sqrt(ms + 1e-6)
        assert abs(r[i] - ri) <= 1e-15 * ri
        for j in range(24):
            assert xn[i, j] == F.bf16(np.array(x[i, j] * ri))


def test_rmsnorm_closed_forms():
    # a constant row c: xn = c / sqrt(c^2 + eps)
    xb = _bits(np.full((1, 64), 3.0))
    xn, r = S.rmsnorm(xb)
    assert r[0] == 1.0 / math.sqrt(9.0 + 1e-6)
    assert (xn == F.bf16(np.array(3.0 / math.sqrt(9.0 + 1e-6)))).all()
    # a zero row stays zero (r = 1/sqrt(eps))
    xn, r = S.rmsnorm(_bits(np.zeros((1, 64))))
    assert (xn == 0).all() and r[0] == 1.0 / math.sqrt(1e-6)
    # unrounded: mean(xh^2) = ms / (ms + eps)
    g = np.random.default_rng(1)
    xb = _bits(g.standard_normal((4, 96)))
    xh, r = S.rmsnorm(xb, rnd=lambda v: v)
    x = F.bf16_to_f64(xb)
    ms = np.mean(x * x, axis=1)
    assert np.allclose(np.mean(xh * xh, axis=1), ms / (ms + 1e-6), rtol=1e-14)


def test_rmsnorm_bwd_finite_differences():
    g = np.random.default_rng(2)
    xb = _bits(g.standard_normal((3, 16)))
    x = F.bf16_to_f64(xb)
    dxn = g.standard_normal((3, 16))
    _, r = S.rmsnorm(xb)
    dx = S.rmsnorm_bwd(xb, r, dxn)

    def f(xx):
        rr = 1.0 / np.sqrt(np.mean(xx * xx, axis=1, keepdims=True) + 1e-6)
        return float(np.sum(dxn * xx * rr))

    h = 1e-6
    num = np.zeros_like(x)
    for i in range(3):
        for j in range(16):
            e = np.zeros_like(x)
            e[i, j] = h
            num[i, j] = (f(x + e) - f(x - e)) / (2 * h)
    assert np.abs(num - dx).max() <= 1e-6 * np.abs(dx).max()


def test_residual_add_matches_torch():
    g = np.random.default_rng(3)
    a = _bits(g.standard_normal(20000) * 10.0 ** g.integers(-8, 8, 20000))
    b = _bits(g.standard_normal(20000) * 10.0 ** g.integers(-8, 8, 20000))
    ours = S.residual_add(a, b)
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).float()
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float()
    ref = (ta + tb).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


def test_grad_add():
    g = np.random.default_rng(4)
    gb = _bits(g.standard_normal(1000))
    assert (S.grad_add(gb, np.zeros(1000)) == gb).all()
    dx = g.standard_normal(1000) * 1e-2
    assert (S.grad_add(_bits(np.zeros(1000)), dx) == F.bf16_round(dx)).all()
    # dx with 8 significant bits and the same binade as g: the fp32 sum is
    # exact, so torch's fp32 add followed by its bf16 cast is one rounding too
    dxq = F.bf16(g.standard_normal(1000))
    tg = torch.from_numpy(gb.view(np.int16)).view(torch.bfloat16).float()
    ref = (tg + torch.from_numpy(dxq.astype(np.float32))).to(torch.bfloat16)
    assert (S.grad_add(gb, dxq) == ref.view(torch.int16).numpy().view(np.uint16)).all()


def test_sgd_matches_torch_fp32():
    g = np.random.default_rng(5)
    W = _bits(g.standard_normal(50000) * 0.05)
    dW = (g.standard_normal(50000) * 10.0 ** g.integers(-6, 2, 50000)).astype(np.float32)
    ours = S.sgd(W, dW, 1e-3)
    tW = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).float()
    lr = torch.tensor(1e-3, dtype=torch.float32)
    ref = (tW - lr * torch.from_numpy(dW)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()
    # a zero gradient leaves the weights untouched
    assert (S.sgd(W, np.zeros(50000, dtype=np.float32), 1e-3) == W).all()


def test_stack_backward_finite_differences():
    g = np.random.default_rng(6)
    M, d, h, L = 3, 4, 6, 3
    x = g.standard_normal((M, d))
    layers = [(g.standard_normal((h, d)) / 2, g.standard_normal((d, h)) / 3) for _ in range(L)]
    gt = g.standard_normal((M, d))
    dx, grads = S.stack_backward_exact(x, layers, gt)

    def loss(xx, ls):
        return float(np.sum(gt * S.stack_forward_exact(xx, ls)))

    eps = 1e-6

    def fd(get, put, ref):
        num = np.zeros_like(ref)
        for idx in np.ndindex(ref.shape):
            orig = get()[idx]
            put(idx, orig + eps)
            fp = lossf()
            put(idx, orig - eps)
            fm = lossf()
            put(idx, orig)
            num[idx] = (fp - fm) / (2 * eps)
        return num

    xs = x.copy()
    lossf = lambda: loss(xs, layers)
    num = fd(lambda: xs, lambda i, v: xs.__setitem__(i, v), dx)
    assert np.abs(num - dx).max() <= 1e-6 * max(1.0, np.abs(dx).max())
    for li in (0, L - 1):
        for wi in (0, 1):
            Wm = [list(p) for p in layers]
            lossf = lambda: loss(x, [tuple(p) for p in Wm])
            ref = grads[li][wi]
            num = fd(lambda: Wm[li][wi], lambda i, v: Wm[li][wi].__setitem__(i, v), ref)
            assert np.abs(num - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())
