"""Pins for the oracle's MLP path (CPU only).

Checks against brute-force loops, closed forms, central finite differences,
exact rational arithmetic, torch's independent fp8 cast, and a lossless
special case in which the FP8 path must equal an integer GEMM bit for bit.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth
from oracle import formats as F
from oracle import mlp as O


def _bf16_bits(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float64))


# ------------------------------------------------------------------ scales
def test_delayed_scale_closed_forms():
    assert O.delayed_scale(7.0, 2.0) == 32.0              # 448 / 14
    assert O.delayed_scale(448.0, 1.0) == 1.0
    assert O.delayed_scale(0.875, 2.0) == 256.0           # 448 / 1.75
    for bad in (0.0, -1.0, float("nan"), float("inf"), -float("inf")):
        assert O.delayed_scale(bad, 2.0) == 1.0
    assert O.delayed_scale(1e-38, 1.0) == 1.0             # 448/1e-38 overflows fp32


def test_delayed_scale_is_correctly_rounded_fp32():
    g = np.random.default_rng(0)
    for a in np.float32(np.abs(g.standard_normal(300)) * 10.0 ** g.integers(-6, 6, 300)):
        s = O.delayed_scale(float(a), 2.0)
        den = Fraction(float(np.float32(2.0 * np.float64(a))))  # 2*a is exact in fp32
        q = Fraction(448) / den
        lo = np.nextafter(np.float32(s), np.float32(0))
        hi = np.nextafter(np.float32(s), np.float32(np.inf))
        err = abs(Fraction(s) - q)
        assert err <= abs(Fraction(float(lo)) - q) and err <= abs(Fraction(float(hi)) - q)


def test_inv_scale_is_correctly_rounded_fp32_reciprocal():
    """inv_scale(s) is the fp32 value nearest to the exact rational 1/s (ties
    to the even significand), for scales that are not powers of two as well:
    checked with exact Fractions against both fp32 neighbours."""
    g = np.random.default_rng(5)
    scales = np.float32(np.abs(g.standard_normal(400)) * 10.0 ** g.integers(-8, 8, 400))
    scales = np.concatenate([scales, np.float32([448.0 / 3.0, 448.0 / 14.0, 0.37, 3.0, 7.0, 2.0 ** -5, 1.0])])
    for s in scales:
        inv = O.inv_scale(float(s))
        assert float(np.float32(inv)) == inv                     # an fp32 value
        q = 1 / Fraction(float(s))
        lo = np.nextafter(np.float32(inv), np.float32(0))
        hi = np.nextafter(np.float32(inv), np.float32(np.inf))
        err = abs(Fraction(inv) - q)
        e_lo, e_hi = abs(Fraction(float(lo)) - q), abs(Fraction(float(hi)) - q)
        assert err <= e_lo and err <= e_hi, s
        if err in (e_lo, e_hi):                                  # a tie: the even significand wins
            assert int(np.float32(inv).view(np.uint32)) % 2 == 0
    # powers of two invert exactly
    for e in range(-20, 21):
        assert O.inv_scale(2.0 ** e) == 2.0 ** -e


def test_amax_definition():
    x = np.array([[0.5, -3.0], [2.0, 1.0]])
    assert O.amax(x) == 3.0
    assert O.amax(np.zeros((0, 4))) == 0.0
    assert np.isnan(O.amax(np.array([1.0, np.nan, -5.0])))
    assert O.amax(np.array([-np.inf, 1.0])) == np.inf


def test_tile_amax_brute_force():
    g = np.random.default_rng(1)
    p = g.random((37, 53))
    t = O.tile_amax(p, 16, 32)
    assert t.shape == (3, 2)
    for i in range(3):
        for j in range(2):
            best = 0.0
            for r in range(i * 16, min(37, i * 16 + 16)):
                for c in range(j * 32, min(53, j * 32 + 32)):
                    best = max(best, p[r, c])
            assert t[i, j] == best
    assert t.max() == O.amax(p)


# ------------------------------------------------------------------ forward
def test_up_relu2_matches_triple_loop():
    M, d, h = 5, 7, 6
    X = synth.normal_bf16((M, d), 1.0, 11, "X")
    W1 = synth.normal_bf16((h, d), 1.0 / d, 11, "W1")
    post = O.up_relu2(X, W1, rnd=O.exact)
    Xf, Wf = F.bf16_to_f64(X), F.bf16_to_f64(W1)
    for m in range(M):
        for j in range(h):
            pre = sum(Fraction(float(Xf[m, k])) * Fraction(float(Wf[j, k])) for k in range(d))
            r = max(pre, Fraction(0))
            assert abs(post[m, j] - float(r * r)) <= 1e-15 * max(1.0, float(r * r))
    # rounded variant = bf16 of the exact one
    assert (F.bf16_round(O.up_relu2(X, W1)) == F.bf16_round(post)).all()


def test_sqrt_post_rebuilds_relu_pre():
    # sqrt of a correctly rounded square of a double is that double (base 2)
    g = np.random.default_rng(2)
    pre = g.standard_normal(100000) * 10.0 ** g.integers(-5, 5, 100000)
    r = np.maximum(pre, 0.0)
    assert (np.sqrt(r * r) == r).all()


def test_down_fp8_exact_against_fractions():
    g = np.random.default_rng(3)
    M, K, N = 3, 40, 4
    q = g.integers(0, 256, size=(M, K)).astype(np.uint8)
    w = g.integers(0, 256, size=(K, N)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x10      # no NaN codes
    w[(w & 0x7F) == 0x7F] = 0x22
    acc = O.down_fp8(q, w, 1.0, 1.0, rnd=O.exact)
    qd, wd = F.e4m3_decode(q), F.e4m3_decode(w)
    for m in range(M):
        for n in range(N):
            s = sum(Fraction(float(qd[m, k])) * Fraction(float(wd[k, n])) for k in range(K))
            assert acc[m, n] == float(s)            # exact, not approximately


def test_quantize_matches_torch_cast():
    g = np.random.default_rng(4)
    post = F.bf16(np.abs(g.standard_normal(50000)) ** 2 * 3)
    s = O.delayed_scale(float(post.max()) * 0.9, 2.0)
    v = (post * s).astype(np.float32)
    assert np.abs(v).max() <= 448
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (O.quantize(post, s) == ref).all()


def _lossless_case(M=24, d=16, h=32, N=12, seed=7):
    # X, W1 in {-1,0,1} with at most 3 non-zeros per W1 row: pre in
    # {-3..3}, post in {0,1,4,9}; amax_prev = 7 and margin 2 give scale 32,
    # so post*scale in {0,32,128,288} is exact e4m3; W2 in {-1,0,1} cast
    # with scale 1 is exact too: the fp8 result must equal the integer GEMM.
    X = synth.ternary_bf16((M, d), seed, "X")
    W1 = synth.ternary_bf16((h, d), seed, "W1", nnz_per_row=3)
    W2 = synth.ternary_bf16((N, h), seed, "W2")
    return X, W1, W2


def test_forward_lossless_special_case():
    X, W1, W2 = _lossless_case()
    W2t, s_w, inv_sw, a_w = O.cast_transpose(W2, scale_in=1.0)
    assert (s_w, inv_sw, a_w) == (1.0, 1.0, 1.0)
    out = O.mlp_fwd(X, W1, W2t, inv_sw, 7.0, 2.0)
    assert out["scale"] == 32.0
    Xi = F.bf16_to_f64(X).astype(np.int64)
    W1i = F.bf16_to_f64(W1).astype(np.int64)
    W2i = F.bf16_to_f64(W2).astype(np.int64)
    pre = Xi @ W1i.T
    post = np.maximum(pre, 0) ** 2
    y = post @ W2i.T
    assert np.abs(y).max() <= 256
    assert (F.bf16_to_f64(out["post"]) == post).all()
    assert (F.e4m3_decode(out["post_q"]) == post * 32).all()
    assert (F.bf16_to_f64(out["y"]) == y).all()
    assert out["amax"] == post.max()
    ev = O.mlp_fwd(X, W1, None, None, None, None, mode="eval", W2_bits=W2)
    assert (F.bf16_to_f64(ev["y"]) == y).all()
    # the same case through the FP8 linear: X in {-1,0,1}, scale 1
    W1t, s1, inv1, _ = O.cast_transpose(W1, scale_in=1.0)
    Y = O.fp8_linear(X, 1.0, W1t, inv1)
    assert (F.bf16_to_f64(Y) == pre).all()


def test_forward_small_against_loops():
    # every step of mlp_fwd re-derived element by element
    M, d, h = 4, 8, 16
    ins = synth.mlp_inputs(M, d, h, 9)
    W2t, s_w, inv_sw, a_w = O.cast_transpose(ins["W2"])
    out = O.mlp_fwd(ins["X"], ins["W1"], W2t, inv_sw, 0.8, 2.0)
    Xf, W1f, W2f = (F.bf16_to_f64(ins[k]) for k in ("X", "W1", "W2"))
    s = out["scale"]
    assert s == float(np.float32(448.0 / np.float32(1.6)))
    assert a_w == np.abs(W2f).max()
    for m in range(M):
        for j in range(h):
            pre = sum(Xf[m, k] * W1f[j, k] for k in range(d))
            p = F.bf16(max(pre, 0.0) ** 2)
            assert F.bf16_to_f64(out["post"][m, j]) == p
            qv = np.float32(np.float32(p) * np.float32(s))
            # torch does not saturate above 464: clamp first (saturating encode)
            qv = min(float(qv), 448.0)
            ref = torch.tensor([qv]).to(torch.float8_e4m3fn).view(torch.uint8).item()
            assert out["post_q"][m, j] == ref
    for k in range(h):
        for n in range(d):
            wv = np.float32(np.float32(W2f[n, k]) * np.float32(s_w))
            ref = torch.tensor([float(wv)]).to(torch.float8_e4m3fn).view(torch.uint8).item()
            assert W2t[k, n] == ref
    qd, wd = F.e4m3_decode(out["post_q"]), F.e4m3_decode(W2t)
    inv_s = float(np.float32(1.0 / s))
    for m in range(M):
        for n in range(d):
            acc = sum(qd[m, k] * wd[k, n] for k in range(h))
            assert F.bf16_to_f64(out["y"][m, n]) == F.bf16(acc * inv_s * inv_sw)


def test_fp8_path_close_to_exact_function():
    # the fp8 approximation stays near the rounding-free MLP (scale sanity)
    M, d, h = 64, 64, 256
    ins = synth.mlp_inputs(M, d, h, 10)
    W2t, s_w, inv_sw, _ = O.cast_transpose(ins["W2"])
    boot = O.mlp_fwd(ins["X"], ins["W1"], W2t, inv_sw, 1.0, 2.0)
    out = O.mlp_fwd(ins["X"], ins["W1"], W2t, inv_sw, boot["amax"], 2.0)
    post = O.up_relu2(ins["X"], ins["W1"], rnd=O.exact)
    y_ex = post @ F.bf16_to_f64(ins["W2"]).T
    y = F.bf16_to_f64(out["y"])
    rel = np.linalg.norm(y - y_ex) / np.linalg.norm(y_ex)
    assert rel < 0.08
    ev = O.mlp_fwd(ins["X"], ins["W1"], None, None, None, None, mode="eval", W2_bits=ins["W2"])
    rel_e = np.linalg.norm(F.bf16_to_f64(ev["y"]) - y_ex) / np.linalg.norm(y_ex)
    assert rel_e < 1e-2


def test_saturation_when_amax_prev_too_small():
    M, d, h = 32, 32, 64
    ins = synth.mlp_inputs(M, d, h, 12)
    post = F.bf16_to_f64(F.bf16_round(O.up_relu2(ins["X"], ins["W1"])))
    a = post.max()
    s = O.delayed_scale(a / 4, 2.0)
    q = O.quantize(post, s)
    big = np.float32(post * s) >= 448
    assert big.any() and (q[big] == 0x7E).all()
    assert (q[~big] != 0x7E).any()


# ------------------------------------------------------------------ backward
def _exact_forward(X, W1, W2):
    pre = X @ W1.T
    return (np.maximum(pre, 0.0) ** 2) @ W2.T


def test_backward_matches_finite_differences():
    M, d, h = 3, 5, 7
    ins = synth.mlp_inputs(M, d, h, 13, with_dy=True)
    X, W1, W2, dY = (F.bf16_to_f64(ins[k]) for k in ("X", "W1", "W2", "dY"))
    post = np.maximum(X @ W1.T, 0.0) ** 2
    g = O.mlp_bwd(ins["dY"], ins["X"], ins["W1"], ins["W2"], post, rnd=O.exact)

    def L(Xv, W1v, W2v):
        return float((dY * _exact_forward(Xv, W1v, W2v)).sum())

    eps = 1e-6
    for name, A, grad in (("X", X, g["dX"]), ("W1", W1, g["dW1"]), ("W2", W2, g["dW2"])):
        fd = np.zeros_like(A)
        for idx in np.ndindex(A.shape):
            Ap, Am = A.copy(), A.copy()
            Ap[idx] += eps
            Am[idx] -= eps
            args_p = {"X": X, "W1": W1, "W2": W2}
            args_m = dict(args_p)
            args_p[name], args_m[name] = Ap, Am
            fd[idx] = (L(**{"Xv": args_p["X"], "W1v": args_p["W1"], "W2v": args_p["W2"]})
                       - L(**{"Xv": args_m["X"], "W1v": args_m["W1"], "W2v": args_m["W2"]})) / (2 * eps)
        err = np.abs(fd - grad).max() / max(np.abs(fd).max(), 1e-30)
        assert err < 1e-6, (name, err)


def test_backward_closed_form_scalar():
    # d = h = 1: y = w2 * relu(w1 x)^2; dy/dx = 2 w2 w1 relu(w1 x)
    for x, w1, w2, dy in ((1.5, 0.75, -2.0, 0.5), (-1.0, 0.5, 3.0, 1.0), (2.0, -0.25, 1.0, -4.0)):
        b = lambda v: _bf16_bits(np.array([[v]]))
        post = np.array([[max(w1 * x, 0.0) ** 2]])
        g = O.mlp_bwd(b(dy), b(x), b(w1), b(w2), post, rnd=O.exact)
        r = max(w1 * x, 0.0)
        assert g["dX"][0, 0] == dy * 2 * w2 * w1 * r
        assert g["dW1"][0, 0] == dy * 2 * w2 * x * r
        assert g["dW2"][0, 0] == dy * r * r


def test_backward_sampled_matches_full():
    M, d, h = 40, 16, 48
    ins = synth.mlp_inputs(M, d, h, 14, with_dy=True)
    post = F.bf16_to_f64(F.bf16_round(O.up_relu2(ins["X"], ins["W1"])))
    full = O.mlp_bwd(ins["dY"], ins["X"], ins["W1"], ins["W2"], post)
    rows, r1, c2 = [0, 7, 39], [3, 47], [0, 5, 47]
    s = O.mlp_bwd_sampled(ins["dY"], ins["X"], ins["W1"], ins["W2"], post, rows, r1, c2)
    assert np.array_equal(s["dX_rows"], full["dX"][rows])
    assert np.array_equal(s["dpre_rows"], full["dpre"][rows])
    assert np.allclose(s["dW1_rows"], full["dW1"][r1], rtol=1e-13, atol=0)
    assert np.allclose(s["dW2_cols"], full["dW2"][:, c2], rtol=1e-13, atol=0)


def test_fp8_linear_matches_loops_and_torch():
    M, K, N = 6, 32, 8
    g = synth.attn_inputs(M=M, d=K, qkv=N, seed=21)
    Wt, s_w, inv_sw, _ = O.cast_transpose(g["Wqkv"])
    sx = O.exact_scale(O.amax(F.bf16_to_f64(g["X"])))
    Y = F.bf16_to_f64(O.fp8_linear(g["X"], sx, Wt, inv_sw))
    Xf = F.bf16_to_f64(g["X"])
    xv = (Xf * sx).astype(np.float32)
    xq = torch.from_numpy(xv).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    wd = F.e4m3_decode(Wt)
    inv_sx = float(np.float32(1.0 / sx))
    for m in range(M):
        for n in range(N):
            acc = sum(xq[m, k] * wd[k, n] for k in range(K))
            assert Y[m, n] == F.bf16(acc * inv_sx * inv_sw)


# ------------------------------------------------------------------ FP8 up-projection
def _pow2_case(M=20, d=32, h=48, seed=11):
    # X = a/4 and W1 = b/8 with small integers |a|, |b| <= 7, and one W1
    # entry at exactly 7/8: the W1 scale is 448 / (7/8) = 512 = 2^9 and X is
    # scaled by 16, so X*16 = 4a and W1*512 = 64b are e4m3 values (<= 3
    # significant bits, <= 448) and both quantisations are exact.
    g = np.random.default_rng(seed)
    X = g.integers(-7, 8, size=(M, d)) / 4.0
    W1 = g.integers(-7, 8, size=(h, d)) / 8.0
    W1[0, 0] = 7 / 8
    W1[np.abs(W1) > 7 / 8] = 0.5
    return _bf16_bits(X), _bf16_bits(W1)


def test_fp8_up_lossless_power_of_two_scales():
    X, W1 = _pow2_case()
    W1t, s1, inv1, a1 = O.cast_transpose(W1)
    assert (a1, s1, inv1) == (7 / 8, 512.0, 2.0 ** -9)
    post, xq, pre = O.up_relu2_fp8(X, 16.0, W1t, inv1, rnd=O.exact)
    Xf, W1f = F.bf16_to_f64(X), F.bf16_to_f64(W1)
    assert (F.e4m3_decode(xq) == Xf * 16).all()
    assert (pre == Xf @ W1f.T).all()               # exact, not approximately
    assert (post == np.maximum(Xf @ W1f.T, 0) ** 2).all()
    # the rounded post equals the bf16 up-projection's
    post_r, _, _ = O.up_relu2_fp8(X, 16.0, W1t, inv1)
    assert (post_r == O.up_relu2(X, W1)).all()


def test_fp8_up_matches_loops_and_torch_cast():
    """Quantise X and W1 with torch's own float8_e4m3fn cast (independent of
    the oracle's encoder), multiply in explicit loops over the untransposed
    W1 (which pins the orientation of the transposed cache) and dequantise."""
    M, d, h = 5, 32, 12
    ins = synth.mlp_inputs(M, d, h, 23)
    W1t, s1, inv1, _ = O.cast_transpose(ins["W1"])
    Xf, W1f = F.bf16_to_f64(ins["X"]), F.bf16_to_f64(ins["W1"])
    sx = O.exact_scale(O.amax(Xf))
    post, xq, pre = O.up_relu2_fp8(ins["X"], sx, W1t, inv1)

    def cast(v):
        return torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()

    xd, wd = cast(Xf * sx), cast(W1f * s1)
    assert (F.e4m3_decode(xq) == xd).all()
    inv_sx = float(np.float32(1.0 / np.float32(sx)))
    for m in range(M):
        for n in range(h):
            acc = sum(Fraction(float(xd[m, k])) * Fraction(float(wd[n, k])) for k in range(d))
            p = float(acc) * inv_sx * inv1
            assert pre[m, n] == p
            assert post[m, n] == F.bf16(max(p, 0.0) ** 2)


def test_fp8_up_close_to_exact_function():
    """e4m3 keeps 4 significant bits (relative step <= 2^-4 per operand), so
    the fp8 pre stays within a few per cent of X W1^T; a dropped or doubled
    dequantisation factor would be off by the scales (>= 2^5 here)."""
    M, d, h = 64, 256, 384
    ins = synth.mlp_inputs(M, d, h, 24)
    W1t, _, inv1, _ = O.cast_transpose(ins["W1"])
    Xf = F.bf16_to_f64(ins["X"])
    sx = O.exact_scale(O.amax(Xf))
    post, _, pre = O.up_relu2_fp8(ins["X"], sx, W1t, inv1)
    exact_pre = Xf @ F.bf16_to_f64(ins["W1"]).T
    e_pre = np.linalg.norm(pre - exact_pre) / np.linalg.norm(exact_pre)
    assert 1e-3 < e_pre < 0.08
    e_post = np.linalg.norm(post - O.up_relu2(ins["X"], ins["W1"])) / np.linalg.norm(post)
    assert e_post < 0.15


def test_fp8_up_forward_composes_like_train_forward():
    M, d, h = 16, 64, 128
    ins = synth.mlp_inputs(M, d, h, 25)
    W1t, _, inv1, _ = O.cast_transpose(ins["W1"])
    W2t, _, inv2, _ = O.cast_transpose(ins["W2"])
    Xf = F.bf16_to_f64(ins["X"])
    sx = O.exact_scale(O.amax(Xf))
    out = O.mlp_fwd_fp8up(ins["X"], sx, W1t, inv1, W2t, inv2, 3.0, 2.0)
    assert out["x_amax"] == np.abs(Xf).max()
    post, xq, _ = O.up_relu2_fp8(ins["X"], sx, W1t, inv1)
    assert (out["xq"] == xq).all() and (F.bf16_to_f64(out["post"]) == post).all()
    ref = O.mlp_fwd(ins["X"], ins["W1"], W2t, inv2, 3.0, 2.0, post_bits=out["post"])
    for k in ("post_q", "y"):
        assert (out[k] == ref[k]).all()
    assert out["scale"] == ref["scale"] == O.delayed_scale(3.0, 2.0)


# ------------------------------------------------------------------ scaling policies
def test_saturation_count_is_the_top_code_count():
    codes = np.arange(256, dtype=np.uint8)
    assert O.saturation_count(codes) == 2                  # 0x7E and 0xFE
    assert O.saturation_count(np.array([0x7E, 0xFE, 0x7F, 0xFF, 0x7D], dtype=np.uint8)) == 2
    # through the quantiser: exactly the products >= 432 (the midpoint between
    # 416 and 448 rounds to the even code 448, and everything above saturates)
    g = np.random.default_rng(31)
    post = F.bf16(np.abs(g.standard_normal(200000)) ** 2)
    s = O.delayed_scale(float(post.max()) / 3, 2.0)
    q = O.quantize(post, s)
    v = (post * s).astype(np.float32).astype(np.float64)
    assert O.saturation_count(q) == int(np.count_nonzero(v >= 432.0)) > 0
    assert O.saturation_count(O.quantize(np.array([431.9, 432.0, 500.0]), 1.0)) == 2


def test_window_scale_special_cases():
    assert O.window_scale([3.0], 2.0) == O.delayed_scale(3.0, 2.0)
    assert O.window_scale([1.0, 5.0, 2.0], 2.0) == O.delayed_scale(5.0, 2.0)
    assert O.window_scale([0.0, 0.0], 2.0) == 1.0                  # guard
    assert O.window_scale([1.0, float("nan")], 2.0) == 1.0         # NaN propagates to the guard
    # a window never gives a larger scale than amax(t-1) alone
    h = [0.5, 4.0, 1.5]
    assert O.window_scale(h, 2.0) <= O.delayed_scale(h[-1], 2.0)


def test_delayed_cast_with_its_own_amax_is_the_exact_cast():
    W = synth.mlp_inputs(8, 64, 128, 32)["W2"]
    a = O.amax(F.bf16_to_f64(W))
    c1 = O.cast_transpose(W)
    c2 = O.delayed_cast_transpose(W, a, 1.0)
    assert (c1[0] == c2[0]).all() and c1[1:] == c2[1:]
    # a larger previous amax gives a smaller scale and codes that never saturate
    c3 = O.delayed_cast_transpose(W, 2 * a, 1.5)
    assert c3[1] == O.delayed_scale(2 * a, 1.5) < c1[1]
    assert O.saturation_count(c3[0]) == 0


# ------------------------------------------------------------------ backward from the e4m3 copy
def test_post_from_q_inverts_the_lossless_quantisation():
    X, W1, _ = _lossless_case()
    post = O.up_relu2(X, W1)
    assert post.max() == 9.0
    q = O.quantize(post, 32.0)
    assert (O.post_from_q(q, 32.0) == post).all()


def test_post_from_q_within_the_e4m3_step():
    """e4m3 keeps 4 significant bits: for scaled values in the normal range
    the decoded copy is within 2^-4 relative of post (half a step), below it
    within half the subnormal step 2^-10 / scale; plus one fp32 rounding."""
    g = np.random.default_rng(41)
    post = F.bf16(np.abs(g.standard_normal(100000)) ** 2)
    s = O.delayed_scale(float(post.max()), 2.0)
    ph = O.post_from_q(O.quantize(post, s), s)
    bound = np.maximum(2.0 ** -4 * post, 2.0 ** -10 / s) * (1 + 2.0 ** -20)
    assert (np.abs(ph - post) <= bound).all()
    assert np.abs(ph - post).max() > 0
    # the bf16-path backward on post_hat equals the calculus one on post_hat
    ins = synth.mlp_inputs(6, 32, 64, 42, with_dy=True)
    post = O.up_relu2(ins["X"], ins["W1"])
    s = O.delayed_scale(float(post.max()), 2.0)
    ph = O.post_from_q(O.quantize(post, s), s)
    a = O.mlp_bwd(ins["dY"], ins["X"], ins["W1"], ins["W2"], ph, rnd=O.exact)
    dY, W2 = F.bf16_to_f64(ins["dY"]), F.bf16_to_f64(ins["W2"])
    assert np.allclose(a["dW2"], dY.T @ ph, rtol=0, atol=1e-12)
    assert np.allclose(a["dpre"], 2 * np.sqrt(ph) * (dY @ W2), rtol=0, atol=1e-12)
