"""GPU parity: amax reduction, device scale computation, weight cast-transpose.

All of these are bit-exact against the CPU oracle (integer / code / exact-max
work): amax is a max of magnitudes, the scale is one correctly rounded fp32
product and quotient, the codes are round-to-nearest-even e4m3 of one fp32
product.
"""
import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth
from oracle import formats as F
from oracle import mlp as O

from .gpu_helpers import DEV, bf16_dev, case, f32_bits, f32_dev, same_codes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    import fp8_relu_mlp_amd as fm
    fm.lib()
    return fm


@pytest.mark.parametrize("n", [0, 1, 7, 1000, 65536, 65537, (1 << 22) + 3])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_amax_reduce(fm, n, dtype):
    case(f"amax_reduce {dtype} n={n}")
    g = np.random.default_rng(n + 17)
    x = (g.standard_normal(n) * 3.0).astype(np.float32)
    if n > 10:
        x[n // 3] = -1234.5          # the largest magnitude is negative
    if dtype == "f32":
        t = torch.from_numpy(x).to(DEV)
        ref = O.amax(x.astype(np.float64))
    else:
        b = synth.to_bf16_bits(x)
        t = bf16_dev(b)
        ref = O.amax(F.bf16_to_f64(b))
    out = f32_dev(-1.0)
    fm.amax_reduce(t, out)
    torch.cuda.synchronize()
    assert f32_bits(out.item()) == f32_bits(ref)


@pytest.mark.parametrize("special", ["nan", "inf"])
def test_amax_reduce_specials(fm, special):
    case(f"amax_reduce special {special}")
    x = np.linspace(-5, 5, 100001).astype(np.float32)
    x[777] = np.nan if special == "nan" else -np.inf
    out = f32_dev(0.0)
    fm.amax_reduce(torch.from_numpy(x).to(DEV), out)
    torch.cuda.synchronize()
    got = out.item()
    if special == "nan":
        assert np.isnan(got)
    else:
        assert got == np.inf


def test_scale_from_amax_bit_exact(fm):
    case("fp8_scale_from_amax sweep")
    g = np.random.default_rng(5)
    amaxes = list(np.float32(np.abs(g.standard_normal(300)) * 10.0 ** g.integers(-8, 8, 300)))
    amaxes += [0.0, -1.0, float("nan"), float("inf"), 1e-38, 7.0, 448.0, 3.4e38, 1.17e-38]
    a_dev = torch.tensor(amaxes, dtype=torch.float32, device=DEV)
    s_dev = torch.zeros(len(amaxes), dtype=torch.float32, device=DEV)
    i_dev = torch.zeros(len(amaxes), dtype=torch.float32, device=DEV)
    for margin in (1.0, 2.0, 1.5):
        for i in range(len(amaxes)):
            fm.fp8_scale_from_amax(a_dev[i:i + 1], margin, s_dev[i:i + 1], i_dev[i:i + 1])
        torch.cuda.synchronize()
        s, inv = s_dev.cpu().numpy(), i_dev.cpu().numpy()
        for i, a in enumerate(amaxes):
            rs = O.delayed_scale(float(a), margin)
            assert f32_bits(s[i]) == f32_bits(rs), (a, margin, s[i], rs)
            assert f32_bits(inv[i]) == f32_bits(O.inv_scale(rs))


@pytest.mark.parametrize("scale", [1.0, 32.0, 448.0 / 13.7, 0.37, 2.0 ** -7])
def test_cast_transpose_all_bf16_patterns(fm, scale):
    case(f"fp8_cast_transpose all bf16 patterns scale={scale}")
    W = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(256, 256)
    Wd = bf16_dev(W)
    out = torch.empty((256, 256), dtype=torch.uint8, device=DEV)
    s_in = f32_dev(scale)
    s_out, inv_out = f32_dev(0.0), f32_dev(0.0)
    fm.fp8_cast_transpose(Wd, out, scale_in=s_in, scale_out=s_out, inv_scale_out=inv_out)
    torch.cuda.synchronize()
    ref, rs, rinv, _ = O.cast_transpose(W, scale_in=scale)
    assert same_codes(out.cpu().numpy(), ref)
    assert f32_bits(s_out.item()) == f32_bits(rs)
    assert f32_bits(inv_out.item()) == f32_bits(rinv)


@pytest.mark.parametrize("shape", [(768, 3072), (3072, 768), (2304, 768), (48, 80), (1040, 784), (2064, 4096)])
def test_cast_transpose_exact_scale(fm, shape):
    N, K = shape
    case(f"fp8_cast_transpose exact N={N} K={K}")
    W = synth.normal_bf16((N, K), 1.0 / K, 31, f"W.{N}.{K}")
    out = torch.empty((K, N), dtype=torch.uint8, device=DEV)
    s, inv, am = f32_dev(0.0), f32_dev(0.0), f32_dev(0.0)
    fm.fp8_cast_transpose(bf16_dev(W), out, scale_out=s, inv_scale_out=inv, amax_out=am)
    torch.cuda.synchronize()
    ref, rs, rinv, ra = O.cast_transpose(W)
    assert (out.cpu().numpy() == ref).all()
    assert f32_bits(s.item()) == f32_bits(rs)
    assert f32_bits(inv.item()) == f32_bits(rinv)
    assert f32_bits(am.item()) == f32_bits(ra)


def test_cast_transpose_w2_matches_generic(fm):
    case("fp8_cast_transpose_w2 c3 W2")
    d, h = 768, 3072
    W2 = synth.mlp_inputs(8, d, h, 2)["W2"]
    out = torch.empty((h, d), dtype=torch.uint8, device=DEV)
    s, inv, am = f32_dev(0.0), f32_dev(0.0), f32_dev(0.0)
    fm.fp8_cast_transpose_w2(bf16_dev(W2), out, s, inv, am)
    torch.cuda.synchronize()
    ref, rs, rinv, ra = O.cast_transpose(W2)
    assert (out.cpu().numpy() == ref).all()
    assert (f32_bits(s.item()), f32_bits(inv.item()), f32_bits(am.item())) == \
        (f32_bits(rs), f32_bits(rinv), f32_bits(ra))


def test_mfma_probe_runs():
    """The matrix-core rate probe runs on bf16 and e4m3 operands and writes its
    sink (a measurement aid; its flop count is what the benchmark divides)."""
    import fp8_relu_mlp_amd as fm
    case("mfma probe")
    a = torch.randn(1 << 16, device=DEV).to(torch.bfloat16)
    b = torch.randn(1 << 16, device=DEV).to(torch.bfloat16)
    sink = torch.zeros(fm.PROBE_BLOCKS * 256, dtype=torch.float32, device=DEV)
    assert fm.mfma_probe(fm.MFMA_BF16, a, b, 10, sink) == fm.PROBE_BLOCKS * 4 * 16 * 10 * 32768
    torch.cuda.synchronize()
    assert (sink != 0).any()
    q = torch.randint(0, 0x77, (1 << 16,), dtype=torch.uint8, device=DEV)
    sink.zero_()
    assert fm.mfma_probe(fm.MFMA_E4M3, q, q, 10, sink) == fm.PROBE_BLOCKS * 4 * 16 * 10 * 131072
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
