"""GPU parity of fp8_linear (FP8 QKV / output projections) against the oracle.

Gates: Y within relative Frobenius 2e-2 of the oracle (an e4m3 GEMM is in its
lineage) and, since the GPU quantises X with the same fp32 product and RNE
encode as the oracle, within the bf16 output rounding (4e-3) as well; the
optional amax of X is bit-exact; the ternary special case is exact.
"""
import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth
from oracle import formats as F
from oracle import mlp as O

from .gpu_helpers import DEV, bf16_dev, bits, case, f32_bits, f32_dev, rel_fro

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    import fp8_relu_mlp_amd as fm
    fm.lib()
    return fm


def run_linear(fm, Xb, Wb, margin=1.0, scale_in=None):
    """Exact per-tensor scales: amax_reduce + fp8_scale_from_amax for X,
    fp8_cast_transpose (exact policy) for W; returns GPU outputs."""
    M, K = Xb.shape
    N = Wb.shape[0]
    X, W = bf16_dev(Xb), bf16_dev(Wb)
    Wt = torch.empty((K, N), dtype=torch.uint8, device=DEV)
    inv_w = f32_dev(0.0)
    if scale_in is None:
        fm.fp8_cast_transpose(W, Wt, inv_scale_out=inv_w)
    else:
        fm.fp8_cast_transpose(W, Wt, scale_in=f32_dev(scale_in), inv_scale_out=inv_w)
    amax = f32_dev(0.0)
    fm.amax_reduce(X, amax)
    sx = f32_dev(0.0)
    fm.fp8_scale_from_amax(amax, margin, sx)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    xam = f32_dev(-1.0)
    fm.fp8_linear(X, sx, Wt, inv_w, Y, xam)
    torch.cuda.synchronize()
    return {"Y": bits(Y), "sx": sx.item(), "inv_w": inv_w.item(), "Wt": Wt.cpu().numpy(), "xamax": xam.item()}


# K = 64, 320: not whole 128-code k-tiles (the e4m3 rows are padded).  K <=
# 768 runs the row-panel kernel: (8192, 768, 2304) and (40000, 128, 512) give
# its blocks several output tiles each, with changes of row panel inside a
# block (the second with two 64-k tiles per output tile); (3000, 768, 320)
# has a part-filled last column tile.  K = 1024 runs the two-launch path,
# K = 960 the same with e4m3 rows padded to 1024 codes.
@pytest.mark.parametrize("M,K,N", [(1000, 768, 2304), (777, 768, 768), (1, 128, 64), (300, 256, 192),
                                   (513, 64, 128), (1000, 320, 576), (8192, 768, 2304), (40000, 128, 512),
                                   (3000, 768, 320), (600, 1024, 256), (400, 960, 192)])
def test_fp8_linear_parity(fm, M, K, N):
    case(f"fp8_linear M={M} K={K} N={N}")
    a = synth.attn_inputs(M=M, d=K, qkv=N, seed=90 + M)
    g = run_linear(fm, a["X"], a["Wqkv"])
    Xf = F.bf16_to_f64(a["X"])
    assert f32_bits(g["xamax"]) == f32_bits(O.amax(Xf))
    sx = O.exact_scale(O.amax(Xf))
    assert f32_bits(g["sx"]) == f32_bits(sx)
    Wt, _, inv_w, _ = O.cast_transpose(a["Wqkv"])
    assert (Wt == g["Wt"]).all()
    ref = F.bf16_to_f64(O.fp8_linear(a["X"], sx, Wt, inv_w))
    Y = F.bf16_to_f64(g["Y"])
    assert rel_fro(Y, ref) < 4e-3
    assert rel_fro(Y, ref) < 2e-2
    # sanity against the unquantised product: two e4m3 roundings with an RMS
    # relative error of about 0.03 each give about 0.04; allow twice that
    exact = Xf @ F.bf16_to_f64(a["Wqkv"]).T
    assert rel_fro(Y, exact) < 0.08


def _sweep_shapes():
    """Eight seeded shapes: M in 1..20000, K a multiple of 64 up to 1536 (the
    row-panel kernel up to 768, the two-launch path above), N a multiple of
    64 up to 3072."""
    rng = np.random.default_rng(2029)
    return [(int(rng.integers(1, 20001)), 64 * int(rng.integers(1, 25)), 64 * int(rng.integers(1, 49)))
            for _ in range(8)]


@pytest.mark.parametrize("M,K,N", _sweep_shapes())
def test_fp8_linear_shape_sweep(fm, M, K, N):
    case(f"fp8_linear shape sweep M={M} K={K} N={N}")
    a = synth.attn_inputs(M=M, d=K, qkv=N, seed=8000 + M)
    g = run_linear(fm, a["X"], a["Wqkv"])
    Xf = F.bf16_to_f64(a["X"])
    assert f32_bits(g["xamax"]) == f32_bits(O.amax(Xf))
    sx = O.exact_scale(O.amax(Xf))
    Wt, _, inv_w, _ = O.cast_transpose(a["Wqkv"])
    assert (Wt == g["Wt"]).all()
    ref = F.bf16_to_f64(O.fp8_linear(a["X"], sx, Wt, inv_w))
    assert rel_fro(F.bf16_to_f64(g["Y"]), ref) < 4e-3


@pytest.mark.parametrize("K", [256, 192])
def test_fp8_linear_lossless(fm, K):
    M, N = 500, 128
    X = synth.ternary_bf16((M, K), 5, "X")
    W = synth.ternary_bf16((N, K), 5, "W")
    case(f"fp8_linear lossless ternary K={K}")
    g = run_linear(fm, X, W, margin=448.0, scale_in=1.0)      # scale 448/(448*1) = 1
    assert g["sx"] == 1.0
    y = F.bf16_to_f64(X).astype(np.int64) @ F.bf16_to_f64(W).astype(np.int64).T
    assert np.abs(y).max() <= 256
    assert (F.bf16_to_f64(g["Y"]) == y).all()


def test_fp8_linear_empty(fm):
    case("fp8_linear M=0")
    X = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    Wt = torch.zeros((256, 128), dtype=torch.uint8, device=DEV)
    Y = torch.empty((0, 128), dtype=torch.bfloat16, device=DEV)
    am = f32_dev(5.0)
    fm.fp8_linear(X, f32_dev(1.0), Wt, f32_dev(1.0), Y, am)
    torch.cuda.synchronize()
    assert am.item() == 0.0


@pytest.mark.parametrize("with_nan", [True, False])
def test_fp8_linear_special_values(fm, with_nan):
    """Non-finite and out-of-range activations: the e4m3 conversion saturates
    +-inf and values past 448 to +-448, a NaN stays a NaN code (so its row of Y
    is NaN), and max |X| is NaN if any element is, else +inf."""
    M, K, N = 300, 256, 192
    case(f"fp8_linear special values nan={with_nan}")
    a = synth.attn_inputs(M=M, d=K, qkv=N, seed=77)
    Xb = a["X"].copy()
    specials = {(130, 3): np.inf, (131, 200): -np.inf, (250, 0): 1e30, (251, 9): -3e4}
    if with_nan:
        specials[(5, 17)] = np.nan
    for (r, c), v in specials.items():
        Xb[r, c] = synth.to_bf16_bits(np.array([v], dtype=np.float32))[0]
    Wt, _, inv_w, _ = O.cast_transpose(a["Wqkv"])
    sx = 0.5
    X = bf16_dev(Xb)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    xam = f32_dev(-1.0)
    fm.fp8_linear(X, f32_dev(sx), torch.from_numpy(Wt).to(DEV), f32_dev(inv_w), Y, xam)
    torch.cuda.synchronize()
    ref = F.bf16_to_f64(O.fp8_linear(Xb, sx, Wt, inv_w))
    got = F.bf16_to_f64(bits(Y))
    assert (np.isnan(got) == np.isnan(ref)).all()
    fin = ~np.isnan(ref)
    assert np.isfinite(got[fin]).all()
    assert rel_fro(got[fin], ref[fin]) < 4e-3
    if with_nan:
        assert np.isnan(xam.item())
    else:
        assert xam.item() == np.inf
