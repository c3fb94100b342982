"""GPU parity of mlp_relu2_fwd_fp8up (both MLP GEMMs in e4m3 on the training
forward) against the CPU oracle.

Gates (element by element on the same seeded inputs):
  * x_amax_out, amax_out and scale_out bit-exact (max |X|, the max of the
    GPU's own post, the delayed-scale formula);
  * the transposed W1 cache bit-exact against the oracle's cast;
  * post within a bound derived per element from the arithmetic: both sides
    quantise X to the same codes (fp32(X * sx) is one correctly rounded
    product), the oracle sums the e4m3 products exactly, the matrix core
    with its own alignment window (``acc_bound``), then two fp32
    dequantisation products, relu^2 and one bf16 rounding on each side;
    and within 1e-2 relative Frobenius error of the oracle's post;
  * post_q codes bit-exact given the GPU's post; Y within the bf16 output
    rounding of the oracle's exact FP8 GEMM on the GPU's codes (< 4e-3
    Frobenius) and within 2e-2 of the oracle run on its own;
  * the lossless special case (ternary X and W1, unit scales) exact.
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


def fexp(v):
    """Exponent field of e4m3 magnitudes as the matrix core aligns them:
    floor(log2 v) for normal values, -6 for subnormal ones (0 for 0)."""
    v = np.asarray(v, dtype=np.float64)
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    return np.where(v > 0, np.maximum(e, -6.0), -np.inf)


def acc_bound(xq, w, slice_k=128):
    """Bound on |acc_gpu - acc_exact| for acc = xq . w (e4m3 values, [M,K] x
    [K,N]) on the gfx950 e4m3 matrix core.  One instruction sums 64 products
    at a time and adds the sum to the fp32 accumulator; inside the
    instruction the products are aligned to the largest one and bits more
    than 13 places below its leading bit are dropped (an in-bounds check of
    single instructions: +2^e - 2^e + 2^-18 gives 2^-18 for e <= -5 and 0
    for e >= -4; 2^e + 3*2^-18 gives 2^e + 2^-17 at e = -4).  The leading bit
    of a product lies at most one place above fexp(x) + fexp(w), so each
    product loses < 2^(fexp(x) + fexp(w) + 1 - 13); which 64 products of a
    128-deep k-slice share an instruction is left open, so the slice's
    largest operands bound every product in it.  The fp32 add of each
    instruction's sum to the accumulator adds one rounding (2^-24 relative)
    of a partial sum bounded by sum |xq w|."""
    M, K = xq.shape
    S = K // slice_k
    ax, aw = np.abs(xq), np.abs(w)
    mx = ax.reshape(M, S, slice_k).max(axis=2)
    mw = aw.reshape(S, slice_k, -1).max(axis=1)
    px = np.where(mx > 0, np.exp2(fexp(mx)), 0.0)
    pw = np.where(mw > 0, np.exp2(fexp(mw)), 0.0)
    trunc = slice_k * 2.0 ** (1 - 13) * (px @ pw)
    return trunc + (K // 64) * 2.0 ** -24 * (ax @ aw)


def post_bound(X_bits, sx, W1t, inv1):
    """Per-element bound on |post_gpu - post_oracle|: the accumulation bound
    above, the two fp32 dequantisation products (2^-24 relative each), then
    relu^2 and one bf16 rounding (2^-9 relative) on each side."""
    X = F.bf16_to_f64(X_bits)
    xq = F.e4m3_decode(F.e4m3_encode(F.fl32(X * sx)))
    w = F.e4m3_decode(W1t)
    a = O.inv_scale(sx) * inv1
    _, _, pre = O.up_relu2_fp8(X_bits, sx, W1t, inv1)
    E = acc_bound(xq, w) * a * 1.001 + 2.0 ** -22 * np.abs(pre)
    r = np.maximum(pre, 0.0)
    return 2.0 ** -9 * ((r + E) ** 2 * 1.001 + r * r) + (2 * r + E) * E * 1.001 + 1e-45


def run(fm, ins, sx, amax_prev, margin=2.0, w_scale_in=None):
    M, d = ins["X"].shape
    h = ins["W1"].shape[0]
    W1t = torch.empty((d, h), dtype=torch.uint8, device=DEV)
    W2t = torch.empty((h, d), dtype=torch.uint8, device=DEV)
    inv1, inv2 = f32_dev(0.0), f32_dev(0.0)
    si = None if w_scale_in is None else f32_dev(w_scale_in)
    fm.fp8_cast_transpose(bf16_dev(ins["W1"]), W1t, scale_in=si, inv_scale_out=inv1)
    fm.fp8_cast_transpose(bf16_dev(ins["W2"]), W2t, scale_in=si, inv_scale_out=inv2)
    post = torch.empty((M, h), dtype=torch.bfloat16, device=DEV)
    post_q = torch.empty((M, h), dtype=torch.uint8, device=DEV)
    Y = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    amax_out, scale_out, x_amax = f32_dev(-7.0), f32_dev(-7.0), f32_dev(-7.0)
    fm.mlp_relu2_fwd_fp8up(bf16_dev(ins["X"]), f32_dev(sx), W1t, inv1, W2t, inv2, f32_dev(amax_prev), margin,
                           post, post_q, amax_out, scale_out, Y, x_amax_out=x_amax)
    torch.cuda.synchronize()
    return {"post": bits(post), "post_q": post_q.cpu().numpy(), "y": bits(Y), "amax": amax_out.item(),
            "scale": scale_out.item(), "x_amax": x_amax.item(), "W1t": W1t.cpu().numpy(),
            "W2t": W2t.cpu().numpy(), "inv1": inv1.item(), "inv2": inv2.item()}


def check(ins, g, sx, amax_prev, margin=2.0):
    X = F.bf16_to_f64(ins["X"])
    post = F.bf16_to_f64(g["post"])
    assert f32_bits(g["x_amax"]) == f32_bits(np.abs(X).max() if X.size else 0.0)
    assert f32_bits(g["amax"]) == f32_bits(post.max() if post.size else 0.0)
    s = O.delayed_scale(amax_prev, margin)
    assert f32_bits(g["scale"]) == f32_bits(s)
    W1t, _, inv1, _ = O.cast_transpose(ins["W1"])
    W2t, _, inv2, _ = O.cast_transpose(ins["W2"])
    assert (W1t == g["W1t"]).all() and (W2t == g["W2t"]).all()
    ref_post, _, _ = O.up_relu2_fp8(ins["X"], sx, W1t, inv1)
    bound = post_bound(ins["X"], sx, W1t, inv1)
    err = np.abs(post - ref_post)
    assert (err <= bound).all(), f"post off by {float((err - bound).max())} beyond the bound"
    assert (O.quantize(post, s) == g["post_q"]).all()
    y = F.bf16_to_f64(g["y"])
    assert rel_fro(y, O.down_fp8(g["post_q"], W2t, O.inv_scale(s), inv2)) < 4e-3
    ref = O.mlp_fwd_fp8up(ins["X"], sx, W1t, inv1, W2t, inv2, amax_prev, margin)
    assert rel_fro(post, F.bf16_to_f64(ref["post"])) < 1e-2
    assert rel_fro(y, F.bf16_to_f64(ref["y"])) < 2e-2


def test_fp8up_tiny(fm):
    """Tiny workload X[256,128], W1[512,128], W2[128,512]: exact X scale
    (448 / max|X|), amax_prev from a first call."""
    ins = synth.mlp_inputs(256, 128, 512, 0)
    sx = O.exact_scale(O.amax(F.bf16_to_f64(ins["X"])))
    case("fp8up tiny bootstrap call")
    g0 = run(fm, ins, sx, 1.0)
    case("fp8up tiny")
    g = run(fm, ins, sx, g0["amax"])
    assert (g["post"] == g0["post"]).all()
    check(ins, g, sx, g0["amax"])


@pytest.mark.parametrize("M,d,h", [(1, 128, 128), (255, 128, 256), (257, 256, 384), (1000, 256, 640),
                                   (777, 768, 3072)])
def test_fp8up_ragged_shapes(fm, M, d, h):
    case(f"fp8up ragged M={M} d={d} h={h}")
    ins = synth.mlp_inputs(M, d, h, 60 + M)
    sx = O.delayed_scale(O.amax(F.bf16_to_f64(ins["X"])), 2.0)
    g = run(fm, ins, sx, 3.0)
    check(ins, g, sx, 3.0)


def _sweep_shapes():
    """Six seeded shapes: M in 1..3000, d and h multiples of 128 (the e4m3
    contractions) up to 1536 and 3072."""
    rng = np.random.default_rng(2027)
    return [(int(rng.integers(1, 3001)), 128 * int(rng.integers(1, 13)), 128 * int(rng.integers(1, 25)))
            for _ in range(6)]


@pytest.mark.parametrize("M,d,h", _sweep_shapes())
def test_fp8up_shape_sweep(fm, M, d, h):
    case(f"fp8up shape sweep M={M} d={d} h={h}")
    ins = synth.mlp_inputs(M, d, h, 6000 + M)
    sx = O.delayed_scale(O.amax(F.bf16_to_f64(ins["X"])), 2.0)
    g = run(fm, ins, sx, 2.5)
    check(ins, g, sx, 2.5)


def test_fp8up_lossless_special_case(fm):
    """X, W1 in {-1,0,1} (<= 3 non-zeros per W1 row), W2 in {-1,0,1}, the X
    and weight scales 1, amax_prev 7, margin 2: every quantisation is exact,
    so post and Y equal the integer results bit for bit."""
    M, d, h, dd = 300, 128, 256, 128
    X = synth.ternary_bf16((M, d), 8, "X")
    W1 = synth.ternary_bf16((h, d), 8, "W1", nnz_per_row=3)
    W2 = synth.ternary_bf16((dd, h), 8, "W2")
    case("fp8up lossless special case")
    g = run(fm, {"X": X, "W1": W1, "W2": W2}, 1.0, 7.0, w_scale_in=1.0)
    pre = F.bf16_to_f64(X).astype(np.int64) @ F.bf16_to_f64(W1).astype(np.int64).T
    post = np.maximum(pre, 0) ** 2
    y = post @ F.bf16_to_f64(W2).astype(np.int64).T
    assert g["scale"] == 32.0 and g["inv1"] == 1.0
    assert (F.bf16_to_f64(g["post"]) == post).all()
    assert (F.e4m3_decode(g["post_q"]) == post * 32).all()
    assert (F.bf16_to_f64(g["y"]) == y).all()


def test_fp8up_empty(fm):
    case("fp8up M=0")
    ins = synth.mlp_inputs(0, 128, 256, 61)
    g = run(fm, ins, 1.0, 2.0)
    assert g["amax"] == 0.0 and g["x_amax"] == 0.0
    assert f32_bits(g["scale"]) == f32_bits(O.delayed_scale(2.0, 2.0))


def test_fp8up_x_saturation(fm):
    """An X scale four times too large clips the largest inputs to 448 on
    both sides; the parity bound still holds."""
    M, d, h = 384, 128, 256
    ins = synth.mlp_inputs(M, d, h, 62)
    sx = 4 * O.exact_scale(O.amax(F.bf16_to_f64(ins["X"])))
    case("fp8up X saturation")
    g = run(fm, ins, sx, 3.0)
    check(ins, g, sx, 3.0)


def test_fp8up_block_state_carry(fm):
    """Relu2MLP(fp8_up=True): the forward derives the X scale from the
    previous call's max |X| with the margin, and carries both amaxes."""
    M, d, h = 512, 256, 512
    ins = synth.mlp_inputs(M, d, h, 63)
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0, fp8_up=True)
    X = bf16_dev(ins["X"])
    case("fp8up block: bootstrap")
    blk.forward(X)
    xa, a = float(blk.x_amax_prev.item()), float(blk.amax_prev.item())
    assert f32_bits(xa) == f32_bits(np.abs(F.bf16_to_f64(ins["X"])).max())
    case("fp8up block: second step")
    Y, post, post_q = blk.forward(X)
    torch.cuda.synchronize()
    sx = O.delayed_scale(xa, 2.0)
    assert f32_bits(blk.x_scale.item()) == f32_bits(sx)
    g = {"post": bits(post), "post_q": post_q.cpu().numpy(), "y": bits(Y), "amax": blk.amax_last.item(),
         "scale": blk.scale_used.item(), "x_amax": blk.x_amax_prev.item(), "W1t": blk.W1t_q.cpu().numpy(),
         "W2t": blk.W2t_q.cpu().numpy()}
    check(ins, g, sx, a)


def test_e4m3_accumulation_window_within_bound(fm):
    """The premise of ``acc_bound`` through the library's own e4m3 GEMM
    (fp8_linear, unit scales): row r of X holds +2^e, -2^e and 2^-9 in
    k = 0, 1, 2 (one 16-byte k-run, hence one instruction) and W's column 0
    holds 1, 1, 2^-9, so the exact dot product is 2^-18.  Every result must
    lie within the bound, and for e <= -5 (the tiny product inside the
    13-place window) be exact."""
    K, N = 128, 64
    es = np.arange(-9, 9)
    X = np.zeros((len(es), K))
    X[:, 0], X[:, 1], X[:, 2] = 2.0 ** es, -(2.0 ** es), 2.0 ** -9
    W = np.zeros((N, K))
    W[0, 0] = W[0, 1] = 1.0
    W[0, 2] = 2.0 ** -9
    Xb, Wb = synth.to_bf16_bits(X), synth.to_bf16_bits(W)
    case("e4m3 accumulation window via fp8_linear")
    Wt = torch.empty((K, N), dtype=torch.uint8, device=DEV)
    inv = f32_dev(0.0)
    fm.fp8_cast_transpose(bf16_dev(Wb), Wt, scale_in=f32_dev(1.0), inv_scale_out=inv)
    Y = torch.empty((len(es), N), dtype=torch.bfloat16, device=DEV)
    fm.fp8_linear(bf16_dev(Xb), f32_dev(1.0), Wt, inv, Y)
    torch.cuda.synchronize()
    y = F.bf16_to_f64(bits(Y))[:, 0]
    bound = acc_bound(X, W.T.copy())[:, 0]
    assert (np.abs(y - 2.0 ** -18) <= bound).all()
    assert (y[es <= -5] == 2.0 ** -18).all()
    print("[window] e:", es.tolist(), "kept:", (y == 2.0 ** -18).tolist(), flush=True)
