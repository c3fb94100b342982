"""GPU parity of the variant that keeps only the e4m3 copy of post: the
forward with post = NULL and mlp_relu2_bwd_fp8post.

Gates (element by element on the same seeded inputs):
  * the forward without the bf16 post writes post_q, Y, amax and scale
    bit-identical to the forward that keeps it;
  * the backward against the oracle's bf16 backward on
    post_hat = fl32(dec(post_q) * fl32(1/scale)) (the GPU's own codes):
    dX, dW1 within 4e-3 relative Frobenius (one bf16 rounding of dpre and of
    dX), dW2 within 1e-4 (fp32 accumulation only);
  * against the backward on the bf16 post (what the variant approximates),
    when nothing saturated (amax_prev = this step's exact amax): within
    5e-2, the e4m3 copy's 4 significant bits.
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


def run(fm, ins, amax_prev=None, accumulate=False, dW_init=None):
    M, d = ins["X"].shape
    h = ins["W1"].shape[0]
    X, W1, W2, dY = bf16_dev(ins["X"]), bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), bf16_dev(ins["dY"])
    W2t = torch.empty((h, d), dtype=torch.uint8, device=DEV)
    inv2 = f32_dev(0.0)
    fm.fp8_cast_transpose_w2(W2, W2t, None, inv2, None)
    if amax_prev is None:
        # bootstrap: this step's exact amax, so the e4m3 copy does not clip
        a = f32_dev(0.0)
        fm.mlp_relu2_fwd(fm.TRAIN_FP8, X, W1, W2t, inv2, None, f32_dev(1.0), 2.0,
                         torch.empty((M, h), dtype=torch.bfloat16, device=DEV),
                         torch.empty((M, h), dtype=torch.uint8, device=DEV), a, None,
                         torch.empty((M, d), dtype=torch.bfloat16, device=DEV))
        amax_prev = a.item()
    out = {}
    for keep in (True, False):
        post = torch.empty((M, h), dtype=torch.bfloat16, device=DEV) if keep else None
        post_q = torch.empty((M, h), dtype=torch.uint8, device=DEV)
        Y = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
        amax, scale = f32_dev(-1.0), f32_dev(-1.0)
        fm.mlp_relu2_fwd(fm.TRAIN_FP8, X, W1, W2t, inv2, None, f32_dev(amax_prev), 2.0, post, post_q, amax, scale, Y)
        out[keep] = {"post": None if post is None else bits(post), "post_q": post_q, "Y": bits(Y),
                     "amax": amax.item(), "scale": scale}
    g = out[False]
    dX = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    if dW_init is None:
        dW1 = torch.full((h, d), 7.0, dtype=torch.float32, device=DEV)
        dW2 = torch.full((d, h), 7.0, dtype=torch.float32, device=DEV)
    else:
        dW1 = torch.from_numpy(dW_init[0]).to(DEV)
        dW2 = torch.from_numpy(dW_init[1]).to(DEV)
    fm.mlp_relu2_bwd_fp8post(dY, X, W1, W2, g["post_q"], g["scale"], dX, dW1, dW2, accumulate)
    torch.cuda.synchronize()
    return out, {"dX": F.bf16_to_f64(bits(dX)), "dW1": dW1.cpu().numpy().astype(np.float64),
                 "dW2": dW2.cpu().numpy().astype(np.float64), "q": g["post_q"].cpu().numpy(),
                 "scale": g["scale"].item()}


def check(ins, out, b, dW_add=None):
    assert (out[True]["post_q"].cpu().numpy() == b["q"]).all()
    assert (out[True]["Y"] == out[False]["Y"]).all()
    assert f32_bits(out[True]["amax"]) == f32_bits(out[False]["amax"])
    assert f32_bits(out[True]["scale"].item()) == f32_bits(b["scale"])
    ph = O.post_from_q(b["q"], b["scale"])
    ref = O.mlp_bwd(ins["dY"], ins["X"], ins["W1"], ins["W2"], ph)
    add = (0.0, 0.0) if dW_add is None else dW_add
    assert rel_fro(b["dX"], ref["dX"]) < 4e-3
    assert rel_fro(b["dW1"], ref["dW1"] + add[0]) < 4e-3
    assert rel_fro(b["dW2"], ref["dW2"] + add[1]) < 1e-4
    if dW_add is None and O.saturation_count(b["q"]) == 0:
        full = O.mlp_bwd(ins["dY"], ins["X"], ins["W1"], ins["W2"], F.bf16_to_f64(out[True]["post"]))
        for k in ("dX", "dW1", "dW2"):
            assert rel_fro(b[k], full[k]) < 5e-2, k


def test_fp8post_tiny(fm):
    case("fp8post tiny M=256 d=128 h=512")
    ins = synth.mlp_inputs(256, 128, 512, 70, with_dy=True)
    out, b = run(fm, ins)
    check(ins, out, b)


@pytest.mark.parametrize("M,d,h", [(1, 64, 128), (255, 128, 256), (257, 192, 384), (1000, 256, 640),
                                   (777, 768, 3072)])
def test_fp8post_ragged_shapes(fm, M, d, h):
    case(f"fp8post ragged M={M} d={d} h={h}")
    ins = synth.mlp_inputs(M, d, h, 71 + M, with_dy=True)
    out, b = run(fm, ins)
    check(ins, out, b)


def _sweep_shapes():
    """Six seeded shapes: M in 1..3000, d a multiple of 64 up to 1536, h a
    multiple of 128 up to 3072."""
    rng = np.random.default_rng(2028)
    return [(int(rng.integers(1, 3001)), 64 * int(rng.integers(1, 25)), 128 * int(rng.integers(1, 25)))
            for _ in range(6)]


@pytest.mark.parametrize("M,d,h", _sweep_shapes())
def test_fp8post_shape_sweep(fm, M, d, h):
    case(f"fp8post shape sweep M={M} d={d} h={h}")
    ins = synth.mlp_inputs(M, d, h, 7000 + M, with_dy=True)
    out, b = run(fm, ins)
    check(ins, out, b)


def test_fp8post_saturating_scale(fm):
    """amax_prev far below this step's amax: the e4m3 copy clips, and the
    backward still matches the oracle run on the same codes."""
    case("fp8post with clipping")
    ins = synth.mlp_inputs(384, 128, 256, 75, with_dy=True)
    out, b = run(fm, ins, amax_prev=0.5)
    assert O.saturation_count(b["q"]) > 0
    check(ins, out, b)


def test_fp8post_accumulate(fm):
    M, d, h = 512, 128, 256
    ins = synth.mlp_inputs(M, d, h, 72, with_dy=True)
    g = np.random.default_rng(72)
    init = (g.standard_normal((h, d)).astype(np.float32), g.standard_normal((d, h)).astype(np.float32))
    case("fp8post accumulate")
    out, b = run(fm, ins, accumulate=True, dW_init=init)
    check(ins, out, b, dW_add=(init[0].astype(np.float64), init[1].astype(np.float64)))


def test_fp8post_empty(fm):
    case("fp8post M=0")
    h, d = 256, 128
    dW1 = torch.full((h, d), 5.0, dtype=torch.float32, device=DEV)
    dW2 = torch.full((d, h), 5.0, dtype=torch.float32, device=DEV)
    e = torch.empty((0, d), dtype=torch.bfloat16, device=DEV)
    W1 = torch.zeros((h, d), dtype=torch.bfloat16, device=DEV)
    W2 = torch.zeros((d, h), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((0, h), dtype=torch.uint8, device=DEV)
    fm.mlp_relu2_bwd_fp8post(e, e, W1, W2, q, f32_dev(1.0), e, dW1, dW2)
    torch.cuda.synchronize()
    assert float(dW1.abs().max()) == 0.0 and float(dW2.abs().max()) == 0.0


def test_fp8post_block_and_stack(fm):
    """Relu2MLP(keep_post=False) returns no post and its backward equals the
    direct call; a two-layer stack trains with every layer on its e4m3 copy."""
    from fp8_relu_mlp_amd.stack import Relu2Stack
    M, d, h = 512, 128, 256
    ins = synth.mlp_inputs(M, d, h, 73, with_dy=True)
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), amax_init=2.0, keep_post=False)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    case("fp8post block")
    Y, post, post_q = blk.forward(X)
    assert post is None
    dX, dW1, dW2 = blk.backward(dY, X, None, post_q=post_q)
    torch.cuda.synchronize()
    ph = O.post_from_q(post_q.cpu().numpy(), blk.scale_used.item())
    ref = O.mlp_bwd(ins["dY"], ins["X"], ins["W1"], ins["W2"], ph)
    assert rel_fro(F.bf16_to_f64(bits(dX)), ref["dX"]) < 4e-3
    assert rel_fro(dW2.cpu().numpy().astype(np.float64), ref["dW2"]) < 1e-4
    wts = synth.stack_weights(2, d, h, 74)
    stk = Relu2Stack([bf16_dev(w1) for w1, _ in wts], [bf16_dev(w2) for _, w2 in wts], lr=1e-2, keep_post=False,
                     telemetry=True)
    for t in range(2):
        bt = synth.stack_batch(M, d, 74, t)
        case(f"fp8post stack step {t}")
        st = stk.step(bf16_dev(bt["X"]), bf16_dev(bt["dY"])).cpu().numpy()
        assert np.isfinite(st).all()
        assert all(torch.isfinite(blk_.W1.float()).all() and torch.isfinite(blk_.W2.float()).all()
                   for blk_ in stk.layers)


def test_fp8up_without_bf16_post(fm):
    """Both variants at once (M=4096, d=768, h=3072): the e4m3 up-projection
    writing only post_q gives the same codes, amax and Y as with post kept,
    and the backward on those codes matches the oracle on post_hat."""
    M, d, h = 4096, 768, 3072
    ins = synth.mlp_inputs(M, d, h, 76, with_dy=True)
    case("fp8up + fp8post, block pair")
    W1, W2 = bf16_dev(ins["W1"]), bf16_dev(ins["W2"])
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    keep = fm.Relu2MLP(W1, W2, amax_init=1.0, fp8_up=True)
    drop = fm.Relu2MLP(W1, W2, amax_init=1.0, fp8_up=True, keep_post=False)
    for blk in (keep, drop):
        blk.forward(X)                                   # bootstrap both amaxes
    Yk, post_k, q_k = keep.forward(X)
    Yd, post_d, q_d = drop.forward(X)
    dX, dW1, dW2 = drop.backward(dY, X, None, post_q=q_d)
    torch.cuda.synchronize()
    assert post_d is None
    assert (q_k.cpu().numpy() == q_d.cpu().numpy()).all()
    assert (bits(Yk) == bits(Yd)).all()
    assert f32_bits(keep.amax_last.item()) == f32_bits(drop.amax_last.item())
    ph = O.post_from_q(q_d.cpu().numpy(), drop.scale_used.item())
    ref = O.mlp_bwd(ins["dY"], ins["X"], ins["W1"], ins["W2"], ph)
    assert rel_fro(F.bf16_to_f64(bits(dX)), ref["dX"]) < 4e-3
    assert rel_fro(dW1.cpu().numpy().astype(np.float64), ref["dW1"]) < 4e-3
    assert rel_fro(dW2.cpu().numpy().astype(np.float64), ref["dW2"]) < 1e-4
