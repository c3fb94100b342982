"""GPU parity of the scaling-policy variants and the clip-rate telemetry:

  * fp8_saturation_count bit-exact against the oracle's count (random codes,
    a ragged length, n = 0, and the e4m3 post copy of a clipping forward);
  * the rolling amax window: every step's scale bit-exact against the
    delayed scale of the maximum of the last L amaxes the GPU measured (each
    of them bit-exact against the max of that step's GPU post);
  * the delayed W2 scale: the refreshed cache bit-exact against the oracle's
    cast with the previous refresh's max|W2| times the margin;
  * a small stack with every option on: the telemetry counts bit-exact
    against the codes the layers wrote, the state carried as specified.
"""
import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth
from oracle import formats as F
from oracle import mlp as O

from .gpu_helpers import DEV, bf16_dev, bits, case, f32_bits, u8_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    import fp8_relu_mlp_amd as fm
    fm.lib()
    return fm


def gpu_count(fm, q_dev):
    out = torch.full((1,), -1, dtype=torch.int64, device=DEV)
    fm.fp8_saturation_count(q_dev, out)
    torch.cuda.synchronize()
    return int(out.item())


@pytest.mark.parametrize("n", [0, 16, 4096 + 48, 1 << 22])
def test_saturation_count_random_codes(fm, n):
    case(f"saturation count n={n}")
    g = np.random.default_rng(n + 5)
    q = g.integers(0, 256, size=n).astype(np.uint8)
    q[g.random(n) < 0.01] = 0x7E
    assert gpu_count(fm, u8_dev(q)) == O.saturation_count(q)


def test_saturation_count_of_a_clipping_forward(fm):
    """M=4096 forward with amax_prev a third of the true amax: the count of
    top codes in post_q equals the oracle's, and equals the number of scaled
    post values >= 432."""
    M, d, h = 4096, 768, 3072
    ins = synth.mlp_inputs(M, d, h, 33)
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0)
    X = bf16_dev(ins["X"])
    case("saturation count: bootstrap")
    blk.forward(X)
    a = float(blk.amax_prev.item()) / 3
    blk.amax_prev.fill_(a)
    case("saturation count: clipping forward")
    _, post, post_q = blk.forward(X, carry=False)
    n = gpu_count(fm, post_q)
    q = post_q.cpu().numpy()
    assert n == O.saturation_count(q) > 0
    v = (F.bf16_to_f64(bits(post)) * O.delayed_scale(a, 2.0)).astype(np.float32)
    assert n == int(np.count_nonzero(v >= 432.0))


def test_rolling_amax_window(fm):
    """Relu2MLP(amax_window=3) over 6 steps whose inputs are scaled by
    different factors: step t's scale comes from the max of the amaxes of
    steps t-3 .. t-1 (the initial amax_prev for the first step)."""
    M, d, h = 512, 256, 512
    ins = synth.mlp_inputs(M, d, h, 34)
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=5.0, amax_window=3)
    factors = [1.0, 2.0, 0.5, 0.25, 1.5, 0.5]
    measured = []
    for t, fct in enumerate(factors):
        Xb = synth.to_bf16_bits(F.bf16_to_f64(ins["X"]) * fct)
        case(f"rolling window step {t}")
        _, post, _ = blk.forward(bf16_dev(Xb))
        torch.cuda.synchronize()
        window = measured[-3:] if measured else [5.0]
        assert f32_bits(blk.scale_used.item()) == f32_bits(O.window_scale(window, 2.0))
        a = float(blk.amax_last.item())
        assert f32_bits(a) == f32_bits(F.bf16_to_f64(bits(post)).max())
        measured.append(a)
        assert f32_bits(blk.amax_prev.item()) == f32_bits(max(measured[-3:]))


def test_delayed_w2_scale(fm):
    d, h = 768, 3072
    ins = synth.mlp_inputs(16, d, h, 35)
    W2 = bf16_dev(ins["W2"])
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), W2, margin=2.0, amax_init=1.0, w2_scale="delayed", w2_margin=1.5)
    torch.cuda.synchronize()
    c0 = O.cast_transpose(ins["W2"])                       # the first refresh is exact
    assert (blk.W2t_q.cpu().numpy() == c0[0]).all()
    assert f32_bits(blk.w2_amax.item()) == f32_bits(c0[3])
    prev = c0[3]
    for t, fct in enumerate([1.25, 0.5, 3.0]):
        Wn = synth.to_bf16_bits(F.bf16_to_f64(ins["W2"]) * fct)
        W2.copy_(bf16_dev(Wn))
        case(f"delayed W2 refresh {t}")
        blk.refresh_w2_cache()
        torch.cuda.synchronize()
        codes, s, inv, a = O.delayed_cast_transpose(Wn, prev, 1.5)
        assert (blk.W2t_q.cpu().numpy() == codes).all()
        assert f32_bits(blk.w2_scale.item()) == f32_bits(s)
        assert f32_bits(blk.w2_inv_scale.item()) == f32_bits(inv)
        assert f32_bits(blk.w2_amax.item()) == f32_bits(a)
        prev = a


def test_stack_with_policies_and_telemetry(fm):
    """Two layers, three steps, fp8 up-projection, window 2, delayed W2
    scale, telemetry on: each layer's count equals the oracle's count of
    the codes that layer wrote, every scale is the delayed scale of the
    amax_prev it used, and from the third step on amax_prev is the max of
    the two amaxes measured before (the first step's window also holds the
    bootstrap measurement)."""
    from fp8_relu_mlp_amd.stack import Relu2Stack
    M, d, h, L = 1024, 256, 512, 2
    wts = synth.stack_weights(L, d, h, 36)
    stk = Relu2Stack([bf16_dev(w1) for w1, _ in wts], [bf16_dev(w2) for _, w2 in wts], lr=1e-2, fp8_up=True,
                     amax_window=2, w2_scale="delayed", w2_margin=1.25, telemetry=True)
    seen = {}
    hist = {l: [] for l in range(L)}

    def obs(l, phase, st):
        if phase == "fwd":
            torch.cuda.synchronize()
            seen[l] = O.saturation_count(st.post_q.cpu().numpy())

    for t in range(3):
        b = synth.stack_batch(M, d, 36, t)
        case(f"policy stack step {t}")
        state = stk.step(bf16_dev(b["X"]), bf16_dev(b["dY"]), observe=obs)
        torch.cuda.synchronize()
        st = state.cpu().numpy()
        for l in range(L):
            assert int(stk.saturated[l].item()) == seen[l]
            assert np.isfinite(st[l]).all()
            assert f32_bits(st[l, 1]) == f32_bits(O.delayed_scale(st[l, 0], 2.0))
            if t >= 2:
                assert f32_bits(st[l, 0]) == f32_bits(max(hist[l][-2:]))
            hist[l].append(float(st[l, 2]))
    assert all(0.0 <= stk.saturation_rate(l) <= 1.0 for l in range(L))
