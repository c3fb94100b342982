"""GPU parity of the layer stack x <- x + MLP(rmsnorm(x)) trained with SGD:
the per-layer delayed-scale state carried from step to step, the W2 cache
refreshed after every update, and each layer checked against the oracle
teacher-forced (the oracle is fed that layer's GPU inputs and weights).

Checks per captured layer and step:
  forward  -- RMSNorm rows within one bf16 ulp; the delayed scale bit-exact
              from the layer's own amax_prev; the W2 cache codes bit-exact;
              post, post_q (bit-exact given the GPU's post) and Y against the
              oracle MLP; the residual add bit-exact;
  backward -- dxn rows, dW1 rows, dW2 columns of the MLP backward; the
              RMSNorm backward plus residual gradient rows;
  update   -- SGD bit-exact given the GPU's gradients; the refreshed W2
              cache bit-exact.
And for every layer and step: amax_prev(t) == amax(t-1) bit for bit (the
first step bootstraps with its own exact amax), the scale used equals the
delayed scale of amax_prev, and the amax equals the max of the GPU's post.
"""
import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth
from oracle import formats as F
from oracle import mlp as O
from oracle import stack as S

from .gpu_helpers import DEV, bf16_dev, bits, case, f32_bits, rel_fro, same_codes

pytestmark = pytest.mark.gpu

MARGIN = 2.0


@pytest.fixture(scope="module")
def fm():
    import fp8_relu_mlp_amd as fm
    fm.lib()
    return fm


def _ulp_key(b):
    b = np.asarray(b, dtype=np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _within_ulps(a, b, n=1):
    return int(np.abs(_ulp_key(a) - _ulp_key(b)).max(initial=0)) <= n


class Recorder:
    """observe() hook: copies the buffers of the selected (step, layer) pairs
    to the host (rows = sampled token rows, None = all) and records the
    state of every layer at every step."""

    def __init__(self, capture, rows, cols, lr):
        self.capture, self.rows, self.cols, self.lr = capture, rows, cols, lr
        self.step = 0
        self.caps = {}
        self.post_max = {}

    def _r(self, t):
        a = bits(t)
        return a if self.rows is None else a[self.rows]

    def __call__(self, l, phase, st):
        if phase == "fwd":
            self.post_max[(self.step, l)] = float(st.post[l].max().float().item())
        if (self.step, l) not in self.capture:
            return
        c = self.caps.setdefault((self.step, l), {})
        blk = st.layers[l]
        if phase == "fwd":
            amax_prev, scale, amax_out = st.state[l].cpu().numpy().tolist()
            c.update(x=self._r(st.x[l]), xn=self._r(st.xn[l]), x_out=self._r(st.x[l + 1]),
                     inv=st.inv[l].cpu().numpy() if self.rows is None else st.inv[l].cpu().numpy()[self.rows],
                     post=self._r(st.post[l]), post_q=st.post_q.cpu().numpy()[slice(None) if self.rows is None
                                                                                else self.rows],
                     Y=self._r(st.Y), W1=bits(blk.W1), W2=bits(blk.W2), W2t_q=blk.W2t_q.cpu().numpy(),
                     w2_inv=float(blk.w2_inv_scale.item()), amax_prev=amax_prev, scale=scale, amax_out=amax_out,
                     xn_full=bits(st.xn[l]), post_cols=bits(st.post[l][:, self.cols]))
        elif phase == "bwd":
            c.update(g_in_full=bits(st.g_in), g_in=self._r(st.g_in), dxn=self._r(st.dxn), g_out=self._r(st.g),
                     dW1=st.dW1.cpu().numpy(), dW2=st.dW2.cpu().numpy(), W1_old=bits(blk.W1), W2_old=bits(blk.W2))
        else:
            c.update(W1_new=bits(blk.W1), W2_new=bits(blk.W2), W2t_new=blk.W2t_q.cpu().numpy(),
                     w2_inv_new=float(blk.w2_inv_scale.item()))


def check_layer(c, cols, lr):
    """Teacher-forced oracle checks of one layer at one step."""
    # RMSNorm
    xn_o, r_o = S.rmsnorm(c["x"])
    assert _within_ulps(c["xn"], F.bf16_round(xn_o), 1)
    assert rel_fro(F.bf16_to_f64(c["xn"]), xn_o) < 4e-3
    assert np.allclose(c["inv"], r_o, rtol=2.5e-5, atol=0)   # fp32 sum of d squares: <= d * 2^-24 / 2
    # delayed scale and the W2 cache this forward read
    s = O.delayed_scale(c["amax_prev"], MARGIN)
    assert f32_bits(c["scale"]) == f32_bits(s)
    W2t, _, inv_sw, _ = O.cast_transpose(c["W2"])
    assert (W2t == c["W2t_q"]).all()
    assert f32_bits(c["w2_inv"]) == f32_bits(inv_sw)
    # MLP forward on the GPU's normalised rows
    ref = O.mlp_fwd(c["xn"], c["W1"], W2t, inv_sw, c["amax_prev"], MARGIN)
    post = F.bf16_to_f64(c["post"])
    assert rel_fro(post, F.bf16_to_f64(ref["post"])) < 1e-2
    assert same_codes(c["post_q"], O.quantize(post, s))
    y = F.bf16_to_f64(c["Y"])
    assert rel_fro(y, O.down_fp8(c["post_q"], W2t, O.inv_scale(s), inv_sw)) < 4e-3
    assert rel_fro(y, F.bf16_to_f64(ref["y"])) < 2e-2
    # residual add, bit for bit
    assert (c["x_out"] == S.residual_add(c["x"], c["Y"])).all()
    # MLP backward: rows of dxn, rows of dW1 / columns of dW2 (all tokens)
    b_rows = O.mlp_bwd_sampled(c["g_in"], c["xn"], c["W1"], c["W2"], post, np.arange(len(post)), [], [])
    assert rel_fro(F.bf16_to_f64(c["dxn"]), b_rows["dX_rows"]) < 4e-3
    k = np.arange(len(cols))
    b_cols = O.mlp_bwd_sampled(c["g_in_full"], c["xn_full"], c["W1"][cols], c["W2"][:, cols],
                               F.bf16_to_f64(c["post_cols"]), [], k, k)
    assert rel_fro(c["dW1"][cols].astype(np.float64), b_cols["dW1_rows"]) < 4e-3
    assert rel_fro(c["dW2"][:, cols].astype(np.float64), b_cols["dW2_cols"]) < 1e-4
    # RMSNorm backward + residual gradient on the GPU's dxn
    dx_o = S.rmsnorm_bwd(c["x"], r_o, F.bf16_to_f64(c["dxn"]))
    g_o = F.bf16_to_f64(S.grad_add(c["g_in"], dx_o))
    g_out, g_in = F.bf16_to_f64(c["g_out"]), F.bf16_to_f64(c["g_in"])
    assert rel_fro(g_out, g_o) < 4e-3
    assert rel_fro(g_out - g_in, dx_o) < 2e-2
    # SGD and the W2 cache refresh, bit for bit given the GPU's gradients
    assert (c["W1_new"] == S.sgd(c["W1_old"], c["dW1"], lr)).all()
    assert (c["W2_new"] == S.sgd(c["W2_old"], c["dW2"], lr)).all()
    W2t_n, _, inv_n, _ = O.cast_transpose(c["W2_new"])
    assert (W2t_n == c["W2t_new"]).all()
    assert f32_bits(c["w2_inv_new"]) == f32_bits(inv_n)


def run_stack(fm, L, M, d, h, steps, seed, capture, rows, cols, lr=1e-3, loss="mean"):
    from fp8_relu_mlp_amd.stack import Relu2Stack
    ws = synth.stack_weights(L, d, h, seed)
    stk = Relu2Stack([bf16_dev(w1) for w1, _ in ws], [bf16_dev(w2) for _, w2 in ws], margin=MARGIN, lr=lr,
                     loss=loss)
    rec = Recorder(capture, rows, cols, lr)
    states = []
    for t in range(steps):
        b = synth.stack_batch(M, d, seed, t)
        rec.step = t
        case(f"stack L={L} M={M} d={d} h={h} step {t}")
        st = stk.step(bf16_dev(b["X"]), bf16_dev(b["dY"]), observe=rec)
        torch.cuda.synchronize()
        states.append(st.cpu().numpy().copy())
    return stk, rec, np.array(states)


def _same_f32(a, b):
    return f32_bits(a) == f32_bits(b) or (np.isnan(a) and np.isnan(b))


def check_state_carry(states, rec, L, steps):
    for t in range(steps):
        for l in range(L):
            amax_prev, scale, amax_out = states[t, l]
            assert _same_f32(amax_out, rec.post_max[(t, l)]), (t, l)
            assert _same_f32(scale, O.delayed_scale(amax_prev, MARGIN)), (t, l)
            expect_prev = amax_out if t == 0 else states[t - 1, l, 2]
            assert _same_f32(amax_prev, expect_prev), (t, l)


def test_stack_helpers_against_oracle(fm):
    M, d = 1001, 768
    g = np.random.default_rng(11)
    xb = synth.to_bf16_bits(g.standard_normal((M, d)) * 3.0)
    case(f"rmsnorm / add / sgd helpers M={M} d={d}")
    x = bf16_dev(xb)
    xn = torch.empty_like(x)
    inv = torch.empty(M, dtype=torch.float32, device=DEV)
    fm.rmsnorm_fwd(x, xn, inv)
    dxb = synth.to_bf16_bits(g.standard_normal((M, d)) * 0.01)
    gb = synth.to_bf16_bits(g.standard_normal((M, d)) * 0.03)
    go = torch.empty_like(x)
    fm.rmsnorm_bwd(x, inv, bf16_dev(dxb), bf16_dev(gb), go)
    yb = synth.to_bf16_bits(g.standard_normal((M, d)))
    s = torch.empty_like(x)
    fm.add_bf16(x, bf16_dev(yb), s)
    Wb = synth.to_bf16_bits(g.standard_normal((384, 768)) * 0.05)
    dW = (g.standard_normal((384, 768)) * 0.3).astype(np.float32)
    W = bf16_dev(Wb)
    fm.sgd_update_bf16(W, torch.from_numpy(dW).to(DEV), 1e-3)
    fm.rmsnorm_fwd(x[:0], xn[:0], inv[:0])          # M = 0 launches nothing
    torch.cuda.synchronize()
    xn_o, r_o = S.rmsnorm(xb)
    assert _within_ulps(bits(xn), F.bf16_round(xn_o), 1)
    assert np.allclose(inv.cpu().numpy(), r_o, rtol=2.5e-5, atol=0)
    dx_o = S.rmsnorm_bwd(xb, r_o, F.bf16_to_f64(dxb))
    assert rel_fro(F.bf16_to_f64(bits(go)), F.bf16_to_f64(S.grad_add(gb, dx_o))) < 4e-3
    assert rel_fro(F.bf16_to_f64(bits(go)) - F.bf16_to_f64(gb), dx_o) < 2e-2
    assert (bits(s) == S.residual_add(xb, yb)).all()
    assert (bits(W) == S.sgd(Wb, dW, 1e-3)).all()


def test_stack_small_every_layer_and_step(fm):
    """3 layers, ragged M, 3 steps: every layer at every step against the oracle."""
    L, M, d, h, steps = 3, 300, 128, 256, 3
    cols = [0, 77, h - 1]
    cap = {(t, l) for t in range(steps) for l in range(L)}
    # the summed-gradient step (lr * dW): at this size it moves the weights
    # by many bf16 ulps per step and stays finite over the three steps
    stk, rec, states = run_stack(fm, L, M, d, h, steps, 7, cap, None, cols, loss="sum")
    assert stk.lr_step == np.float32(1e-3)
    check_state_carry(states, rec, L, steps)
    for (t, l), c in sorted(rec.caps.items()):
        case(f"stack small: oracle check layer {l} step {t}")
        check_layer(c, cols, stk.lr_step)


def test_stack_full_size(fm):
    """The layer-stack workload: 12 layers, M=65536, d=768, h=3072, 8 SGD
    steps.  State carry checked at every layer and step; layers 0 and 11 at
    steps 0, 1 and 7 checked against the oracle on sampled rows."""
    M, d, h, seed = synth.WORKLOADS["stack"]
    L, steps, lr = synth.STACK["layers"], synth.STACK["steps"], synth.STACK["lr"]
    rows = np.sort(np.random.default_rng(5).choice(M, size=40, replace=False))
    rows = np.concatenate([[0], rows, [M - 1]])
    cols = [0, 1234, h - 1]
    cap = {(t, l) for t in (0, 1, steps - 1) for l in (0, L - 1)}
    stk, rec, states = run_stack(fm, L, M, d, h, steps, seed, cap, rows, cols, lr)
    assert stk.lr_step == np.float32(lr / M)                # token-mean loss
    assert np.isfinite(states).all()
    check_state_carry(states, rec, L, steps)
    for (t, l), c in sorted(rec.caps.items()):
        case(f"stack full size: oracle check layer {l} step {t}")
        check_layer(c, cols, stk.lr_step)


@pytest.mark.parametrize("opts", [{}, {"fp8_up": True, "amax_window": 3, "w2_scale": "delayed", "w2_margin": 1.5}])
def test_stack_checkpoint_resume_bit_identical(fm, opts):
    """Stop a 3-layer stack after step k, save its state (torch.save to a
    byte buffer, loaded back with weights_only), load it into a freshly built
    stack and continue: every weight, cache, amax and output of the following
    steps equals the uninterrupted run bit for bit."""
    import io
    from fp8_relu_mlp_amd.stack import Relu2Stack
    L, M, d, h, steps, stop = 3, 1536, 256, 768, 5, 2
    case(f"stack checkpoint/resume L={L} M={M} d={d} h={h} opts={opts}")
    ws = [synth.mlp_inputs(8, d, h, 100 + l) for l in range(L)]
    batches = [synth.mlp_inputs(M, d, h, 200 + t, with_dy=True) for t in range(steps)]

    def fresh():
        return Relu2Stack([bf16_dev(w["W1"]) for w in ws], [bf16_dev(w["W2"]) for w in ws], margin=MARGIN,
                          lr=1e-3, **opts)

    def snapshot(st):
        torch.cuda.synchronize()
        return {k: v.reshape(-1).contiguous().view(torch.uint8).numpy().copy() for k, v in st.state_dict().items()}

    def run(st, t0, t1):
        outs = []
        for t in range(t0, t1):
            state = st.step(bf16_dev(batches[t]["X"]), bf16_dev(batches[t]["dY"]))
            torch.cuda.synchronize()
            outs.append((state.cpu().numpy().copy(), bits(st.x[L]), snapshot(st)))
        return outs

    full = run(fresh(), 0, steps)
    a = fresh()
    run(a, 0, stop)
    buf = io.BytesIO()
    torch.save(a.state_dict(), buf)
    del a
    buf.seek(0)
    b = fresh()
    b.load_state_dict(torch.load(buf, weights_only=True))
    resumed = run(b, stop, steps)
    for (s_full, x_full, sd_full), (s_res, x_res, sd_res) in zip(full[stop:], resumed):
        assert (f32_bits(s_full) == f32_bits(s_res)).all()
        assert (x_full == x_res).all()
        assert sd_full.keys() == sd_res.keys()
        for k in sd_full:
            assert sd_full[k].tobytes() == sd_res[k].tobytes(), k
