"""GPU parity at the full benchmark sizes, in the launch configuration the
benchmark times (Relu2MLP: fwd TRAIN + bwd + W2 cache refresh).

At the timed workload (M=49152, d=768, h=3072) every element of post, post_q,
Y, dX, dW1, dW2 and of the two intermediate workspaces (the forward's
partial-amax tensor, the backward's dpre) is compared with the oracle, in
row chunks of 4096: against the oracle run on its own from X, W1, W2 and dY
(the gates 1e-2 / 2e-2), and, tighter, against the oracle fed the GPU's own
intermediates.  The other tests check sampled outputs the oracle computes
one by one, plus properties over whole tensors.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth
from oracle import formats as F
from oracle import mlp as O

from .gpu_helpers import DEV, bf16_dev, bits, case, f32_bits, rel_fro

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    import fp8_relu_mlp_amd as fm
    fm.lib()
    return fm


def _max_bf16_nonneg(b):
    """max of non-negative bf16 values given as bits (unsigned order = value order)."""
    return float(F.bf16_to_f64(np.uint16(b.max()))) if b.size else 0.0


def test_fwdbwd_full_size_sampled(fm):
    M, d, h = synth.WORKLOADS["fwdbwd"][:3]
    seed = synth.WORKLOADS["fwdbwd"][3]
    ins = synth.mlp_inputs(M, d, h, seed, with_dy=True)
    case(f"full-size fwd+bwd M={M} d={d} h={h}")
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    blk.forward(X)                                   # bootstrap amax_prev
    amax_prev = float(blk.amax_prev.item())
    Y, post, post_q = blk.forward(X)
    dX, dW1, dW2 = blk.backward(dY, X, post)
    torch.cuda.synchronize()
    post_b = bits(post)
    # amax: bit-exact over the whole tensor
    assert f32_bits(blk.amax_last.item()) == f32_bits(_max_bf16_nonneg(post_b))
    s = O.delayed_scale(amax_prev, 2.0)
    assert f32_bits(blk.scale_used.item()) == f32_bits(s)
    rows = np.random.default_rng(1).choice(M, size=48, replace=False)
    rows.sort()
    rows = np.concatenate([rows, [0, M - 1]])
    pq = post_q.cpu().numpy()[rows]
    pb = post_b[rows]
    # codes bit-exact given the GPU's post (sampled rows)
    assert (O.quantize(F.bf16_to_f64(pb), s) == pq).all()
    W2t, _, inv_sw, _ = O.cast_transpose(ins["W2"])
    assert (W2t == blk.W2t_q.cpu().numpy()).all()
    ref = O.mlp_fwd(ins["X"][rows], ins["W1"], W2t, inv_sw, amax_prev, 2.0)
    assert rel_fro(F.bf16_to_f64(pb), F.bf16_to_f64(ref["post"])) < 1e-2
    y = F.bf16_to_f64(bits(Y)[rows])
    assert rel_fro(y, F.bf16_to_f64(ref["y"])) < 2e-2
    assert rel_fro(y, O.down_fp8(pq, W2t, O.inv_scale(s), inv_sw)) < 4e-3
    # backward on sampled rows / columns, fed the GPU's post
    post_f = F.bf16_to_f64(post_b)
    r1 = [0, 1234, h - 1]
    c2 = [0, 777, h - 1]
    bs = O.mlp_bwd_sampled(ins["dY"], ins["X"], ins["W1"], ins["W2"], post_f, rows, r1, c2)
    assert rel_fro(F.bf16_to_f64(bits(dX)[rows]), bs["dX_rows"]) < 4e-3
    assert rel_fro(dW1.cpu().numpy()[r1].astype(np.float64), bs["dW1_rows"]) < 4e-3
    assert rel_fro(dW2.cpu().numpy()[:, c2].astype(np.float64), bs["dW2_cols"]) < 1e-4


class _Fro:
    """Relative Frobenius error of a tensor compared chunk by chunk."""

    def __init__(self):
        self.num = 0.0
        self.den = 0.0

    def add(self, got, ref):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        self.num += float(np.sum((got - ref) ** 2))
        self.den += float(np.sum(ref ** 2))

    def value(self):
        return (self.num / max(self.den, 1e-300)) ** 0.5


def test_fwdbwd_full_size_whole_tensors(fm):
    """The timed workload (M=49152, d=768, h=3072, margin 2, the first step's
    own amax as amax_prev), every output element against the oracle.

    Independent chain: the oracle alone from X, W1, W2, dY -- its own post,
    its own amax as the bootstrap amax_prev, its own e4m3 codes, Y, dpre, dX,
    dW1, dW2 -- against the GPU: post, dX, dW1, dW2 within 1e-2, Y within
    2e-2 (relative Frobenius over the whole tensor).
    Given the GPU's intermediates: every post_q code bit-exact from the GPU's
    post and scale; the partial-amax workspace bit-exact against the oracle's
    tile maxima of the GPU's post (256 x 256 tiles); Y within 4e-3 of the
    oracle's FP8 GEMM of the GPU's codes; dpre (the backward workspace), dX
    and dW1 within 4e-3 and dW2 within 1e-4 of the oracle's backward fed the
    GPU's post."""
    M, d, h = synth.WORKLOADS["fwdbwd"][:3]
    seed = synth.WORKLOADS["fwdbwd"][3]
    ins = synth.mlp_inputs(M, d, h, seed, with_dy=True)
    case(f"full-size fwd+bwd whole tensors M={M} d={d} h={h}")
    L = fm.lib()
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    ws_f = torch.zeros(L.mlp_relu2_fwd_workspace(M, d, h), dtype=torch.uint8, device=DEV)
    ws_b = torch.zeros(L.mlp_relu2_bwd_workspace(M, d, h), dtype=torch.uint8, device=DEV)
    blk.forward(X, workspace=ws_f)                   # bootstrap amax_prev
    amax_prev = float(blk.amax_prev.item())
    Y, post, post_q = blk.forward(X, workspace=ws_f)
    dX, dW1, dW2 = blk.backward(dY, X, post, workspace=ws_b)
    torch.cuda.synchronize()
    BM = BN = 256
    tm, tn = -(-M // BM), -(-h // BN)
    part_g = ws_f[:tm * tn * 4].view(torch.float32).cpu().numpy().reshape(tm, tn)
    dpre_g = bits(ws_b[:M * h * 2].view(torch.bfloat16).view(M, h))
    post_g, pq_g, y_g, dx_g = bits(post), post_q.cpu().numpy(), bits(Y), bits(dX)
    dw1_g = dW1.cpu().numpy().astype(np.float64)
    dw2_g = dW2.cpu().numpy().astype(np.float64)
    s_g = O.delayed_scale(amax_prev, 2.0)
    assert f32_bits(blk.scale_used.item()) == f32_bits(s_g)
    assert f32_bits(blk.amax_last.item()) == f32_bits(_max_bf16_nonneg(post_g))
    W2t, _, inv_sw, _ = O.cast_transpose(ins["W2"])
    assert (W2t == blk.W2t_q.cpu().numpy()).all()

    CH = 4096
    chunks = [(r0, min(M, r0 + CH)) for r0 in range(0, M, CH)]
    workers = max(1, min(4, (os.cpu_count() or 4) // 4))

    # pass 1: the oracle's own post, and its amax (the bootstrap amax_prev)
    def pass1(c):
        r0, r1 = c
        return F.bf16_round(O.up_relu2(ins["X"][r0:r1], ins["W1"]))

    with ThreadPoolExecutor(workers) as ex:
        post_o = np.concatenate(list(ex.map(pass1, chunks)))
    amax_o = O.amax(F.bf16_to_f64(post_o))

    # pass 2: the rest of both chains, chunk by chunk
    def pass2(c):
        r0, r1 = c
        Xc, dYc = ins["X"][r0:r1], ins["dY"][r0:r1]
        pg = F.bf16_to_f64(post_g[r0:r1])
        out = {}
        # independent chain
        fo = O.mlp_fwd(Xc, ins["W1"], W2t, inv_sw, amax_o, 2.0, post_bits=post_o[r0:r1])
        bo = O.mlp_bwd(dYc, Xc, ins["W1"], ins["W2"], F.bf16_to_f64(post_o[r0:r1]))
        out["post"] = (F.bf16_to_f64(post_g[r0:r1]), F.bf16_to_f64(post_o[r0:r1]))
        out["y"] = (F.bf16_to_f64(y_g[r0:r1]), F.bf16_to_f64(fo["y"]))
        out["dx"] = (F.bf16_to_f64(dx_g[r0:r1]), bo["dX"])
        out["dpre_o"] = (F.bf16_to_f64(dpre_g[r0:r1]), bo["dpre"])
        out["dw1_o"], out["dw2_o"] = bo["dW1"], bo["dW2"]
        # given the GPU's intermediates
        out["codes_ok"] = bool((O.quantize(pg, s_g) == pq_g[r0:r1]).all())
        out["y_g"] = (out["y"][0], O.down_fp8(pq_g[r0:r1], W2t, O.inv_scale(s_g), inv_sw))
        bg = O.mlp_bwd(dYc, Xc, ins["W1"], ins["W2"], pg)
        out["dpre_g"] = (out["dpre_o"][0], bg["dpre"])
        out["dx_g"] = (out["dx"][0], bg["dX"])
        out["dw1_g"], out["dw2_g"] = bg["dW1"], bg["dW2"]
        # partial amax of the tile rows in this chunk (chunks hold whole tile rows)
        out["tiles"] = (r0 // BM, O.tile_amax(pg, BM, BN))
        return out

    fro = {k: _Fro() for k in ("post", "y", "dx", "dpre_o", "y_g", "dpre_g", "dx_g")}
    dw1_o, dw2_o = np.zeros((h, d)), np.zeros((d, h))
    dw1_gf, dw2_gf = np.zeros((h, d)), np.zeros((d, h))
    tiles_ok = True
    with ThreadPoolExecutor(workers) as ex:
        for out in ex.map(pass2, chunks):
            assert out["codes_ok"], "post_q codes"
            for k in fro:
                fro[k].add(*out[k])
            dw1_o += out["dw1_o"]
            dw2_o += out["dw2_o"]
            dw1_gf += out["dw1_g"]
            dw2_gf += out["dw2_g"]
            t0, ta = out["tiles"]
            tiles_ok &= bool((f32_bits(ta) == f32_bits(part_g[t0:t0 + ta.shape[0]])).all())
    assert tiles_ok, "partial-amax workspace"
    # the oracle on its own
    assert fro["post"].value() < 1e-2, fro["post"].value()
    assert fro["y"].value() < 2e-2, fro["y"].value()
    assert fro["dx"].value() < 1e-2, fro["dx"].value()
    assert fro["dpre_o"].value() < 1e-2, fro["dpre_o"].value()
    assert rel_fro(dw1_g, dw1_o) < 1e-2
    assert rel_fro(dw2_g, dw2_o) < 1e-2
    # fed the GPU's intermediates
    assert fro["y_g"].value() < 4e-3, fro["y_g"].value()
    assert fro["dpre_g"].value() < 4e-3, fro["dpre_g"].value()
    assert fro["dx_g"].value() < 4e-3, fro["dx_g"].value()
    assert rel_fro(dw1_g, dw1_gf) < 4e-3
    assert rel_fro(dw2_g, dw2_gf) < 1e-4


def test_fwd_two_steps_full_size(fm):
    """Two-step forward at M=16384 with the W1 perturbation between steps."""
    M, d, h = synth.WORKLOADS["fwd2"][:3]
    seed = synth.WORKLOADS["fwd2"][3]
    ins = synth.mlp_inputs(M, d, h, seed)
    case(f"two-step forward M={M}")
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0)
    X = bf16_dev(ins["X"])
    blk.forward(X)
    a0 = float(blk.amax_prev.item())
    blk.forward(X)                                   # step 1 with its own exact amax
    a1 = float(blk.amax_prev.item())
    assert a1 == a0
    W1b = synth.perturbed_w1(ins["W1"], seed)
    X2 = synth.mlp_inputs(M, d, h, seed, step=1)["X"]
    blk.W1 = bf16_dev(W1b)
    Y, post, post_q = blk.forward(bf16_dev(X2))      # step 2 uses step 1's amax
    torch.cuda.synchronize()
    assert f32_bits(blk.scale_used.item()) == f32_bits(O.delayed_scale(a1, 2.0))
    post_b = bits(post)
    assert f32_bits(blk.amax_last.item()) == f32_bits(_max_bf16_nonneg(post_b))
    s = O.delayed_scale(a1, 2.0)
    # every code of step 2, bit-exact given the GPU's post
    pq = post_q.cpu().numpy()
    for r0 in range(0, M, 4096):
        assert (O.quantize(F.bf16_to_f64(post_b[r0:r0 + 4096]), s) == pq[r0:r0 + 4096]).all()
    rows = np.arange(0, M, 257)
    W2t, _, inv_sw, _ = O.cast_transpose(ins["W2"])
    ref = O.mlp_fwd(X2[rows], W1b, W2t, inv_sw, a1, 2.0)
    assert rel_fro(F.bf16_to_f64(bits(Y)[rows]), F.bf16_to_f64(ref["y"])) < 2e-2


@pytest.mark.parametrize("which", ["qkv", "o"])
def test_fp8_linear_full_size(fm, which):
    a = synth.attn_inputs()
    Xb = a["X"] if which == "qkv" else a["Xo"]
    Wb = a["Wqkv"] if which == "qkv" else a["Wo"]
    M, K = Xb.shape
    N = Wb.shape[0]
    case(f"fp8_linear full size {which} M={M} K={K} N={N}")
    X, W = bf16_dev(Xb), bf16_dev(Wb)
    Wt = torch.empty((K, N), dtype=torch.uint8, device=DEV)
    inv_w = torch.zeros(1, dtype=torch.float32, device=DEV)
    fm.fp8_cast_transpose(W, Wt, inv_scale_out=inv_w)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    fm.amax_reduce(X, amax)
    sx = torch.zeros(1, dtype=torch.float32, device=DEV)
    fm.fp8_scale_from_amax(amax, 1.0, sx)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    fm.fp8_linear(X, sx, Wt, inv_w, Y)
    torch.cuda.synchronize()
    assert f32_bits(amax.item()) == f32_bits(O.amax(F.bf16_to_f64(Xb)))
    rows = np.arange(0, M, 997)
    Wt_o, _, inv_o, _ = O.cast_transpose(Wb)
    assert (Wt_o == Wt.cpu().numpy()).all()
    ref = F.bf16_to_f64(O.fp8_linear(Xb[rows], float(sx.item()), Wt_o, inv_o))
    assert rel_fro(F.bf16_to_f64(bits(Y)[rows]), ref) < 4e-3


def test_bwd_ragged_mid_size(fm):
    """M = 22983 (not a multiple of any tile height) at d=768, h=3072: rows
    around tile boundaries and the ragged last row of dX, rows of dW1 and
    columns of dW2 against the oracle; two backward calls give the same bits."""
    M, d, h = 22983, 768, 3072
    ins = synth.mlp_inputs(M, d, h, 9, with_dy=True)
    case(f"ragged mid-size backward M={M} d={d} h={h}")
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    blk.forward(X)
    Y, post, post_q = blk.forward(X)
    dX, dW1, dW2 = blk.backward(dY, X, post)
    dX2, _, _ = blk.backward(dY, X, post)
    torch.cuda.synchronize()
    assert (bits(dX) == bits(dX2)).all()                       # deterministic
    rows = np.array([0, 1, 191, 192, 255, 256, 21760, 22783, 22784, M - 200, M - 1])
    post_f = F.bf16_to_f64(bits(post))
    bs = O.mlp_bwd_sampled(ins["dY"], ins["X"], ins["W1"], ins["W2"], post_f, rows, [0, 2000], [5, h - 1])
    dx = F.bf16_to_f64(bits(dX)[rows])
    assert rel_fro(dx, bs["dX_rows"]) < 4e-3
    for i in range(len(rows)):
        assert rel_fro(dx[i], bs["dX_rows"][i]) < 1e-2, rows[i]
    assert rel_fro(dW1.cpu().numpy()[[0, 2000]].astype(np.float64), bs["dW1_rows"]) < 4e-3
    assert rel_fro(dW2.cpu().numpy()[:, [5, h - 1]].astype(np.float64), bs["dW2_cols"]) < 1e-4


@pytest.mark.timeout(300)
def test_bwd_token_ranges_past_32bit_offsets(fm):
    """The backward of a wider block, d=2048, h=8192, at M = 300000 tokens.
    dW has 256 tiles here, enough blocks without splitting the tokens, but
    rows of dpre and post hold 16384 bytes: the dW GEMMs address one token
    range per block with 32-bit offsets, so the tokens go in ranges of at
    most 131072 (2^31 bytes of a row-contiguous operand): three ranges, the
    last ragged (37856 tokens), where one range of all tokens would span
    4.9 GB.  Rows of dW1 and columns of dW2 (sums over every token) and rows
    of dX against the oracle.  post is a synthetic non-negative input
    (|N(0,1)|).  The sampled dW entries come from the oracle's sampled
    backward restricted to the hidden units they involve (hidden unit i's
    dpre column depends only on post column i and W2 column i)."""
    M, d, h = 300000, 2048, 8192
    seed = 11
    case(f"backward over several token ranges: drawing inputs M={M} d={d} h={h}")
    X = synth.normal_bf16_rows((M, d), 1.0, seed, "X")
    dY = synth.normal_bf16_rows((M, d), 1e-3, seed, "dY")
    post = synth.abs_normal_bf16_rows((M, h), seed, "post")
    W1 = synth.normal_bf16((h, d), 1.0 / d, seed, "W1")
    W2 = synth.normal_bf16((d, h), 1.0 / h, seed, "W2")
    case(f"backward over several token ranges M={M} d={d} h={h}")
    Xd, dYd, postd = bf16_dev(X), bf16_dev(dY), bf16_dev(post)
    dX = torch.empty_like(Xd)
    dW1 = torch.empty((h, d), dtype=torch.float32, device=DEV)
    dW2 = torch.empty((d, h), dtype=torch.float32, device=DEV)
    fm.mlp_relu2_bwd(dYd, Xd, bf16_dev(W1), bf16_dev(W2), postd, dX, dW1, dW2)
    torch.cuda.synchronize()
    del postd
    bounds = [131072, 262144]
    rows = np.array(sorted({0, M - 1, *bounds, *(b - 1 for b in bounds), 12345, 200001}))
    r1, c2 = [0, 5000, h - 1], [0, 777, h - 1]
    dx = F.bf16_to_f64(bits(dX)[rows])
    dw1 = dW1.cpu().numpy()[r1].astype(np.float64)
    dw2 = dW2.cpu().numpy()[:, c2].astype(np.float64)
    case("backward over several token ranges: oracle on sampled outputs")
    ref_rows = O.mlp_bwd_sampled(dY[rows], X[rows], W1, W2, F.bf16_to_f64(post[rows]), np.arange(len(rows)), [], [])
    units = r1 + c2
    ref_w = O.mlp_bwd_sampled(dY, X, W1[units], W2[:, units], F.bf16_to_f64(post[:, units]), [], [0, 1, 2],
                              [3, 4, 5])
    assert rel_fro(dx, ref_rows["dX_rows"]) < 4e-3
    assert rel_fro(dw1, ref_w["dW1_rows"]) < 4e-3
    assert rel_fro(dw2, ref_w["dW2_cols"]) < 1e-4
    for k in range(3):
        # every sampled gradient row / column on its own, not only in aggregate
        assert rel_fro(dw1[k], ref_w["dW1_rows"][k]) < 1e-2, r1[k]
        assert rel_fro(dw2[:, k], ref_w["dW2_cols"][:, k]) < 1e-4, c2[k]


def test_fp8up_full_size_sampled(fm):
    """The e4m3 up-projection forward at the timed workload's size
    (M=49152, d=768, h=3072) through Relu2MLP(fp8_up=True): amaxes
    bit-exact over whole tensors, both weight caches bit-exact, sampled rows
    of post within the per-element bound, their codes bit-exact, Y close to
    the oracle's FP8 GEMM of the GPU's codes."""
    from .test_gpu_fp8up import post_bound
    M, d, h = synth.WORKLOADS["fwdbwd"][:3]
    seed = synth.WORKLOADS["fwdbwd"][3]
    ins = synth.mlp_inputs(M, d, h, seed)
    case(f"full-size fp8-up forward M={M} d={d} h={h}")
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0, fp8_up=True)
    X = bf16_dev(ins["X"])
    blk.forward(X)                                   # bootstrap both amaxes
    xa, a = float(blk.x_amax_prev.item()), float(blk.amax_prev.item())
    Y, post, post_q = blk.forward(X)
    torch.cuda.synchronize()
    Xf_max = max(float(np.abs(F.bf16_to_f64(ins["X"][r0:r0 + 8192])).max()) for r0 in range(0, M, 8192))
    assert f32_bits(xa) == f32_bits(Xf_max) and f32_bits(blk.x_amax_prev.item()) == f32_bits(Xf_max)
    post_b = bits(post)
    assert f32_bits(blk.amax_last.item()) == f32_bits(_max_bf16_nonneg(post_b))
    sx, s = O.delayed_scale(xa, 2.0), O.delayed_scale(a, 2.0)
    assert f32_bits(blk.x_scale.item()) == f32_bits(sx) and f32_bits(blk.scale_used.item()) == f32_bits(s)
    W1t, _, inv1, _ = O.cast_transpose(ins["W1"])
    W2t, _, inv2, _ = O.cast_transpose(ins["W2"])
    assert (W1t == blk.W1t_q.cpu().numpy()).all() and (W2t == blk.W2t_q.cpu().numpy()).all()
    rows = np.concatenate([np.arange(0, M, 1009), [255, 256, M - 1]])
    pb = F.bf16_to_f64(post_b[rows])
    ref_post, _, _ = O.up_relu2_fp8(ins["X"][rows], sx, W1t, inv1)
    assert (np.abs(pb - ref_post) <= post_bound(ins["X"][rows], sx, W1t, inv1)).all()
    pq = post_q.cpu().numpy()[rows]
    assert (O.quantize(pb, s) == pq).all()
    y = F.bf16_to_f64(bits(Y)[rows])
    assert rel_fro(y, O.down_fp8(pq, W2t, O.inv_scale(s), inv2)) < 4e-3


def test_fp8post_full_size_sampled(fm):
    """The e4m3-post variant at the timed workload's size: forward without
    the bf16 post, backward from post_q; sampled rows of dX, rows of dW1 and
    columns of dW2 against the oracle's backward on post_hat."""
    M, d, h = synth.WORKLOADS["fwdbwd"][:3]
    seed = synth.WORKLOADS["fwdbwd"][3]
    ins = synth.mlp_inputs(M, d, h, seed, with_dy=True)
    case(f"full-size fp8-post fwd+bwd M={M} d={d} h={h}")
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0, keep_post=False)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    blk.forward(X)
    Y, post, post_q = blk.forward(X)
    dX, dW1, dW2 = blk.backward(dY, X, None, post_q=post_q)
    torch.cuda.synchronize()
    assert post is None
    rows = np.concatenate([np.arange(0, M, 1021), [255, 256, M - 1]])
    ph = O.post_from_q(post_q.cpu().numpy(), blk.scale_used.item())
    r1, c2 = [0, 1234, h - 1], [0, 777, h - 1]
    bs = O.mlp_bwd_sampled(ins["dY"], ins["X"], ins["W1"], ins["W2"], ph, rows, r1, c2)
    assert rel_fro(F.bf16_to_f64(bits(dX)[rows]), bs["dX_rows"]) < 4e-3
    assert rel_fro(dW1.cpu().numpy()[r1].astype(np.float64), bs["dW1_rows"]) < 4e-3
    assert rel_fro(dW2.cpu().numpy()[:, c2].astype(np.float64), bs["dW2_cols"]) < 1e-4


def test_ce_full_size_sampled(fm):
    """The fused softcapped cross-entropy at the head workload's size
    (M=49152, d=768, V=50304, three targets, softcap 15): sampled rows of
    lse, G and dX against the oracle, sampled columns of dW against the
    oracle fed the GPU's G, and the loss against the oracle's reduction of
    the GPU's lse with exact target logits."""
    from oracle import ce as C
    from .test_gpu_ce import U
    cfg = synth.CE
    M, d, V, T, c = cfg["M"], cfg["d"], cfg["V"], cfg["T"], cfg["softcap"]
    wts = list(cfg["weights"])
    ins = synth.ce_inputs(M, d, V, T, cfg["seed"], seq=cfg["seq"])
    case(f"full-size softcapped CE M={M} d={d} V={V} T={T}")
    X, W = bf16_dev(ins["X"]), bf16_dev(ins["W"])
    t_dev = torch.from_numpy(ins["targets"].astype(np.int32)).to(DEV)
    w_dev = torch.tensor(wts, dtype=torch.float32, device=DEV)
    loss = torch.zeros(1, device=DEV)
    lse = torch.zeros(M, device=DEV)
    dX = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((V, d), dtype=torch.float32, device=DEV)
    ws = fm.softcap_ce_fwd_bwd(X, W, t_dev, w_dev, c, loss, dX, dW, lse_out=lse)
    torch.cuda.synchronize()
    Gd = ws[:M * V * 2].view(torch.bfloat16).view(M, V)
    rows = np.array([0, 1, 1023, 1024, 20000, 33333, M - 1025, M - 1])
    Xf, Wf = F.bf16_to_f64(ins["X"]), F.bf16_to_f64(ins["W"])
    ref = C.softcap_ce(ins["X"][rows], ins["W"], ins["targets"][rows], wts, c, dloss=len(rows) / M)
    # lse of the sampled rows, within the bound of the parity tests
    S = np.abs(Xf[rows]) @ np.abs(Wf).T
    ez = (d + 2) * U * S.max(axis=1) * 1.01 + 16 * U * c + 4 * U * np.abs(Xf[rows] @ Wf.T).max(axis=1)
    e_lse = ez + (48 + 197) * U + 2.0 ** -22 + 2.0 ** -23 * np.abs(ref["lse"])
    lse_g = lse.cpu().numpy().astype(np.float64)
    assert (np.abs(lse_g[rows] - ref["lse"]) <= e_lse).all()
    # loss = (1/M) sum_m sum_j w_j (lse_m - z'_t): the GPU's lse, exact target logits
    t = ins["targets"]
    valid = t >= 0
    zt = np.zeros(t.shape)
    for j in range(T):
        m = np.nonzero(valid[:, j])[0]
        zt[m, j] = C.softcap(np.einsum("md,md->m", Xf[m], Wf[t[m, j]]), c)
    w = np.asarray(wts)
    expect = (np.where(valid, w[None, :] * (lse_g[:, None] - zt), 0.0)).sum() / M
    ez_all = (d + 2) * U * np.abs(Xf).sum(axis=1) * np.abs(Wf).max() + 16 * U * c
    bound = (np.where(valid, w[None, :], 0.0).sum(axis=1) * ez_all).sum() / M + (512 + M / 256) * U * abs(expect)
    assert abs(loss.item() - expect) <= bound
    # G rows and dX rows
    Gr = F.bf16_to_f64(bits(Gd[torch.from_numpy(rows).to(DEV)]))
    assert rel_fro(Gr, ref["G"]) < 1e-2
    assert rel_fro(F.bf16_to_f64(bits(dX)[rows]), Gr @ Wf) < 4e-3
    # dW columns from the GPU's own G
    cols = np.array([0, 7, 25000, 50256, V - 1])
    Gc = F.bf16_to_f64(bits(Gd[:, torch.from_numpy(cols).to(DEV)].contiguous()))
    assert rel_fro(dW.cpu().numpy()[cols].astype(np.float64), Gc.T @ Xf) < 1e-4


def test_ce_fp8_full_size_sampled(fm):
    """The FP8-head cross-entropy at the head workload's size: the e4m3 W
    cache bit-exact, sampled rows of lse and G against the oracle on the
    e4m3 logits (lse within the alignment-window bound), dX rows and dW
    columns against the oracle fed the GPU's G."""
    from oracle import ce as C
    from .test_gpu_ce import U
    from .test_gpu_fp8up import acc_bound
    cfg = synth.CE
    M, d, V, T, c = cfg["M"], cfg["d"], cfg["V"], cfg["T"], cfg["softcap"]
    wts = list(cfg["weights"])
    ins = synth.ce_inputs(M, d, V, T, cfg["seed"], seq=cfg["seq"])
    case(f"full-size FP8-head softcapped CE M={M} d={d} V={V} T={T}")
    X, W = bf16_dev(ins["X"]), bf16_dev(ins["W"])
    Wt = torch.empty((d, V), dtype=torch.uint8, device=DEV)
    inv = torch.zeros(1, dtype=torch.float32, device=DEV)
    fm.fp8_cast_transpose(W, Wt, inv_scale_out=inv)
    am = torch.zeros(1, dtype=torch.float32, device=DEV)
    fm.amax_reduce(X, am)
    sx = torch.zeros(1, dtype=torch.float32, device=DEV)
    fm.fp8_scale_from_amax(am, 1.0, sx)
    t_dev = torch.from_numpy(ins["targets"].astype(np.int32)).to(DEV)
    w_dev = torch.tensor(wts, dtype=torch.float32, device=DEV)
    loss, lse = torch.zeros(1, device=DEV), torch.zeros(M, device=DEV)
    dX = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((V, d), dtype=torch.float32, device=DEV)
    ws = fm.softcap_ce_fwd_bwd_fp8(X, sx, Wt, inv, W, t_dev, w_dev, c, loss, dX, dW, lse_out=lse)
    torch.cuda.synchronize()
    Wt_o, _, inv_o, _ = O.cast_transpose(ins["W"])
    assert (Wt.cpu().numpy() == Wt_o).all() and inv.item() == inv_o
    sxv = float(sx.item())
    assert f32_bits(sxv) == f32_bits(O.exact_scale(O.amax(F.bf16_to_f64(ins["X"]))))
    rows = np.array([0, 1023, 1024, 30000, M - 1])
    Z = C.fp8_logits(ins["X"][rows], sxv, Wt_o, inv_o)
    ref = C.softcap_ce(ins["X"][rows], ins["W"], ins["targets"][rows], wts, c, dloss=len(rows) / M, Z=Z)
    Xf, Wf = F.bf16_to_f64(ins["X"]), F.bf16_to_f64(ins["W"])
    xq = F.e4m3_decode(F.e4m3_encode(F.fl32(Xf[rows] * sxv)))
    ez = ((acc_bound(xq, F.e4m3_decode(Wt_o)) * O.inv_scale(sxv) * inv_o).max(axis=1) * 1.001
          + 4 * U * np.abs(Z).max(axis=1) + 16 * U * c)
    e_lse = ez + (48 + 197) * U + 2.0 ** -22 + 2.0 ** -23 * np.abs(ref["lse"])
    lse_g = lse.cpu().numpy().astype(np.float64)
    assert (np.abs(lse_g[rows] - ref["lse"]) <= e_lse).all()
    Gd = ws[:M * V * 2].view(torch.bfloat16).view(M, V)
    Gr = F.bf16_to_f64(bits(Gd[torch.from_numpy(rows).to(DEV)]))
    assert rel_fro(Gr, ref["G"]) < 1e-2
    assert rel_fro(F.bf16_to_f64(bits(dX)[rows]), Gr @ Wf) < 4e-3
    cols = np.array([3, 25001, V - 1])
    Gc = F.bf16_to_f64(bits(Gd[:, torch.from_numpy(cols).to(DEV)].contiguous()))
    assert rel_fro(dW.cpu().numpy()[cols].astype(np.float64), Gc.T @ Xf) < 1e-4
