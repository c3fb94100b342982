"""The library under HIP graph capture: a whole training step of the block
(delayed-scale FP8 forward, bf16 backward, SGD on both weights, the W2 cache
refresh and the amax carry as a device copy) captured once with
torch.cuda.graph and replayed three times must reproduce, bit for bit, the
same three steps run eagerly.  Between replays the program does its own
eager work and synchronises, and every replay is checked.

Capture works because no entry point allocates, synchronises or reads a
device value on the host: buffers and workspaces come from the caller and
the per-step scalars (amax, scales) live on the device.
"""
import numpy as np
import pytest
import torch

import fp8_relu_mlp_amd as fm
from fp8_relu_mlp_amd import synth

from .gpu_helpers import DEV, bf16_dev, bits, case

pytestmark = pytest.mark.gpu


def test_step_captured_in_a_graph_replays_like_eager():
    fm.lib()
    M, d, h = 2048, 768, 3072
    ins = synth.mlp_inputs(M, d, h, 95, with_dy=True)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    W1, W2 = bf16_dev(ins["W1"]), bf16_dev(ins["W2"])
    f = lambda v=0.0: torch.full((1,), v, dtype=torch.float32, device=DEV)
    W2t = torch.empty((h, d), dtype=torch.uint8, device=DEV)
    w2_scale, w2_inv, w2_amax = f(), f(), f()
    amax_prev, amax_out, scale_out = f(1.0), f(), f()
    post = torch.empty((M, h), dtype=torch.bfloat16, device=DEV)
    post_q = torch.empty((M, h), dtype=torch.uint8, device=DEV)
    Y, dX = torch.empty((M, d), dtype=torch.bfloat16, device=DEV), torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    dW1 = torch.empty((h, d), dtype=torch.float32, device=DEV)
    dW2 = torch.empty((d, h), dtype=torch.float32, device=DEV)
    L = fm.lib()
    wsf = torch.empty(max(1, L.mlp_relu2_fwd_workspace(M, d, h)), dtype=torch.uint8, device=DEV)
    wsb = torch.empty(max(1, L.mlp_relu2_bwd_workspace(M, d, h)), dtype=torch.uint8, device=DEV)
    wsc = torch.empty(max(1, L.fp8_cast_transpose_workspace(d, h)), dtype=torch.uint8, device=DEV)
    lr = float(np.float32(1e-3 / M))

    def step():
        fm.mlp_relu2_fwd(fm.TRAIN_FP8, X, W1, W2t, w2_inv, None, amax_prev, 2.0, post, post_q, amax_out, scale_out,
                         Y, workspace=wsf)
        fm.mlp_relu2_bwd(dY, X, W1, W2, post, dX, dW1, dW2, workspace=wsb)
        fm.sgd_update_bf16(W1, dW1, lr)
        fm.sgd_update_bf16(W2, dW2, lr)
        fm.fp8_cast_transpose_w2(W2, W2t, w2_scale, w2_inv, w2_amax, workspace=wsc)
        amax_prev.copy_(amax_out)

    def snapshot():
        return {"Y": bits(Y), "dX": bits(dX), "post_q": post_q.cpu().numpy(), "W1": bits(W1), "W2t": W2t.cpu().numpy(),
                "dW2": dW2.cpu().numpy(), "amax": amax_out.cpu().numpy(), "scale": scale_out.cpu().numpy()}

    # the state every run starts from: the W2 cache and a measured amax
    fm.fp8_cast_transpose_w2(W2, W2t, w2_scale, w2_inv, w2_amax, workspace=wsc)
    # (amax_out may not alias amax_prev: the launch writes one while it reads the other)
    fm.mlp_relu2_fwd(fm.TRAIN_FP8, X, W1, W2t, w2_inv, None, amax_prev, 2.0, post, post_q, amax_out, None, Y,
                     workspace=wsf)
    amax_prev.copy_(amax_out)
    torch.cuda.synchronize()
    start = {k: v.clone() for k, v in (("W1", W1), ("W2", W2), ("W2t", W2t), ("w2_inv", w2_inv),
                                       ("amax_prev", amax_prev))}

    def reset():
        W1.copy_(start["W1"])
        W2.copy_(start["W2"])
        W2t.copy_(start["W2t"])
        w2_inv.copy_(start["w2_inv"])
        amax_prev.copy_(start["amax_prev"])
        torch.cuda.synchronize()

    case("graph: three eager steps")
    eager = []
    for _ in range(3):
        step()
        torch.cuda.synchronize()
        eager.append(snapshot())
    assert not (eager[0]["W1"] == eager[2]["W1"]).all()      # the state does move

    case("graph: capture one step")
    reset()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    reset()                                                   # capture ran nothing; start over anyway
    for i in range(3):
        case(f"graph: replay {i}")
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, v in eager[i].items():
            assert np.array_equal(got[k], v), (i, k)
        _ = float(amax_out.sum().item())                     # eager work between replays


def test_linear_and_cross_entropy_captured_in_a_graph():
    """fp8_linear on both of its paths (the row-panel kernel at K = 768, the
    conversion pass and GEMM at K = 1024; max |X| from the per-block maxima)
    and the softcapped cross-entropy in bf16 and with the e4m3 head, captured
    once and replayed three times on new inputs written eagerly between the
    replays: every replay equals the eager calls bit for bit."""
    fm.lib()
    L = fm.lib()
    f = lambda v=0.0: torch.full((1,), v, dtype=torch.float32, device=DEV)
    M = 1500
    lin = []
    for K, N in ((768, 2304), (1024, 320)):
        a = synth.attn_inputs(M=M, d=K, qkv=N, seed=96 + K)
        W = bf16_dev(a["Wqkv"])
        Wt, inv = torch.empty((K, N), dtype=torch.uint8, device=DEV), f()
        fm.fp8_cast_transpose(W, Wt, inv_scale_out=inv)
        lin.append({"X": bf16_dev(a["X"]), "Wt": Wt, "inv": inv, "sx": f(8.0), "Y": torch.empty((M, N),
                    dtype=torch.bfloat16, device=DEV), "xam": f(),
                    "ws": torch.empty(max(1, L.fp8_linear_workspace(M, K)), dtype=torch.uint8, device=DEV)})
    Mc, dc, V, T = 700, 256, 2048, 3
    ci = synth.ce_inputs(Mc, dc, V, T, 97, seq=100, head_var=16.0)
    Xc, Wc = bf16_dev(ci["X"]), bf16_dev(ci["W"])
    tg = torch.from_numpy(ci["targets"].astype(np.int32)).to(DEV)
    wts = torch.tensor([1.0, 0.5, 0.25], dtype=torch.float32, device=DEV)
    Wct, cinv = torch.empty((dc, V), dtype=torch.uint8, device=DEV), f()
    fm.fp8_cast_transpose(Wc, Wct, inv_scale_out=cinv)
    ce = {q: {"loss": f(), "dX": torch.empty((Mc, dc), dtype=torch.bfloat16, device=DEV),
              "dW": torch.empty((V, dc), dtype=torch.float32, device=DEV),
              "ws": torch.empty(max(1, (L.softcap_ce_fp8_workspace if q else L.softcap_ce_workspace)(Mc, V, dc, T)),
                                dtype=torch.uint8, device=DEV)} for q in (False, True)}
    xs = f(4.0)

    def calls():
        for c in lin:
            fm.fp8_linear(c["X"], c["sx"], c["Wt"], c["inv"], c["Y"], x_amax_out=c["xam"], workspace=c["ws"])
        o = ce[False]
        fm.softcap_ce_fwd_bwd(Xc, Wc, tg, wts, 15.0, o["loss"], o["dX"], o["dW"], workspace=o["ws"])
        o = ce[True]
        fm.softcap_ce_fwd_bwd_fp8(Xc, xs, Wct, cinv, Wc, tg, wts, 15.0, o["loss"], o["dX"], o["dW"],
                                  workspace=o["ws"])

    def snapshot():
        s = [bits(c["Y"]) for c in lin] + [c["xam"].cpu().numpy() for c in lin]
        for q in (False, True):
            s += [ce[q]["loss"].cpu().numpy(), bits(ce[q]["dX"]), ce[q]["dW"].cpu().numpy()]
        return s

    inputs = [(c["X"].clone()) for c in lin] + [Xc.clone()]

    def set_inputs(r):
        # new activations for replay r, written eagerly (a sign flip and a scale by 2^r: exact in bf16)
        for c, x0 in zip(lin, inputs):
            c["X"].copy_(x0 * (float(2 ** r) * (-1.0) ** r))
        Xc.copy_(inputs[-1] * (-1.0) ** r)

    case("fp8_linear and cross-entropy: capture")
    set_inputs(0)
    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for r in range(1, 4):
        case(f"fp8_linear and cross-entropy: replay {r}")
        set_inputs(r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        calls()
        torch.cuda.synchronize()
        want = snapshot()
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(np.asarray(a), np.asarray(b)), (r, i)
    del g


def test_variant_step_captured_in_a_graph():
    """The forward with both GEMMs in e4m3 (mlp_relu2_fwd_fp8up, X converted
    in the launch sequence, max |X| out) and the backward on the e4m3 post copy
    (mlp_relu2_bwd_fp8post) captured once, replayed three times on new X and
    dY written between the replays: bit-identical to the eager calls."""
    fm.lib()
    L = fm.lib()
    M, d, h = 2000, 768, 3072
    ins = synth.mlp_inputs(M, d, h, 98, with_dy=True)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    X0, dY0 = X.clone(), dY.clone()
    W1, W2 = bf16_dev(ins["W1"]), bf16_dev(ins["W2"])
    f = lambda v=0.0: torch.full((1,), v, dtype=torch.float32, device=DEV)
    W1t = torch.empty((d, h), dtype=torch.uint8, device=DEV)
    W2t = torch.empty((h, d), dtype=torch.uint8, device=DEV)
    inv1, inv2 = f(), f()
    fm.fp8_cast_transpose(W1, W1t, inv_scale_out=inv1)
    fm.fp8_cast_transpose(W2, W2t, inv_scale_out=inv2)
    sx, amax_prev, amax_out, scale_out, xam = f(40.0), f(3.0), f(), f(), f()
    post_q = torch.empty((M, h), dtype=torch.uint8, device=DEV)
    Y, dX = torch.empty((M, d), dtype=torch.bfloat16, device=DEV), torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    dW1 = torch.empty((h, d), dtype=torch.float32, device=DEV)
    dW2 = torch.empty((d, h), dtype=torch.float32, device=DEV)
    wsf = torch.empty(max(1, L.mlp_relu2_fwd_fp8up_workspace(M, d, h)), dtype=torch.uint8, device=DEV)
    wsb = torch.empty(max(1, L.mlp_relu2_bwd_workspace(M, d, h)), dtype=torch.uint8, device=DEV)

    def calls():
        # post = None: only the e4m3 copy is kept, and the backward reads it
        fm.mlp_relu2_fwd_fp8up(X, sx, W1t, inv1, W2t, inv2, amax_prev, 2.0, None, post_q, amax_out, scale_out, Y,
                               x_amax_out=xam, workspace=wsf)
        fm.mlp_relu2_bwd_fp8post(dY, X, W1, W2, post_q, scale_out, dX, dW1, dW2, workspace=wsb)

    def snapshot():
        return [bits(Y), post_q.cpu().numpy(), amax_out.cpu().numpy(), scale_out.cpu().numpy(), xam.cpu().numpy(),
                bits(dX), dW1.cpu().numpy(), dW2.cpu().numpy()]

    def set_inputs(r):
        X.copy_(X0 * (-1.0) ** r)
        dY.copy_(dY0 * float(2 ** r))

    case("variant step: capture")
    set_inputs(0)
    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for r in range(1, 4):
        case(f"variant step: replay {r}")
        set_inputs(r)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        calls()
        torch.cuda.synchronize()
        want = snapshot()
        for i, (a, b) in enumerate(zip(got, want)):
            assert np.array_equal(np.asarray(a), np.asarray(b)), (r, i)
    del g
