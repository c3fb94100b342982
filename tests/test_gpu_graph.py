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
    fm.mlp_relu2_fwd(fm.TRAIN_FP8, X, W1, W2t, w2_inv, None, amax_prev, 2.0, post, post_q, amax_prev, None, Y,
                     workspace=wsf)
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
