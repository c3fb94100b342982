"""FP8MLP_SYNC_CHECK=1 debug mode: every launch waits for its stream and
checks for a kernel failure.  The results must be bit-identical to the normal
asynchronous mode, nothing may be reported as failed, and graph capture must
still work (the wait is skipped on a capturing stream)."""
import numpy as np
import pytest
import torch

import fp8_relu_mlp_amd as fm
from fp8_relu_mlp_amd import synth

from .gpu_helpers import DEV, bf16_dev, bits, case

pytestmark = pytest.mark.gpu


def _step(M, d, h):
    ins = synth.mlp_inputs(M, d, h, 123, with_dy=True)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    W1, W2 = bf16_dev(ins["W1"]), bf16_dev(ins["W2"])
    blk = fm.Relu2MLP(W1, W2, margin=2.0, amax_init=1.0)
    post = torch.empty((M, h), dtype=torch.bfloat16, device=DEV)
    post_q = torch.empty((M, h), dtype=torch.uint8, device=DEV)
    Y = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    dX = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    dW1 = torch.empty((h, d), dtype=torch.float32, device=DEV)
    dW2 = torch.empty((d, h), dtype=torch.float32, device=DEV)
    for _ in range(2):
        blk.forward(X, post=post, post_q=post_q, Y=Y)
        blk.backward(dY, X, post, dX, dW1, dW2)
        blk.refresh_w2_cache()
    torch.cuda.synchronize()
    return {"post": bits(post), "post_q": post_q.cpu().numpy(), "Y": bits(Y), "dX": bits(dX),
            "dW1": dW1.cpu().numpy(), "dW2": dW2.cpu().numpy(), "W2t": blk.W2t_q.cpu().numpy()}


def test_sync_check_mode_matches_async(monkeypatch):
    fm.lib()
    M, d, h = 1000, 256, 640
    case("sync check: async reference")
    monkeypatch.delenv("FP8MLP_SYNC_CHECK", raising=False)
    ref = _step(M, d, h)
    case("sync check: FP8MLP_SYNC_CHECK=1")
    monkeypatch.setenv("FP8MLP_SYNC_CHECK", "1")
    got = _step(M, d, h)
    for k in ref:
        assert np.array_equal(ref[k], got[k]), k
    assert fm.lib().fp8mlp_last_failed_kernel() is None


def test_sync_check_mode_under_graph_capture(monkeypatch):
    fm.lib()
    monkeypatch.setenv("FP8MLP_SYNC_CHECK", "1")
    case("sync check: graph capture")
    N, K = 768, 3072
    W = bf16_dev(synth.normal_bf16((N, K), 1.0 / K, 9, "Wdbg"))
    out = torch.empty((K, N), dtype=torch.uint8, device=DEV)
    s, inv, am = (torch.zeros(1, dtype=torch.float32, device=DEV) for _ in range(3))
    ws = torch.empty(max(1, fm.lib().fp8_cast_transpose_workspace(N, K)), dtype=torch.uint8, device=DEV)
    fm.fp8_cast_transpose(W, out, scale_out=s, inv_scale_out=inv, amax_out=am, workspace=ws)
    torch.cuda.synchronize()
    eager = out.cpu().numpy().copy()
    out.zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fm.fp8_cast_transpose(W, out, scale_out=s, inv_scale_out=inv, amax_out=am, workspace=ws)
    for _ in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), eager)
    assert fm.lib().fp8mlp_last_failed_kernel() is None
