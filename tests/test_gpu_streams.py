"""Calls on two streams at once share no state: two blocks, each with its own
inputs, buffers and workspaces, run a training step (forward, backward, W2
cache refresh) concurrently on two streams, and each result must equal, bit
for bit, the same step run alone on the default stream."""
import numpy as np
import pytest
import torch

import fp8_relu_mlp_amd as fm
from fp8_relu_mlp_amd import synth

from .gpu_helpers import DEV, bf16_dev, bits, case

pytestmark = pytest.mark.gpu


def _setup(seed, M, d, h):
    ins = synth.mlp_inputs(M, d, h, seed, with_dy=True)
    X, dY = bf16_dev(ins["X"]), bf16_dev(ins["dY"])
    blk = fm.Relu2MLP(bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), margin=2.0, amax_init=1.0)
    L = fm.lib()
    bufs = {"post": torch.empty((M, h), dtype=torch.bfloat16, device=DEV),
            "post_q": torch.empty((M, h), dtype=torch.uint8, device=DEV),
            "Y": torch.empty((M, d), dtype=torch.bfloat16, device=DEV),
            "dX": torch.empty((M, d), dtype=torch.bfloat16, device=DEV),
            "dW1": torch.empty((h, d), dtype=torch.float32, device=DEV),
            "dW2": torch.empty((d, h), dtype=torch.float32, device=DEV),
            "wsf": torch.empty(max(1, L.mlp_relu2_fwd_workspace(M, d, h)), dtype=torch.uint8, device=DEV),
            "wsb": torch.empty(max(1, L.mlp_relu2_bwd_workspace(M, d, h)), dtype=torch.uint8, device=DEV),
            "wsc": torch.empty(max(1, L.fp8_cast_transpose_workspace(d, h)), dtype=torch.uint8, device=DEV)}
    return X, dY, blk, bufs


def _steps(X, dY, blk, b, stream, n=2):
    for _ in range(n):
        blk.forward(X, post=b["post"], post_q=b["post_q"], Y=b["Y"], workspace=b["wsf"], stream=stream)
        blk.backward(dY, X, b["post"], b["dX"], b["dW1"], b["dW2"], workspace=b["wsb"], stream=stream)
        blk.refresh_w2_cache(workspace=b["wsc"], stream=stream)


def _snap(blk, b):
    return {"Y": bits(b["Y"]), "dX": bits(b["dX"]), "post_q": b["post_q"].cpu().numpy(),
            "dW1": b["dW1"].cpu().numpy(), "dW2": b["dW2"].cpu().numpy(), "W2t": blk.W2t_q.cpu().numpy(),
            "amax": blk.amax_prev.cpu().numpy()}


def test_two_streams_match_sequential():
    fm.lib()
    shapes = [(3000, 256, 1024), (2048, 768, 3072)]
    case("streams: sequential reference")
    ref = []
    for i, (M, d, h) in enumerate(shapes):
        X, dY, blk, b = _setup(200 + i, M, d, h)
        _steps(X, dY, blk, b, None)
        torch.cuda.synchronize()
        ref.append(_snap(blk, b))
    case("streams: two at once")
    runs = [_setup(200 + i, M, d, h) for i, (M, d, h) in enumerate(shapes)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for (X, dY, blk, b), s in zip(runs, streams):
        with torch.cuda.stream(s):
            _steps(X, dY, blk, b, s)
    torch.cuda.synchronize()
    for i, (X, dY, blk, b) in enumerate(runs):
        got = _snap(blk, b)
        for k, v in ref[i].items():
            assert np.array_equal(got[k], v), (i, k)
