"""The allocation-free forward entry point (mlp_relu2_fwd_noalloc) against
mlp_relu2_fwd, through the C ABI: two calls in a row on one GPU, the second
with a smaller input, each bit-identical to the workspace entry point (the
same kernels run on the same inputs), in TRAIN and EVAL mode."""
import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth

from .gpu_helpers import DEV, bf16_dev, bits, case, f32_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fm():
    import fp8_relu_mlp_amd as fm
    fm.lib()
    return fm


def _run(fm, fn, mode, ins, W2t, w2_inv, amax_prev, ws=None):
    M, d = ins["X"].shape
    h = ins["W1"].shape[0]
    X, W1, W2 = bf16_dev(ins["X"]), bf16_dev(ins["W1"]), bf16_dev(ins["W2"])
    post = torch.full((M, h), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    post_q = torch.full((M, h), 0x55, dtype=torch.uint8, device=DEV) if mode == 0 else None
    Y = torch.full((M, d), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    amax_out, scale_out = f32_dev(-7.0), f32_dev(-7.0)
    args = (mode, X, W1, W2t, w2_inv, W2, f32_dev(amax_prev), 2.0, post, post_q, amax_out,
            scale_out if mode == 0 else None, Y)
    if fn == "noalloc":
        fm.mlp_relu2_fwd_noalloc(*args)
    else:
        fm.mlp_relu2_fwd(*args, workspace=ws)
    torch.cuda.synchronize()
    return {"post": bits(post), "post_q": None if post_q is None else post_q.cpu().numpy(), "y": bits(Y),
            "amax": amax_out.item(), "scale": scale_out.item()}


@pytest.mark.parametrize("mode", [0, 1])
def test_noalloc_matches_workspace_entry_point(fm, mode):
    d, h = 256, 1024
    for step, M in enumerate((3000, 700)):
        ins = synth.mlp_inputs(M, d, h, 21 + step)
        case(f"noalloc forward mode={mode} call {step + 1} M={M} d={d} h={h}")
        W2 = bf16_dev(ins["W2"])
        W2t = torch.empty((h, d), dtype=torch.uint8, device=DEV)
        w2_inv = f32_dev(0.0)
        fm.fp8_cast_transpose_w2(W2, W2t, None, w2_inv, None)
        ws = torch.empty(max(1, fm.lib().mlp_relu2_fwd_workspace(M, d, h)), dtype=torch.uint8, device=DEV)
        a = _run(fm, "workspace", mode, ins, W2t, w2_inv, 3.5, ws)
        b = _run(fm, "noalloc", mode, ins, W2t, w2_inv, 3.5)
        assert (a["post"] == b["post"]).all()
        assert (a["y"] == b["y"]).all()
        assert np.float32(a["amax"]).view(np.uint32) == np.float32(b["amax"]).view(np.uint32)
        if mode == 0:
            assert (a["post_q"] == b["post_q"]).all()
            assert np.float32(a["scale"]).view(np.uint32) == np.float32(b["scale"]).view(np.uint32)
