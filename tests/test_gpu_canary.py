"""Guard bands around every output (no byte outside an output tensor or a
workspace is written).

Every output of the forward (post, post_q, Y, amax, scale), the backward
(dX, dW1, dW2), the W2 cache refresh, fp8_linear and the softcapped
cross-entropy -- and every workspace -- is carved out of a larger buffer
whose bytes before and after the tensor hold a sentinel pattern.  The calls
run with ragged token counts (not a multiple of any tile height) and feature
sizes that leave partial column tiles; afterwards every sentinel byte must be
unchanged.  The interior tiles of the GEMM epilogues store through unchecked
32-bit buffer offsets, so this is the check that they stay inside their
tensor.
"""
import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth

from .gpu_helpers import DEV, bf16_dev, case

pytestmark = pytest.mark.gpu

PAD = 4096          # sentinel bytes on each side (a multiple of 256: keeps alignment)
SENT = 0xA5


@pytest.fixture(scope="module")
def fm():
    import fp8_relu_mlp_amd as fm
    fm.lib()
    return fm


class Guarded:
    """Tensors carved out of sentinel-filled byte buffers."""

    def __init__(self):
        self.bufs = []

    def __call__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((PAD + n + PAD,), SENT, dtype=torch.uint8, device=DEV)
        t = raw[PAD:PAD + n].view(dtype).view(shape)
        if fill is not None:
            t.fill_(fill)
        self.bufs.append((raw, n))
        return t

    def ws(self, nbytes):
        return self((max(1, nbytes),), torch.uint8, fill=0)

    def check(self):
        torch.cuda.synchronize()
        for i, (raw, n) in enumerate(self.bufs):
            head = raw[:PAD].cpu().numpy()
            tail = raw[PAD + n:].cpu().numpy()
            assert (head == SENT).all() and (tail == SENT).all(), f"buffer {i}: bytes written outside the tensor"


@pytest.mark.parametrize("M,d,h", [(777, 192, 384), (1000, 64, 640), (2500, 256, 1152), (257, 768, 3072)])
def test_mlp_fwd_bwd_stay_inside(fm, M, d, h):
    case(f"guard bands fwd+bwd M={M} d={d} h={h}")
    L = fm.lib()
    ins = synth.mlp_inputs(M, d, h, 31, with_dy=True)
    g = Guarded()
    X, W1, W2, dY = bf16_dev(ins["X"]), bf16_dev(ins["W1"]), bf16_dev(ins["W2"]), bf16_dev(ins["dY"])
    W2t = g((h, d), torch.uint8)
    w2s, w2i, w2a = (g((1,), torch.float32) for _ in range(3))
    fm.fp8_cast_transpose_w2(W2, W2t, w2s, w2i, w2a, workspace=g.ws(L.fp8_cast_transpose_workspace(d, h)))
    post = g((M, h), torch.bfloat16)
    post_q = g((M, h), torch.uint8)
    Y = g((M, d), torch.bfloat16)
    amax_prev = g((1,), torch.float32, fill=5.0)
    amax_out, scale_out = g((1,), torch.float32), g((1,), torch.float32)
    fm.mlp_relu2_fwd(0, X, W1, W2t, w2i, W2, amax_prev, 2.0, post, post_q, amax_out, scale_out, Y,
                     workspace=g.ws(L.mlp_relu2_fwd_workspace(M, d, h)))
    Ye = g((M, d), torch.bfloat16)
    poste = g((M, h), torch.bfloat16)
    amax_e = g((1,), torch.float32)
    fm.mlp_relu2_fwd(1, X, W1, None, None, W2, None, 2.0, poste, None, amax_e, None, Ye,
                     workspace=g.ws(L.mlp_relu2_fwd_workspace(M, d, h)))
    dX = g((M, d), torch.bfloat16)
    dW1, dW2 = g((h, d), torch.float32), g((d, h), torch.float32)
    fm.mlp_relu2_bwd(dY, X, W1, W2, post, dX, dW1, dW2, workspace=g.ws(L.mlp_relu2_bwd_workspace(M, d, h)))
    fm.mlp_relu2_bwd(dY, X, W1, W2, post, dX, dW1, dW2, accumulate=True,
                     workspace=g.ws(L.mlp_relu2_bwd_workspace(M, d, h)))
    g.check()
    assert torch.isfinite(dW1).all() and torch.isfinite(Y.float()).all()


@pytest.mark.parametrize("M,K,N", [(1000, 256, 320), (333, 768, 2304), (700, 192, 256), (601, 960, 320)])
def test_fp8_linear_stays_inside(fm, M, K, N):
    case(f"guard bands fp8_linear M={M} K={K} N={N}")
    L = fm.lib()
    a = synth.attn_inputs(M=M, d=K, qkv=N, seed=4)
    g = Guarded()
    X, W = bf16_dev(a["X"]), bf16_dev(a["Wqkv"])
    Wt = g((K, N), torch.uint8)
    inv = g((1,), torch.float32)
    fm.fp8_cast_transpose(W, Wt, inv_scale_out=inv, workspace=g.ws(L.fp8_cast_transpose_workspace(N, K)))
    sx = g((1,), torch.float32, fill=40.0)
    xam = g((1,), torch.float32)
    Y = g((M, N), torch.bfloat16)
    fm.fp8_linear(X, sx, Wt, inv, Y, x_amax_out=xam, workspace=g.ws(L.fp8_linear_workspace(M, K)))
    g.check()


def test_ce_stays_inside(fm):
    M, d, V, T = 1000, 128, 1088, 3
    case(f"guard bands softcapped CE M={M} d={d} V={V}")
    L = fm.lib()
    ins = synth.ce_inputs(M, d, V, T, 6, seq=256)
    g = Guarded()
    X, W = bf16_dev(ins["X"]), bf16_dev(ins["W"])
    t = torch.from_numpy(ins["targets"].astype(np.int32)).to(DEV)
    w = torch.tensor([1.0, 0.5, 0.25], dtype=torch.float32, device=DEV)
    loss, lse = g((1,), torch.float32), g((M,), torch.float32)
    dX, dW = g((M, d), torch.bfloat16), g((V, d), torch.float32)
    fm.softcap_ce_fwd_bwd(X, W, t, w, 15.0, loss, dX, dW, lse_out=lse,
                          workspace=g.ws(L.softcap_ce_workspace(M, V, d, T)))
    g.check()
