"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

* libfp8mlp.so loads and exports every function include/fp8mlp.h declares;
* the Python binding declares exactly those functions;
* workspace queries and argument validation (which runs on the host before
  any device call) return the documented status codes.

The validation tests pass small integers as device addresses: they rely on
the library rejecting the call before it touches a device.  On a host where a
GPU is visible a regression in the order of the checks could launch a kernel
on such an address, so those tests skip themselves there (the `L_nogpu`
fixture); the load / export checks run everywhere.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8mlp.h")
LIBP = os.path.join(ROOT, "fp8_relu_mlp_amd", "libfp8mlp.so")

OK, E_NULL, E_SHAPE, E_ALIGN, E_WS, E_ARCH, E_HIP, E_ARG = 0, -1, -2, -3, -4, -5, -6, -7


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIBP):
        pytest.fail("libfp8mlp.so is not built (run __graft_entry__.build())")
    from fp8_relu_mlp_amd import _lib
    return _lib.lib()


def _gpu_visible():
    """A GPU is visible to this process (device_count does not initialise HIP)."""
    if os.environ.get("HIP_VISIBLE_DEVICES") == "-1":
        return False
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return os.path.exists("/dev/kfd")


@pytest.fixture(scope="module")
def L_nogpu(L):
    if _gpu_visible():
        pytest.skip("fake device addresses are passed to the library: not run where a GPU is visible")
    return L


def test_header_declares_the_boundary():
    names = declared()
    for must in ("mlp_relu2_fwd", "mlp_relu2_bwd", "fp8_cast_transpose_w2", "amax_reduce", "fp8_linear"):
        assert must in names


def test_library_exports_every_declared_symbol(L):
    raw = ctypes.CDLL(LIBP)
    missing = [n for n in declared() if not hasattr(raw, n)]
    assert not missing, missing


def test_no_failed_kernel_before_any_launch(L):
    """fp8mlp_last_failed_kernel() (FP8MLP_SYNC_CHECK=1 debug mode) names
    nothing until a checked launch has failed on this thread."""
    assert L.fp8mlp_last_failed_kernel() is None


def test_binding_covers_the_header(L):
    from fp8_relu_mlp_amd import _lib
    assert sorted(_lib.SIGNATURES) == declared()


def test_version_and_status_strings(L):
    assert L.fp8mlp_abi_version() == 1
    for st in (OK, E_NULL, E_SHAPE, E_ALIGN, E_WS, E_ARCH, E_HIP, E_ARG):
        assert len(L.fp8mlp_status_str(st)) >= 2
    assert L.fp8mlp_status_str(12345) == b"unknown status"


def test_workspace_sizes(L):
    M, d, h = 49152, 768, 3072
    assert L.mlp_relu2_fwd_workspace(M, d, h) == 192 * 12 * 4 + (256 - (192 * 12 * 4) % 256) % 256
    bw = L.mlp_relu2_bwd_workspace(M, d, h)
    assert bw >= M * h * 2                      # dpre
    assert L.mlp_relu2_fwd_workspace(0, d, h) == 0
    assert L.amax_reduce_workspace(100) == 0
    assert L.amax_reduce_workspace(1 << 20) > 0
    assert L.fp8_cast_transpose_workspace(768, 3072) >= 256


def test_bwd_split_ranges_fit_32bit_offsets(L):
    """The dW GEMMs address one token range of dpre / dY (rows of 2 max(d, h)
    bytes) with 32-bit byte offsets: the backward's workspace must hold
    split-k partials for at least M * 2 max(d, h) / 2^31 ranges (each split:
    one fp32 copy of dW1 and one of dW2), at 4M and 6M tokens of the
    GPT-2-small block and at 300000 tokens of a d=2048, h=8192 block, whose
    256 dW tiles alone would leave the tokens in one range."""
    for M, d, h in ((1 << 22, 768, 3072), (3 << 21, 768, 3072), (300000, 2048, 8192)):
        ws = L.mlp_relu2_bwd_workspace(M, d, h)
        fixed = M * h * 2 + 2 * h * d * 2                  # dpre, W1t and W2t
        min_splits = -(-M * 2 * max(d, h) // (1 << 31))
        assert ws - fixed >= 2 * min_splits * h * d * 4, (M, ws)


def _fwd(L, **kw):
    args = dict(mode=0, X=16, W1=16, W2t_q=16, w2_inv=16, W2=None, amax_prev=32, margin=2.0, post=16,
                post_q=16, amax_out=48, scale_out=None, Y=16, M=256, d=128, h=512, ws=16, wsb=1 << 20,
                stream=None)
    args.update(kw)
    return L.mlp_relu2_fwd(*args.values())


def test_fwd_validation_before_any_device_call(L_nogpu):
    L = L_nogpu
    assert _fwd(L, mode=7) == E_ARG
    assert _fwd(L, d=100) == E_SHAPE
    assert _fwd(L, h=192) == E_SHAPE            # train needs h % 128 == 0
    assert _fwd(L, M=-1) == E_SHAPE
    # past the 32-bit addressing limits: a feature size above 2^22, a weight of 2^31 elements
    assert _fwd(L, d=(1 << 22) + 64) == E_SHAPE
    assert _fwd(L, d=1 << 16, h=1 << 15) == E_SHAPE
    assert _fwd(L, X=None) == E_NULL
    assert _fwd(L, amax_out=None) == E_NULL
    assert _fwd(L, post_q=None) == E_NULL
    assert _fwd(L, X=24) == E_ALIGN
    assert _fwd(L, margin=0.0) == E_ARG
    assert _fwd(L, margin=float("nan")) == E_ARG
    assert _fwd(L, ws=None) == E_WS
    assert _fwd(L, wsb=8) == E_WS
    assert _fwd(L, mode=1, W2=None) == E_NULL   # eval needs the bf16 W2
    # the allocation-free variant: the same checks, and a size limit instead of a workspace
    nf = lambda **kw: L.mlp_relu2_fwd_noalloc(*[v for k, v in dict(
        dict(mode=0, X=16, W1=16, W2t_q=16, w2_inv=16, W2=None, amax_prev=32, margin=2.0, post=16, post_q=16,
             amax_out=48, scale_out=None, Y=16, M=256, d=128, h=512, stream=None), **kw).items()])
    assert L.mlp_relu2_fwd_noalloc_max_bytes() == 256 * 1024
    assert nf(d=100) == E_SHAPE
    assert nf(X=None) == E_NULL
    assert nf(amax_out=32) == E_ARG
    assert nf(M=1 << 20, h=1 << 15) == E_WS                    # partial amax > 256 KB
    # amax_t is written while amax_{t-1} is still read: no aliasing
    assert _fwd(L, amax_out=32) == E_ARG
    assert _fwd(L, scale_out=32) == E_ARG
    assert _fwd(L, scale_out=48) == E_ARG


def test_bwd_and_misc_validation(L_nogpu):
    L = L_nogpu
    b = lambda **kw: L.mlp_relu2_bwd(*dict(dict(dY=16, X=16, W1=16, W2=16, post=16, dX=16, dW1=16, dW2=16,
                                                 acc=0, M=256, d=128, h=512, ws=16, wsb=1 << 30,
                                                 stream=None), **kw).values())
    assert b(acc=2) == E_ARG
    assert b(h=100) == E_SHAPE
    assert b(h=(1 << 22) + 128) == E_SHAPE
    assert b(d=1 << 15, h=1 << 16) == E_SHAPE
    assert b(dW1=None) == E_NULL
    assert b(post=40) == E_ALIGN
    assert b(wsb=10) == E_WS
    assert L.amax_reduce(5, 16, 10, 16, None, 0, None) == E_ARG
    assert L.amax_reduce(0, 16, -1, 16, None, 0, None) == E_SHAPE
    assert L.amax_reduce(0, 16, 10, None, None, 0, None) == E_NULL
    assert L.amax_reduce(0, 16, 1 << 20, 16, None, 0, None) == E_WS
    assert L.fp8_cast_transpose(16, 30, 64, 16, None, None, None, None, 16, 1 << 20, None) == E_SHAPE
    assert L.fp8_cast_transpose(None, 64, 64, 16, None, None, None, None, 16, 1 << 20, None) == E_NULL
    assert L.fp8_cast_transpose(16, 64, 64, 16, None, None, None, None, None, 0, None) == E_WS
    assert L.fp8_scale_from_amax(None, 2.0, None, None, None) == E_NULL
    assert L.fp8_scale_from_amax(16, -1.0, None, None, None) == E_ARG
    lin = lambda **kw: L.fp8_linear(*dict(dict(X=16, xs=16, W=16, wi=16, Y=16, am=None, M=100, K=256, N=256,
                                                ws=16, wsb=1 << 20, st=None), **kw).values())
    assert lin(K=160) == E_SHAPE              # K % 64
    assert lin(N=(1 << 22) + 64) == E_SHAPE
    assert lin(K=1 << 16, N=1 << 15) == E_SHAPE   # Wt_q of 2^31 codes
    assert lin(xs=None) == E_NULL
    assert lin(Y=17) == E_ALIGN
    assert lin(ws=None) == E_WS
    assert lin(wsb=100) == E_WS
    assert lin(am=16) == E_ARG                # x_amax_out aliases x_scale
    # X, W, targets, T, weights, softcap, dloss, loss_out, lse_out, dX, dW, accumulate, M, V, d
    ce = lambda M, V, d: L.softcap_ce_fwd_bwd(16, 16, 16, 1, 16, 15.0, None, 16, None, 16, 16, 0, M, V, d,
                                              16, 1 << 40, None)
    assert ce(256, 100, 64) == E_SHAPE        # V % 64
    assert ce(256, (1 << 22) + 64, 64) == E_SHAPE
    assert ce(256, 1 << 16, 1 << 15) == E_SHAPE   # W of 2^31 elements


def test_stack_helpers_validation(L_nogpu):
    L = L_nogpu
    assert L.rmsnorm_fwd(16, 16, 16, 4, 100, 1e-6, None) == E_SHAPE     # d % 8
    assert L.rmsnorm_fwd(16, 16, 16, -1, 64, 1e-6, None) == E_SHAPE
    assert L.rmsnorm_fwd(16, 16, 16, 4, 64, -1.0, None) == E_ARG
    assert L.rmsnorm_fwd(None, 16, 16, 4, 64, 1e-6, None) == E_NULL
    assert L.rmsnorm_fwd(16, 24, 16, 4, 64, 1e-6, None) == E_ALIGN
    assert L.rmsnorm_fwd(None, None, None, 0, 64, 1e-6, None) == OK       # empty: nothing to do
    assert L.rmsnorm_bwd(16, 16, 16, None, 16, 4, 64, None) == E_NULL
    assert L.rmsnorm_bwd(16, 18, 16, 16, 16, 4, 64, None) == E_ALIGN     # inv_rms 4-byte aligned
    assert L.add_bf16(16, 16, 16, 12, None) == E_SHAPE
    assert L.add_bf16(16, None, 16, 16, None) == E_NULL
    assert L.sgd_update_bf16(16, 16, 12, 1e-3, None) == E_SHAPE
    assert L.sgd_update_bf16(16, 16, 16, float("nan"), None) == E_ARG
    assert L.sgd_update_bf16(16, 40, 16, 1e-3, None) == E_ALIGN


def test_variant_entry_points_validation(L_nogpu):
    """The e4m3 up-projection forward, the backward on the e4m3 post copy and
    the top-code count reject bad arguments before touching a device."""
    L = L_nogpu
    ws = L.mlp_relu2_fwd_fp8up_workspace(256, 128, 256)
    assert ws >= 256 * 128 and L.mlp_relu2_fwd_fp8up_workspace(0, 128, 256) == 0
    # X, x_scale, W1t_q, w1_inv, W2t_q, w2_inv, amax_prev, margin, post, post_q, amax_out, scale_out, Y,
    # x_amax_out
    args = [16, 20, 16, 24, 16, 28, 32, 2.0, 16, 16, 36, 40, 16, 44]
    assert L.mlp_relu2_fwd_fp8up(*args, 256, 192, 256, 16, ws, None) == E_SHAPE    # d % 128
    assert L.mlp_relu2_fwd_fp8up(*args, 256, 128, 192, 16, ws, None) == E_SHAPE    # h % 128
    assert L.mlp_relu2_fwd_fp8up(*args, 256, 1 << 16, 1 << 15, 16, ws, None) == E_SHAPE  # 2^31-element W1
    bad = list(args)
    bad[1] = None                                                                   # x_scale
    assert L.mlp_relu2_fwd_fp8up(*bad, 256, 128, 256, 16, ws, None) == E_NULL
    bad = list(args)
    bad[7] = 0.0                                                                    # margin
    assert L.mlp_relu2_fwd_fp8up(*bad, 256, 128, 256, 16, ws, None) == E_ARG
    assert L.mlp_relu2_fwd_fp8up(*args, 256, 128, 256, 16, ws - 1, None) == E_WS
    for i, j in ((10, 6), (11, 6), (11, 10), (13, 1), (13, 6), (13, 10)):
        bad = list(args)
        bad[i] = bad[j]                                                             # aliased scalars
        assert L.mlp_relu2_fwd_fp8up(*bad, 256, 128, 256, 16, ws, None) == E_ARG, (i, j)
    wb = L.mlp_relu2_bwd_workspace(256, 128, 256)
    assert L.mlp_relu2_bwd_fp8post(16, 16, 16, 16, 16, None, 16, 16, 16, 0, 256, 128, 256, 16, wb,
                                   None) == E_NULL                                  # post_scale
    assert L.mlp_relu2_bwd_fp8post(16, 16, 16, 16, 16, 18, 16, 16, 16, 0, 256, 128, 256, 16, wb,
                                   None) == E_ALIGN
    assert L.mlp_relu2_bwd_fp8post(16, 16, 16, 16, 16, 16, 16, 16, 16, 2, 256, 128, 256, 16, wb,
                                   None) == E_ARG                                   # accumulate
    assert L.fp8_saturation_count_workspace(0) == 0 and L.fp8_saturation_count_workspace(16) > 0
    assert L.fp8_saturation_count(16, 24, 16, 16, 1 << 20, None) == E_SHAPE          # n % 16
    assert L.fp8_saturation_count(16, 32, None, 16, 1 << 20, None) == E_NULL
    assert L.fp8_saturation_count(16, 32, 12, 16, 1 << 20, None) == E_ALIGN           # 8-byte count
    assert L.fp8_saturation_count(16, 32, 16, 16, 0, None) == E_WS


def test_product_path_fails_loudly(monkeypatch):
    """No CPU fallback: without the built library the first call raises, and
    tensors outside GPU memory are refused before any call."""
    import torch
    import fp8_relu_mlp_amd as fm
    from fp8_relu_mlp_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libfp8mlp.so")
    with pytest.raises(ImportError):
        fm.amax_reduce(torch.zeros(16), torch.zeros(1))
    with pytest.raises(ValueError):
        fm._p(torch.zeros(4))
