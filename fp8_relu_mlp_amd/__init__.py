"""Fused FP8 ReLU^2 MLP for AMD Instinct MI355X (gfx950).

Python binding of libfp8mlp (include/fp8mlp.h).  The functions below only
marshal torch tensors (device pointers, sizes, the current HIP stream) into
the C ABI; every step of the computation runs in the library's HIP kernels.
PyTorch supplies device memory and streams and nothing else.  If the library
is not built, the first call raises.

Entry points (same names as the C ABI):
  mlp_relu2_fwd, mlp_relu2_fwd_noalloc, mlp_relu2_fwd_fp8up, mlp_relu2_bwd, mlp_relu2_bwd_fp8post, fp8_cast_transpose, fp8_cast_transpose_w2,
  amax_reduce, fp8_scale_from_amax, fp8_linear, fp8_saturation_count,
  softcap_ce_fwd_bwd, softcap_ce_fwd_bwd_fp8, and the layer-stack helpers
  rmsnorm_fwd, rmsnorm_bwd, add_bf16, sgd_update_bf16
and ``Relu2MLP``, one MLP block's device state (bf16 weights, the transposed
fp8 W2 cache with its scales, the delayed-scale amax carried between steps);
``stack.Relu2Stack`` trains a stack of such blocks.
"""
import torch

from ._lib import Fp8MlpError, check, lib  # noqa: F401

TRAIN_FP8 = 0
EVAL_BF16 = 1
F32 = 0
BF16 = 1

__all__ = ["mlp_relu2_fwd", "mlp_relu2_fwd_noalloc", "mlp_relu2_fwd_fp8up", "mlp_relu2_bwd", "mlp_relu2_bwd_fp8post", "fp8_cast_transpose", "fp8_cast_transpose_w2", "amax_reduce",
           "fp8_scale_from_amax", "fp8_linear", "fp8_saturation_count", "softcap_ce_fwd_bwd", "softcap_ce_fwd_bwd_fp8",
           "rmsnorm_fwd", "rmsnorm_bwd", "add_bf16", "sgd_update_bf16",
           "Relu2MLP", "KernelTimer", "Fp8MlpError", "TRAIN_FP8", "EVAL_BF16"]


def _p(t):
    """Device pointer of a tensor (or NULL for None)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("fp8mlp tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("fp8mlp tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ws(nbytes, workspace, device):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def mlp_relu2_fwd(mode, X, W1, W2t_q, w2_inv_scale, W2, amax_prev, margin, post, post_q, amax_out, scale_out, Y,
                  workspace=None, stream=None):
    """See mlp_relu2_fwd in include/fp8mlp.h.  X [M,d] bf16, W1 [h,d] bf16,
    W2t_q [h,d] uint8, W2 [d,h] bf16, post [M,h] bf16, post_q [M,h] uint8,
    Y [M,d] bf16; scalars are 1-element fp32 device tensors."""
    M, d = X.shape
    h = W1.shape[0]
    L = lib()
    ws, wsb = _ws(L.mlp_relu2_fwd_workspace(M, d, h), workspace, X.device)
    check("mlp_relu2_fwd", L.mlp_relu2_fwd(
        mode, _p(X), _p(W1), _p(W2t_q), _p(w2_inv_scale), _p(W2), _p(amax_prev), float(margin), _p(post),
        _p(post_q), _p(amax_out), _p(scale_out), _p(Y), M, d, h, _p(ws), wsb, _stream(stream)))


def mlp_relu2_fwd_noalloc(mode, X, W1, W2t_q, w2_inv_scale, W2, amax_prev, margin, post, post_q, amax_out,
                          scale_out, Y, stream=None):
    """See mlp_relu2_fwd_noalloc in include/fp8mlp.h: mlp_relu2_fwd without a
    workspace (the library's per-GPU scratch array holds the partial amax)."""
    M, d = X.shape
    h = W1.shape[0]
    check("mlp_relu2_fwd_noalloc", lib().mlp_relu2_fwd_noalloc(
        mode, _p(X), _p(W1), _p(W2t_q), _p(w2_inv_scale), _p(W2), _p(amax_prev), float(margin), _p(post),
        _p(post_q), _p(amax_out), _p(scale_out), _p(Y), M, d, h, _stream(stream)))


def mlp_relu2_fwd_fp8up(X, x_scale, W1t_q, w1_inv_scale, W2t_q, w2_inv_scale, amax_prev, margin, post, post_q,
                        amax_out, scale_out, Y, x_amax_out=None, workspace=None, stream=None):
    """See mlp_relu2_fwd_fp8up in include/fp8mlp.h: the training forward with
    both GEMMs in e4m3.  X [M,d] bf16, W1t_q [d,h] uint8 (fp8_cast_transpose of
    W1), W2t_q [h,d] uint8; scalars are 1-element fp32 device tensors."""
    M, d = X.shape
    h = W1t_q.shape[1]
    L = lib()
    ws, wsb = _ws(L.mlp_relu2_fwd_fp8up_workspace(M, d, h), workspace, X.device)
    check("mlp_relu2_fwd_fp8up", L.mlp_relu2_fwd_fp8up(
        _p(X), _p(x_scale), _p(W1t_q), _p(w1_inv_scale), _p(W2t_q), _p(w2_inv_scale), _p(amax_prev),
        float(margin), _p(post), _p(post_q), _p(amax_out), _p(scale_out), _p(Y), _p(x_amax_out), M, d, h,
        _p(ws), wsb, _stream(stream)))


def mlp_relu2_bwd(dY, X, W1, W2, post, dX, dW1, dW2, accumulate=False, workspace=None, stream=None):
    """See mlp_relu2_bwd in include/fp8mlp.h.  dW1 [h,d], dW2 [d,h] fp32."""
    M, d = X.shape
    h = W1.shape[0]
    L = lib()
    ws, wsb = _ws(L.mlp_relu2_bwd_workspace(M, d, h), workspace, X.device)
    check("mlp_relu2_bwd", L.mlp_relu2_bwd(
        _p(dY), _p(X), _p(W1), _p(W2), _p(post), _p(dX), _p(dW1), _p(dW2), int(bool(accumulate)), M, d, h,
        _p(ws), wsb, _stream(stream)))


def mlp_relu2_bwd_fp8post(dY, X, W1, W2, post_q, post_scale, dX, dW1, dW2, accumulate=False, workspace=None,
                          stream=None):
    """See mlp_relu2_bwd_fp8post in include/fp8mlp.h: the backward from the
    e4m3 post copy post_q [M,h] (uint8) and the scale its forward used."""
    M, d = X.shape
    h = W1.shape[0]
    L = lib()
    ws, wsb = _ws(L.mlp_relu2_bwd_workspace(M, d, h), workspace, X.device)
    check("mlp_relu2_bwd_fp8post", L.mlp_relu2_bwd_fp8post(
        _p(dY), _p(X), _p(W1), _p(W2), _p(post_q), _p(post_scale), _p(dX), _p(dW1), _p(dW2), int(bool(accumulate)),
        M, d, h, _p(ws), wsb, _stream(stream)))


def fp8_cast_transpose(W, Wt_q, scale_in=None, scale_out=None, inv_scale_out=None, amax_out=None,
                       workspace=None, stream=None):
    """bf16 W [N,K] -> e4m3 Wt_q [K,N] (uint8); see include/fp8mlp.h."""
    N, K = W.shape
    L = lib()
    ws, wsb = _ws(L.fp8_cast_transpose_workspace(N, K), workspace, W.device)
    check("fp8_cast_transpose", L.fp8_cast_transpose(
        _p(W), N, K, _p(Wt_q), _p(scale_in), _p(scale_out), _p(inv_scale_out), _p(amax_out), _p(ws), wsb,
        _stream(stream)))


def fp8_cast_transpose_w2(W2, W2t_q, scale_out=None, inv_scale_out=None, amax_out=None, workspace=None,
                          stream=None):
    """Exact refresh of the transposed fp8 W2 cache: W2 [d,h] -> W2t_q [h,d]."""
    d, h = W2.shape
    L = lib()
    ws, wsb = _ws(L.fp8_cast_transpose_workspace(d, h), workspace, W2.device)
    check("fp8_cast_transpose_w2", L.fp8_cast_transpose_w2(
        _p(W2), d, h, _p(W2t_q), _p(scale_out), _p(inv_scale_out), _p(amax_out), _p(ws), wsb,
        _stream(stream)))


def amax_reduce(x, amax_out, workspace=None, stream=None):
    """amax_out = max |x| for an fp32 or bf16 tensor."""
    if x.dtype == torch.float32:
        dt = F32
    elif x.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise ValueError("amax_reduce takes float32 or bfloat16")
    n = x.numel()
    L = lib()
    ws, wsb = _ws(L.amax_reduce_workspace(n), workspace, x.device)
    check("amax_reduce", L.amax_reduce(dt, _p(x) if n else None, n, _p(amax_out), _p(ws), wsb, _stream(stream)))


def fp8_scale_from_amax(amax, margin, scale_out=None, inv_scale_out=None, stream=None):
    """scale = 448 / (margin * amax) on the device (1 if not positive finite)."""
    check("fp8_scale_from_amax", lib().fp8_scale_from_amax(
        _p(amax), float(margin), _p(scale_out), _p(inv_scale_out), _stream(stream)))


def fp8_linear(X, x_scale, Wt_q, w_inv_scale, Y, x_amax_out=None, workspace=None, stream=None):
    """Y [M,N] = FP8 linear of X [M,K] bf16 with Wt_q [K,N] e4m3."""
    M, K = X.shape
    N = Wt_q.shape[1]
    L = lib()
    ws, wsb = _ws(L.fp8_linear_workspace(M, K), workspace, X.device)
    check("fp8_linear", L.fp8_linear(
        _p(X), _p(x_scale), _p(Wt_q), _p(w_inv_scale), _p(Y), _p(x_amax_out), M, K, N, _p(ws), wsb,
        _stream(stream)))


def fp8_saturation_count(q, count_out, workspace=None, stream=None):
    """count_out (1-element int64 device tensor) = number of e4m3 codes of
    magnitude 448 in the uint8 tensor q (clip-rate telemetry)."""
    n = q.numel()
    L = lib()
    ws, wsb = _ws(L.fp8_saturation_count_workspace(n), workspace, q.device)
    check("fp8_saturation_count", L.fp8_saturation_count(_p(q) if n else None, n, _p(count_out), _p(ws), wsb,
                                                         _stream(stream)))


def softcap_ce_fwd_bwd(X, W, targets, weights, softcap, loss_out, dX, dW, dloss=None, lse_out=None,
                       accumulate=False, workspace=None, stream=None):
    """Fused softcapped cross-entropy, forward and backward (see
    include/fp8mlp.h).  X [M,d] bf16, W [V,d] bf16, targets [M,T] int32
    (device), weights [T] fp32 (device), softcap a float (0: none),
    loss_out [1] fp32, dX [M,d] bf16, dW [V,d] fp32.  Returns the workspace,
    which begins with the bf16 logit gradient G [M,V]."""
    M, d = X.shape
    V = W.shape[0]
    T = targets.shape[1]
    if targets.dtype != torch.int32:
        raise ValueError("targets must be int32")
    L = lib()
    ws, wsb = _ws(L.softcap_ce_workspace(M, V, d, T), workspace, X.device)
    check("softcap_ce_fwd_bwd", L.softcap_ce_fwd_bwd(
        _p(X), _p(W), _p(targets), T, _p(weights), float(softcap), _p(dloss), _p(loss_out), _p(lse_out), _p(dX),
        _p(dW), int(bool(accumulate)), M, V, d, _p(ws), wsb, _stream(stream)))
    return ws


def softcap_ce_fwd_bwd_fp8(X, x_scale, Wt_q, w_inv_scale, W, targets, weights, softcap, loss_out, dX, dW,
                           dloss=None, lse_out=None, accumulate=False, workspace=None, stream=None):
    """The softcapped cross-entropy with the head in e4m3: Wt_q [d,V] uint8
    (fp8_cast_transpose of W), x_scale / w_inv_scale 1-element fp32 device
    tensors; the rest as softcap_ce_fwd_bwd.  Returns the workspace (it
    begins with G)."""
    M, d = X.shape
    V = W.shape[0]
    T = targets.shape[1]
    if targets.dtype != torch.int32:
        raise ValueError("targets must be int32")
    L = lib()
    ws, wsb = _ws(L.softcap_ce_fp8_workspace(M, V, d, T), workspace, X.device)
    check("softcap_ce_fwd_bwd_fp8", L.softcap_ce_fwd_bwd_fp8(
        _p(X), _p(x_scale), _p(Wt_q), _p(w_inv_scale), _p(W), _p(targets), T, _p(weights), float(softcap), _p(dloss),
        _p(loss_out), _p(lse_out), _p(dX), _p(dW), int(bool(accumulate)), M, V, d, _p(ws), wsb, _stream(stream)))
    return ws


def rmsnorm_fwd(x, xn, inv_rms, eps=1e-6, stream=None):
    """xn = bf16(x * r), r = 1/sqrt(mean(x^2) + eps) per row -> inv_rms [M] fp32."""
    M, d = x.shape
    check("rmsnorm_fwd", lib().rmsnorm_fwd(_p(x), _p(xn), _p(inv_rms), M, d, float(eps), _stream(stream)))


def rmsnorm_bwd(x, inv_rms, dxn, g_in, g_out, stream=None):
    """g_out = bf16(g_in + RMSNorm backward of dxn) per row."""
    M, d = x.shape
    check("rmsnorm_bwd", lib().rmsnorm_bwd(_p(x), _p(inv_rms), _p(dxn), _p(g_in), _p(g_out), M, d,
                                           _stream(stream)))


def add_bf16(a, b, out, stream=None):
    """out = bf16(a + b) elementwise."""
    check("add_bf16", lib().add_bf16(_p(a), _p(b), _p(out), a.numel(), _stream(stream)))


def sgd_update_bf16(W, dW, lr, stream=None):
    """W = bf16(W - fp32(lr * dW)) in place (W bf16, dW fp32)."""
    if W.numel() != dW.numel():
        raise ValueError("W and dW sizes differ")
    check("sgd_update_bf16", lib().sgd_update_bf16(_p(W), _p(dW), W.numel(), float(lr), _stream(stream)))


PROBE_BLOCKS = 256
MFMA_BF16, MFMA_E4M3 = 0, 1


def mfma_probe(dtype, a, b, iters, sink, stream=None):
    """Matrix-core rate probe on operands taken from tensors a and b (see
    fp8mlp_mfma_probe); sink: fp32 [PROBE_BLOCKS * 256].  Returns the flop
    count of the call."""
    if sink.numel() < PROBE_BLOCKS * 256 or sink.dtype != torch.float32:
        raise ValueError("sink must hold PROBE_BLOCKS * 256 fp32 values")
    check("fp8mlp_mfma_probe", lib().fp8mlp_mfma_probe(
        int(dtype), _p(a), a.numel() * a.element_size(), _p(b), b.numel() * b.element_size(), int(iters), _p(sink),
        _stream(stream)))
    return PROBE_BLOCKS * 4 * 16 * int(iters) * (32768 if dtype == MFMA_BF16 else 131072)


class KernelTimer:
    """Context manager around the library's per-kernel timing events.

        with KernelTimer(4096) as kt:
            ...library calls...
        torch.cuda.synchronize()
        kt.records()   # [(kernel name, milliseconds), ...] in launch order
    """

    def __init__(self, capacity=4096):
        self.capacity = capacity
        self.n = 0

    def __enter__(self):
        check("fp8mlp_timing_start", lib().fp8mlp_timing_start(self.capacity))
        return self

    def __exit__(self, *exc):
        self.n = lib().fp8mlp_timing_stop()
        return False

    def records(self):
        import ctypes
        L = lib()
        out = []
        for i in range(self.n):
            name = ctypes.c_char_p()
            ms = ctypes.c_float()
            check("fp8mlp_timing_get", L.fp8mlp_timing_get(i, ctypes.byref(name), ctypes.byref(ms)))
            out.append((name.value.decode(), ms.value))
        return out

    def dropped(self):
        return lib().fp8mlp_timing_dropped()


class Relu2MLP:
    """Device state of one MLP block for delayed-scale FP8 training.

    Holds the bf16 master weights W1 [h,d] and W2 [d,h], the transposed e4m3
    W2 cache W2t_q [h,d] with its scale / inverse scale / amax (refreshed by
    ``refresh_w2_cache`` after every weight update), and the activation amax
    of the previous step (``amax_prev``), which the next forward turns into
    its quantisation scale.  Carrying the state is a buffer swap: the amax a
    forward writes becomes the next forward's ``amax_prev``.

    With ``fp8_up`` the training forward runs the up-projection in e4m3 too
    (mlp_relu2_fwd_fp8up): the block then also keeps the transposed e4m3 W1
    cache W1t_q [d,h] (``refresh_caches`` renews both caches) and the amax of
    its input X from the previous step (``x_amax_prev``), from which each
    forward derives the input's scale with the same margin.

    Scaling policies (the alternatives the delayed-scaling paragraph of "A
    Retrospective on Our World Records" weighs): ``amax_window`` = L > 1
    takes the activation scale from the maximum of the last L measured amaxes
    (a rolling window) instead of amax(t-1) alone; ``w2_scale="delayed"``
    casts W2 with the scale of the previous refresh's max|W2| times
    ``w2_margin`` instead of the exact max|W2| of the weights being cast (the
    first refresh is exact).

    With ``keep_post=False`` the training forward writes only the e4m3 copy
    of post (no bf16 post) and ``backward`` must be given that copy
    (``post_q``); it then runs mlp_relu2_bwd_fp8post with the scale of the
    last forward (``scale_used``), so the backward has to follow its own
    forward before the next one.
    """

    def __init__(self, W1, W2, margin=2.0, amax_init=None, fp8_up=False, x_amax_init=None, amax_window=1,
                 w2_scale="exact", w2_margin=1.0, keep_post=True):
        dev = W1.device
        self.W1, self.W2, self.margin = W1, W2, float(margin)
        h, d = W1.shape
        self.d, self.h = d, h
        f = lambda: torch.zeros(1, dtype=torch.float32, device=dev)
        if int(amax_window) < 1:
            raise ValueError("amax_window must be >= 1")
        if w2_scale not in ("exact", "delayed"):
            raise ValueError("w2_scale is 'exact' or 'delayed'")
        self.amax_window, self.w2_policy, self.w2_margin = int(amax_window), w2_scale, float(w2_margin)
        self.keep_post = bool(keep_post)
        # rolling window: the last L measured amaxes, written in turn
        self.amax_hist = torch.zeros(self.amax_window, dtype=torch.float32, device=dev)
        self._hist_pos = 0
        self.amax_last_measured = None
        self.w2_scale, self.w2_inv_scale, self.w2_amax = f(), f(), f()
        self._w2_amax_next, self._w2_scale_in = f(), f()
        self._w2_refreshed = False
        self.W2t_q = torch.empty((h, d), dtype=torch.uint8, device=dev)
        self.amax_prev, self._amax_next, self.scale_used = f(), f(), f()
        if amax_init is not None:
            self.amax_prev.fill_(float(amax_init))
        self.amax_last_measured = self.amax_prev
        self.fp8_up = bool(fp8_up)
        if self.fp8_up:
            self.w1_scale, self.w1_inv_scale, self.w1_amax = f(), f(), f()
            self.W1t_q = torch.empty((d, h), dtype=torch.uint8, device=dev)
            self.x_amax_prev, self._x_amax_next, self.x_scale = f(), f(), f()
            if x_amax_init is not None:
                self.x_amax_prev.fill_(float(x_amax_init))
        self.refresh_caches()

    # the device tensors whose values carry a block from one step to the next
    _STATE = ("W1", "W2", "W2t_q", "w2_scale", "w2_inv_scale", "w2_amax", "amax_prev", "scale_used",
              "amax_hist")
    _STATE_FP8UP = ("W1t_q", "w1_scale", "w1_inv_scale", "w1_amax", "x_amax_prev", "x_scale")

    def state_dict(self):
        """The block's step-to-step state as CPU tensors (weights, weight
        caches with their scales, the delayed-scale amaxes and the window
        position), for a checkpoint; ``load_state_dict`` restores it so that
        the following steps give the same bits as an uninterrupted run."""
        names = self._STATE + (self._STATE_FP8UP if self.fp8_up else ())
        sd = {k: getattr(self, k).detach().cpu().clone() for k in names}
        sd["hist_pos"] = torch.tensor(self._hist_pos)
        sd["w2_refreshed"] = torch.tensor(int(self._w2_refreshed))
        sd["last_is_hist"] = torch.tensor(int(self.amax_window > 1))
        return sd

    def load_state_dict(self, sd):
        """Copy a ``state_dict`` into this block's device buffers (same shapes,
        same options)."""
        names = self._STATE + (self._STATE_FP8UP if self.fp8_up else ())
        for k in names:
            t = getattr(self, k)
            if tuple(sd[k].shape) != tuple(t.shape) or sd[k].dtype != t.dtype:
                raise ValueError(f"state {k}: {tuple(sd[k].shape)} {sd[k].dtype} does not fit {tuple(t.shape)} {t.dtype}")
            t.copy_(sd[k])
        self._hist_pos = int(sd["hist_pos"])
        self._w2_refreshed = bool(int(sd["w2_refreshed"]))
        if self.amax_window > 1:
            # the amax last measured sits in the slot before the next write
            p = (self._hist_pos - 1) % self.amax_window
            self.amax_last_measured = self.amax_hist[p:p + 1]
        else:
            self.amax_last_measured = self.amax_prev

    def refresh_w2_cache(self, workspace=None, stream=None):
        if self.w2_policy == "exact" or not self._w2_refreshed:
            fp8_cast_transpose_w2(self.W2, self.W2t_q, self.w2_scale, self.w2_inv_scale, self.w2_amax,
                                  workspace=workspace, stream=stream)
        else:
            # delayed: the scale comes from the previous refresh's max|W2|
            fp8_scale_from_amax(self.w2_amax, self.w2_margin, self._w2_scale_in, stream=stream)
            fp8_cast_transpose(self.W2, self.W2t_q, self._w2_scale_in, self.w2_scale, self.w2_inv_scale,
                               self._w2_amax_next, workspace=workspace, stream=stream)
            self.w2_amax, self._w2_amax_next = self._w2_amax_next, self.w2_amax
        self._w2_refreshed = True

    def refresh_caches(self, workspace=None, stream=None):
        """Renew the e4m3 weight caches after an update of W2 (and of W1 with fp8_up)."""
        self.refresh_w2_cache(workspace=workspace, stream=stream)
        if self.fp8_up:
            fp8_cast_transpose(self.W1, self.W1t_q, None, self.w1_scale, self.w1_inv_scale, self.w1_amax,
                               workspace=workspace, stream=stream)

    def forward(self, X, mode=TRAIN_FP8, post=None, post_q=None, Y=None, carry=True, workspace=None, stream=None):
        """Returns (Y, post, post_q).  With carry, the amax measured here
        becomes amax_prev for the next call (and, with fp8_up, max |X| becomes
        x_amax_prev)."""
        M = X.shape[0]
        dev = X.device
        if mode == TRAIN_FP8 and not self.keep_post:
            post = None
        elif post is None:
            post = torch.empty((M, self.h), dtype=torch.bfloat16, device=dev)
        if mode == TRAIN_FP8 and post_q is None:
            post_q = torch.empty((M, self.h), dtype=torch.uint8, device=dev)
        Y = torch.empty((M, self.d), dtype=torch.bfloat16, device=dev) if Y is None else Y
        # with a window the measured amax lands in the next slot of the history
        windowed = carry and self.amax_window > 1
        amax_out = self.amax_hist[self._hist_pos:self._hist_pos + 1] if windowed else self._amax_next
        if mode == TRAIN_FP8 and self.fp8_up:
            fp8_scale_from_amax(self.x_amax_prev, self.margin, self.x_scale, stream=stream)
            mlp_relu2_fwd_fp8up(X, self.x_scale, self.W1t_q, self.w1_inv_scale, self.W2t_q, self.w2_inv_scale,
                                self.amax_prev, self.margin, post, post_q, amax_out, self.scale_used, Y,
                                x_amax_out=self._x_amax_next, workspace=workspace, stream=stream)
            if carry:
                self.x_amax_prev, self._x_amax_next = self._x_amax_next, self.x_amax_prev
        else:
            mlp_relu2_fwd(mode, X, self.W1, self.W2t_q, self.w2_inv_scale, self.W2, self.amax_prev, self.margin,
                          post, post_q if mode == TRAIN_FP8 else None, amax_out,
                          self.scale_used if mode == TRAIN_FP8 else None, Y, workspace=workspace, stream=stream)
        if windowed:
            self.amax_last_measured = amax_out
            self._hist_pos = (self._hist_pos + 1) % self.amax_window
            amax_reduce(self.amax_hist, self.amax_prev, stream=stream)
        elif carry:
            self.amax_prev, self._amax_next = self._amax_next, self.amax_prev
        return Y, post, post_q

    @property
    def amax_last(self):
        """The amax measured by the most recent carried forward."""
        return self.amax_last_measured if self.amax_window > 1 else self.amax_prev

    def backward(self, dY, X, post, dX=None, dW1=None, dW2=None, accumulate=False, workspace=None, stream=None,
                 post_q=None, post_scale=None):
        """From the bf16 post, or (post None) from the e4m3 copy post_q and
        the scale its forward used (default: this block's last scale)."""
        dev = X.device
        dX = torch.empty_like(X) if dX is None else dX
        dW1 = torch.empty((self.h, self.d), dtype=torch.float32, device=dev) if dW1 is None else dW1
        dW2 = torch.empty((self.d, self.h), dtype=torch.float32, device=dev) if dW2 is None else dW2
        if post is not None:
            mlp_relu2_bwd(dY, X, self.W1, self.W2, post, dX, dW1, dW2, accumulate, workspace=workspace,
                          stream=stream)
        else:
            if post_q is None:
                raise ValueError("backward needs post or post_q")
            mlp_relu2_bwd_fp8post(dY, X, self.W1, self.W2, post_q, self.scale_used if post_scale is None else post_scale,
                                  dX, dW1, dW2, accumulate, workspace=workspace, stream=stream)
        return dX, dW1, dW2
