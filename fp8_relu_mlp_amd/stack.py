"""A stack of FP8 ReLU^2 MLP blocks trained step by step, each layer carrying
its own delayed-scale state.

The speedrun pages run the MLP block inside a pre-norm transformer: the FP8
scale of a layer at step t comes from that layer's amax at step t-1 times a
safety margin, and the transposed FP8 copy of W2 is refreshed after every
optimizer update ("A Retrospective on Our World Records", Main Track: the
delayed-scaling and W2-cache paragraphs).  ``Relu2Stack`` trains

    x_{l+1} = x_l + MLP_l(rmsnorm(x_l)),   l = 0 .. L-1

with plain SGD on every W1 / W2.  The weight gradients of mlp_relu2_bwd are
sums over the M tokens of the batch; with ``loss="mean"`` (the default) the
step is taken on the gradient of the token-mean loss, lr * dW / M, as a
mean-reduced training loss gives, and with ``loss="sum"`` on lr * dW.  The
step multiplier is rounded to fp32 once (``lr_step``).  At the 12-layer,
M=65536 workload with a N(0, 1e-3) top gradient, the summed-gradient step
makes the stack diverge within a few steps.

Every computation is a library call: rmsnorm_fwd, mlp_relu2_fwd, add_bf16 on
the way up; mlp_relu2_bwd,
rmsnorm_bwd (which also adds the residual gradient) on the way down;
sgd_update_bf16 and fp8_cast_transpose_w2 after each layer's backward.
PyTorch only allocates the buffers.

State carry: a layer's forward turns its ``amax_prev`` into the quantisation
scale and writes the amax it measures, which becomes ``amax_prev`` for the
next step (a buffer swap inside ``Relu2MLP``).  The very first step has no
previous amax: each layer first runs one forward to measure the exact amax of
that step and then runs again with it.

Options passed to every block: ``fp8_up`` (both forward GEMMs in e4m3; the
W1 cache is refreshed after each update as well), ``amax_window`` and
``w2_scale`` / ``w2_margin`` (the scaling policies of ``Relu2MLP``).  With
``telemetry`` each layer's forward is followed by fp8_saturation_count on its
e4m3 post copy; ``saturated`` [L] (int64, device) holds the counts of the
last step and ``saturation_rate(l)`` their share of the M*h codes.  With
``keep_post=False`` no layer keeps its bf16 post: each keeps its e4m3 copy,
and the backward runs on it with the scale recorded in ``state``.
"""
import numpy as np
import torch

from . import (TRAIN_FP8, Relu2MLP, add_bf16, fp8_saturation_count, lib,
               rmsnorm_bwd, rmsnorm_fwd, sgd_update_bf16)


class Relu2Stack:
    def __init__(self, W1s, W2s, margin=2.0, lr=1e-3, eps=1e-6, loss="mean", fp8_up=False, amax_window=1,
                 w2_scale="exact", w2_margin=1.0, telemetry=False, keep_post=True):
        if len(W1s) != len(W2s) or not W1s:
            raise ValueError("need the same positive number of W1 and W2 tensors")
        self.layers = [Relu2MLP(w1, w2, margin=margin, amax_init=1.0, fp8_up=fp8_up, amax_window=amax_window,
                                w2_scale=w2_scale, w2_margin=w2_margin, keep_post=keep_post)
                       for w1, w2 in zip(W1s, W2s)]
        self.fp8_up, self.telemetry, self.keep_post = bool(fp8_up), bool(telemetry), bool(keep_post)
        self.L = len(self.layers)
        self.d, self.h = self.layers[0].d, self.layers[0].h
        if loss not in ("mean", "sum"):
            raise ValueError("loss is 'mean' or 'sum'")
        self.lr, self.eps, self.loss = float(lr), float(eps), loss
        self.lr_step = None
        self.steps_done = 0
        self._M = None

    def _alloc(self, M, dev):
        if self._M == M:
            return
        L, d, h = self.L, self.d, self.h
        bf, f32 = torch.bfloat16, torch.float32
        self.x = [torch.empty((M, d), dtype=bf, device=dev) for _ in range(L + 1)]
        self.xn = [torch.empty((M, d), dtype=bf, device=dev) for _ in range(L)]
        self.inv = [torch.empty((M,), dtype=f32, device=dev) for _ in range(L)]
        if self.keep_post:
            self.post = [torch.empty((M, h), dtype=bf, device=dev) for _ in range(L)]
            self.post_q = torch.empty((M, h), dtype=torch.uint8, device=dev)
            self.post_qs = None
        else:
            self.post = [None] * L
            self.post_qs = [torch.empty((M, h), dtype=torch.uint8, device=dev) for _ in range(L)]
            self.post_q = self.post_qs[0]
        self.Y = torch.empty((M, d), dtype=bf, device=dev)
        self.g = torch.empty((M, d), dtype=bf, device=dev)
        self.dxn = torch.empty((M, d), dtype=bf, device=dev)
        self.dW1 = torch.empty((h, d), dtype=f32, device=dev)
        self.dW2 = torch.empty((d, h), dtype=f32, device=dev)
        Lb = lib()
        u8 = torch.uint8
        ws_fwd = Lb.mlp_relu2_fwd_workspace(M, d, h)
        if self.fp8_up:
            ws_fwd = max(ws_fwd, Lb.mlp_relu2_fwd_fp8up_workspace(M, d, h))
        self.ws_f = torch.empty(max(1, ws_fwd), dtype=u8, device=dev)
        self.ws_b = torch.empty(max(1, Lb.mlp_relu2_bwd_workspace(M, d, h)), dtype=u8, device=dev)
        self.ws_c = torch.empty(max(1, Lb.fp8_cast_transpose_workspace(d, h)), dtype=u8, device=dev)
        self.ws_t = torch.empty(max(1, Lb.fp8_saturation_count_workspace(M * h)), dtype=u8, device=dev)
        self.saturated = torch.zeros((self.L,), dtype=torch.int64, device=dev)
        # per step and layer: amax_prev used, scale used, amax measured
        self.state = torch.zeros((self.L, 3), dtype=f32, device=dev)
        self.lr_step = float(np.float32(self.lr / M if self.loss == "mean" else self.lr))
        self._M = M

    def step(self, X, dY_top, observe=None):
        """One training step on the batch X [M, d] (bf16) with the top
        gradient dY_top [M, d] (bf16).  ``observe(layer, phase, stack)``, if
        given, is called after each layer's forward ("fwd"), after its
        backward but before its update ("bwd", with ``stack.g_in`` holding
        the gradient that arrived from above) and after the update and the W2
        refresh ("upd"); it may read the stack's buffers.
        Returns a [L, 3] fp32 device tensor: per layer the amax_prev the
        forward used, the scale it used and the amax it measured."""
        M, d = X.shape
        self._alloc(M, X.device)
        self.x[0].copy_(X)
        for l, blk in enumerate(self.layers):
            if not self.keep_post:
                self.post_q = self.post_qs[l]
            rmsnorm_fwd(self.x[l], self.xn[l], self.inv[l], self.eps)
            if self.steps_done == 0:
                blk.forward(self.xn[l], post=self.post[l], post_q=self.post_q, Y=self.Y, workspace=self.ws_f)
            self.state[l, 0].copy_(blk.amax_prev[0])
            blk.forward(self.xn[l], mode=TRAIN_FP8, post=self.post[l], post_q=self.post_q, Y=self.Y,
                        workspace=self.ws_f)
            self.state[l, 1].copy_(blk.scale_used[0])
            self.state[l, 2].copy_(blk.amax_last[0])
            if self.telemetry:
                fp8_saturation_count(self.post_q, self.saturated[l:l + 1], workspace=self.ws_t)
            add_bf16(self.x[l], self.Y, self.x[l + 1])
            if observe:
                observe(l, "fwd", self)
        self.g.copy_(dY_top)
        for l in range(self.L - 1, -1, -1):
            blk = self.layers[l]
            if observe:
                self.g_in = self.g.clone()
            if self.keep_post:
                blk.backward(self.g, self.xn[l], self.post[l], self.dxn, self.dW1, self.dW2, workspace=self.ws_b)
            else:
                blk.backward(self.g, self.xn[l], None, self.dxn, self.dW1, self.dW2, workspace=self.ws_b,
                             post_q=self.post_qs[l], post_scale=self.state[l, 1:2])
            rmsnorm_bwd(self.x[l], self.inv[l], self.dxn, self.g, self.g)
            if observe:
                observe(l, "bwd", self)
            sgd_update_bf16(blk.W1, self.dW1, self.lr_step)
            sgd_update_bf16(blk.W2, self.dW2, self.lr_step)
            blk.refresh_caches(workspace=self.ws_c)
            if observe:
                observe(l, "upd", self)
        self.steps_done += 1
        return self.state

    def state_dict(self):
        """Checkpoint of the training state: every layer's ``Relu2MLP`` state
        (weights, weight caches, delayed-scale amaxes) and the step count,
        as CPU tensors.  Restored into a stack built with the same options,
        the following steps reproduce an uninterrupted run bit for bit."""
        sd = {"steps_done": torch.tensor(self.steps_done)}
        for l, blk in enumerate(self.layers):
            for k, v in blk.state_dict().items():
                sd[f"layer{l}.{k}"] = v
        return sd

    def load_state_dict(self, sd):
        for l, blk in enumerate(self.layers):
            pre = f"layer{l}."
            blk.load_state_dict({k[len(pre):]: v for k, v in sd.items() if k.startswith(pre)})
        self.steps_done = int(sd["steps_done"])

    def saturation_rate(self, l):
        """Share of layer l's e4m3 post codes at the top code (448) in the
        last step (needs telemetry=True)."""
        return float(self.saturated[l].item()) / float(self._M * self.h)
