"""Seeded synthetic inputs for the MLP path (shared by tests, smoke and bench).

This module only draws random numbers and stores them as bf16 bit patterns.
It holds none of the method's arithmetic, imports nothing from the library
binding and nothing from the CPU oracle, so both sides can be fed the very
same bits.

Stand-in workload: the speedrun pages train a GPT-2-small tier model
(model width 768, ReLU^2 MLP with hidden width 4*768) on FineWeb tokens.  No
dataset is used here; activations are drawn as post-RMSNorm-like N(0, 1) rows
and weights with fan-in variance, the shapes of that model's MLP block and
attention projections.  N(mu, v) always names the variance v.

Every tensor has its own stream: ``numpy.random.default_rng`` seeded with
(seed, crc32(name)), so adding a tensor never shifts another one's values.
Draws are float64, rounded to fp32 by numpy and to bf16 by torch's CPU cast
(round-to-nearest-even); the resulting bit patterns are the inputs.
"""
import zlib

import numpy as np
import torch

WORKLOADS = {
    # name: (M, d, h, seed)
    "tiny": (256, 128, 512, 0),           # one forward step, exact amax as amax_prev
    "fwd2": (16384, 768, 3072, 1),        # two forward steps, delayed scale
    "fwdbwd": (49152, 768, 3072, 2),      # forward + backward, the timed workload
    "stack": (65536, 768, 3072, 4),       # 12 layers x 8 steps with state carry
}
STACK = {"layers": 12, "steps": 8, "lr": 1e-3}
ATTN = {"M": 49152, "d": 768, "qkv": 2304, "seed": 3}


def rng(seed, name):
    return np.random.default_rng([int(seed), zlib.crc32(name.encode())])


def to_bf16_bits(x):
    """float array -> uint16 bf16 bit patterns via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shape, var, seed, name):
    """bf16 bits of N(0, var) draws for one named tensor."""
    g = rng(seed, name)
    x = g.standard_normal(size=shape) * np.sqrt(var)
    return to_bf16_bits(x)


def ternary_bf16(shape, seed, name, nnz_per_row=None):
    """bf16 bits of values in {-1, 0, +1}; with nnz_per_row, each row has at
    most that many non-zeros (used for the lossless special case)."""
    g = rng(seed, name)
    if nnz_per_row is None:
        x = g.integers(-1, 2, size=shape).astype(np.float64)
    else:
        x = np.zeros(shape)
        for r in range(shape[0]):
            cols = g.choice(shape[1], size=nnz_per_row, replace=False)
            x[r, cols] = g.choice([-1.0, 1.0], size=nnz_per_row)
    return to_bf16_bits(x)


def mlp_inputs(M, d, h, seed, with_dy=False, step=0):
    """X [M,d] ~ N(0,1); W1 [h,d] ~ N(0,1/d); W2 [d,h] ~ N(0,1/h);
    dY [M,d] ~ N(0,1e-3) when requested.  ``step`` selects a fresh X/dY."""
    out = {
        "X": normal_bf16((M, d), 1.0, seed, f"X.{step}"),
        "W1": normal_bf16((h, d), 1.0 / d, seed, "W1"),
        "W2": normal_bf16((d, h), 1.0 / h, seed, "W2"),
    }
    if with_dy:
        out["dY"] = normal_bf16((M, d), 1e-3, seed, f"dY.{step}")
    return out


def normal_f32_rows(shape, seed, name, blocks=16):
    """float32 N(0, 1) draws for tensors of millions of rows, fast: the rows
    split into ``blocks`` runs of equal length (the last one shorter), each
    drawn in float32 from its own stream seeded with (seed, crc32(name),
    block) on up to 8 threads.  The values do not depend on the threads."""
    from concurrent.futures import ThreadPoolExecutor
    rows = shape[0]
    out = np.empty(shape, dtype=np.float32)
    per = -(-rows // blocks)

    def fill(b):
        g = np.random.default_rng([int(seed), zlib.crc32(name.encode()), b])
        part = out[b * per:(b + 1) * per]
        if part.size:
            g.standard_normal(out=part, dtype=np.float32)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(fill, range(blocks)))
    return out


def normal_bf16_rows(shape, var, seed, name):
    """bf16 bits of N(0, var) from ``normal_f32_rows`` (scaled in float32)."""
    x = normal_f32_rows(shape, seed, name)
    x *= np.float32(np.sqrt(var))
    return to_bf16_bits(x)


def abs_normal_bf16_rows(shape, seed, name):
    """bf16 bits of |N(0, 1)| from ``normal_f32_rows``: a non-negative stand-in
    for the stored activation when the backward is tested on its own."""
    x = normal_f32_rows(shape, seed, name)
    np.abs(x, out=x)
    return to_bf16_bits(x)


def perturbed_w1(W1_bits, seed):
    """Step-2 weights of the two-step forward workload: W1 + 1e-3 * N(0, 1/d),
    added in fp32 and rounded back to bf16 (a new input, not part of the path)."""
    h, d = W1_bits.shape
    g = rng(seed, "W1.delta")
    delta = (1e-3 * g.standard_normal(size=(h, d)) * np.sqrt(1.0 / d)).astype(np.float32)
    w = torch.from_numpy(W1_bits.view(np.int16).copy()).view(torch.bfloat16).float()
    w = w + torch.from_numpy(delta)
    return w.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def stack_weights(L, d, h, seed):
    """Per-layer weights of the layer-stack workload: W1 [h,d] ~ N(0,1/d),
    W2 [d,h] ~ N(0,1/h), one named stream per layer and matrix."""
    return [(normal_bf16((h, d), 1.0 / d, seed, f"W1.{l}"), normal_bf16((d, h), 1.0 / h, seed, f"W2.{l}"))
            for l in range(L)]


def stack_batch(M, d, seed, step):
    """Batch of one step of the layer-stack workload: X [M,d] ~ N(0,1) and
    the top gradient dY [M,d] ~ N(0,1e-3)."""
    return {"X": normal_bf16((M, d), 1.0, seed, f"stack.X.{step}"),
            "dY": normal_bf16((M, d), 1e-3, seed, f"stack.dY.{step}")}


def attn_inputs(M=None, d=None, qkv=None, seed=None):
    """FP8 attention projection workload: X [M,d] ~ N(0,1), Wqkv [qkv,d] and
    Wo [d,d] ~ N(0,1/d), O-projection input Xo [M,d] ~ N(0,0.5)."""
    M = ATTN["M"] if M is None else M
    d = ATTN["d"] if d is None else d
    qkv = ATTN["qkv"] if qkv is None else qkv
    seed = ATTN["seed"] if seed is None else seed
    return {
        "X": normal_bf16((M, d), 1.0, seed, "X"),
        "Wqkv": normal_bf16((qkv, d), 1.0 / d, seed, "Wqkv"),
        "Xo": normal_bf16((M, d), 0.5, seed, "Xo"),
        "Wo": normal_bf16((d, d), 1.0 / d, seed, "Wo"),
    }


# Language-model head workload of the fused softcapped cross-entropy:
# GPT-2-small shapes, the GPT-2 vocabulary padded to a multiple of 64, three
# successive targets per position, sequences of 1024 tokens.
CE = {"M": 49152, "d": 768, "V": 50304, "T": 3, "seq": 1024, "softcap": 15.0,
      "weights": (1.0, 0.5, 0.25), "head_var": 4.0, "seed": 5}


def ce_inputs(M, d, V, T, seed, seq=None, head_var=None, vocab_used=None):
    """X [M,d] ~ N(0,1) (the final normalised hidden states), W [V,d] ~
    N(0, head_var/d) (default 4/d: logits of standard deviation about 2), and
    targets [M,T] int64: target j of position m is token m+1+j of a uniform
    random token stream cut into sequences of `seq` positions (-1 past a
    sequence's end).  `vocab_used` (default: V, or 50257 when V = 50304)
    bounds the token ids, as a padded vocabulary leaves its tail unused."""
    seq = M if seq is None else seq
    hv = CE["head_var"] if head_var is None else head_var
    if vocab_used is None:
        vocab_used = 50257 if V == 50304 else V
    g = rng(seed, "ce.tokens")
    tok = g.integers(0, vocab_used, size=M + T + 1)
    t = np.full((M, T), -1, dtype=np.int64)
    pos = np.arange(M) % seq
    for j in range(T):
        ok = pos + 1 + j < seq
        t[ok, j] = tok[np.arange(M)[ok] + 1 + j]
    return {"X": normal_bf16((M, d), 1.0, seed, "ce.X"), "W": normal_bf16((V, d), hv / d, seed, "ce.W"),
            "targets": t}
