"""GPU parity of softcap_ce_fwd_bwd (fused softcapped cross-entropy over a
language-model head) against the CPU oracle.

Gates (element by element on the same seeded inputs):
  * loss and every row's lse within a bound derived from the arithmetic:
    the logits carry the fp32 accumulation error (d + 2) 2^-24 sum|x w| of
    their row plus the softcap's few ulps of c; a row's sum of exponentials
    is formed from per-lane runs of 32, the lane pair, four waves and then
    the column tiles in order, so its relative error is at most
    (48 + tiles) 2^-24, plus the exp / log rounding (2^-22 and 2^-23 |lse|);
  * G (the bf16 logit gradient) within 1e-2 relative Frobenius error of the
    oracle's (the bf16-path gate);
  * dX within 4e-3 and dW within 1e-4 of the oracle fed the GPU's own G (one
    bf16 rounding of dX; fp32 accumulation only for dW);
  * no-softcap, missing and out-of-range targets, accumulation, M = 0;
  * the FP8 head (softcap_ce_fwd_bwd_fp8): the transposed e4m3 W cache
    bit-exact, the logits' error bounded by the e4m3 matrix core's alignment
    window (``acc_bound`` of the FP8 up-projection tests) and the two fp32
    dequantisation products, the rest as above.
"""
import numpy as np
import pytest
import torch

from fp8_relu_mlp_amd import synth
from oracle import ce as C
from oracle import formats as F

from .gpu_helpers import DEV, bf16_dev, bits, case, rel_fro

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def fm():
    import fp8_relu_mlp_amd as fm
    fm.lib()
    return fm


def run(fm, ins, weights, c, dloss=None, accumulate=False, dW_init=None):
    X, W = bf16_dev(ins["X"]), bf16_dev(ins["W"])
    M, d = ins["X"].shape
    V = ins["W"].shape[0]
    t = torch.from_numpy(ins["targets"].astype(np.int32)).to(DEV)
    w = torch.tensor(weights, dtype=torch.float32, device=DEV)
    loss, lse = torch.full((1,), -1.0, device=DEV), torch.full((max(M, 1),), -1.0, device=DEV)
    dX = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    dW = (torch.full((V, d), 3.0, device=DEV) if dW_init is None else torch.from_numpy(dW_init).to(DEV))
    dl = None if dloss is None else torch.tensor([dloss], dtype=torch.float32, device=DEV)
    ws = fm.softcap_ce_fwd_bwd(X, W, t, w, c, loss, dX, dW, dloss=dl, lse_out=lse[:M] if M else None,
                               accumulate=accumulate)
    torch.cuda.synchronize()
    G = None if M == 0 else bits(ws[:M * V * 2].view(torch.bfloat16).view(M, V))
    return {"loss": float(loss.item()), "lse": lse[:M].cpu().numpy().astype(np.float64), "G": G,
            "dX": F.bf16_to_f64(bits(dX)) if M else None, "dW": dW.cpu().numpy().astype(np.float64)}


def z_error(ins, c):
    """Per-row bound on |z'_gpu - z'| (fp32 accumulation and the softcap)."""
    X, W = F.bf16_to_f64(ins["X"]), F.bf16_to_f64(ins["W"])
    d = X.shape[1]
    S = (np.abs(X) @ np.abs(W).T).max(axis=1)
    return (d + 2) * U * S * 1.01 + 16 * U * (c if c else 0.0) + 4 * U * np.abs(X @ W.T).max(axis=1)


def check(ins, g, weights, c, dloss=1.0, dW_add=None):
    cc = c if c else float("inf")
    ref = C.softcap_ce(ins["X"], ins["W"], ins["targets"], weights, cc, dloss=dloss)
    M, V = ins["targets"].shape[0], ins["W"].shape[0]
    tiles = -(-V // 256)
    ez = z_error(ins, c)
    e_lse = ez + (48 + tiles) * U + 2.0 ** -22 + 2.0 ** -23 * np.abs(ref["lse"])
    assert (np.abs(g["lse"] - ref["lse"]) <= e_lse).all()
    t = ins["targets"]
    valid = (t >= 0) & (t < V)
    wsum = np.where(valid, np.asarray(weights)[None, :], 0.0).sum(axis=1)
    eloss = (wsum * (e_lse + ez)).sum() / M + (256 + M / 256 + 8) * U * np.abs(ref["per_row"]).sum() / M
    assert abs(g["loss"] - ref["loss"]) <= eloss, (g["loss"], ref["loss"], eloss)
    Gg = F.bf16_to_f64(g["G"])
    assert rel_fro(Gg, ref["G"]) < 1e-2
    Wf, Xf = F.bf16_to_f64(ins["W"]), F.bf16_to_f64(ins["X"])
    assert rel_fro(g["dX"], Gg @ Wf) < 4e-3
    dW = Gg.T @ Xf + (0.0 if dW_add is None else dW_add)
    assert rel_fro(g["dW"], dW) < 1e-4
    return ref


def test_ce_small(fm):
    case("ce small M=300 d=128 V=1024 T=3")
    ins = synth.ce_inputs(300, 128, 1024, 3, 80, seq=128)
    w = [1.0, 0.5, 0.25]
    check(ins, run(fm, ins, w, 15.0), w, 15.0)


@pytest.mark.parametrize("M,d,V,T,c", [(1, 64, 64, 1, 15.0), (255, 128, 832, 3, 15.0), (300, 192, 1024, 2, 5.0),
                                       (777, 768, 4096, 3, 30.0)])
def test_ce_ragged_shapes(fm, M, d, V, T, c):
    case(f"ce ragged M={M} d={d} V={V} T={T} c={c}")
    ins = synth.ce_inputs(M, d, V, T, 81 + M, seq=100, head_var=16.0)
    w = [1.0, 0.5, 0.25][:T]
    check(ins, run(fm, ins, w, c), w, c)


def test_ce_no_softcap_and_dloss(fm):
    case("ce without softcap, dloss 0.5")
    ins = synth.ce_inputs(256, 128, 512, 1, 82)
    check(ins, run(fm, ins, [1.0], 0.0, dloss=0.5), [1.0], 0.0, dloss=0.5)


def test_ce_missing_and_out_of_range_targets(fm):
    case("ce missing / out-of-range targets")
    ins = synth.ce_inputs(256, 128, 512, 2, 83)
    t = ins["targets"]
    t[::7, 0] = -1
    t[::5, 1] = 512 + 3          # >= V: no target, on both sides
    ref_t = np.where(t >= 512, -1, t)
    g = run(fm, ins, [0.7, 0.3], 15.0)
    check(dict(ins, targets=ref_t), g, [0.7, 0.3], 15.0)


def test_ce_duplicate_targets(fm):
    # Rows whose successive targets repeat a token: the gradient at that
    # column carries the sum of their weights.  Checked entry by entry at
    # every target column (a bf16 value, so within a few bf16 ulps of the
    # fp64 oracle), and as a whole by check().
    case("ce duplicate targets")
    ins = synth.ce_inputs(256, 128, 512, 3, 84)
    t = ins["targets"]
    t[::3, 1] = t[::3, 0]
    t[1::4, 2] = t[1::4, 0]
    t[2::5, 2] = t[2::5, 1]
    w = [1.0, 0.5, 0.25]
    g = run(fm, ins, w, 15.0)
    ref = check(ins, g, w, 15.0)
    Gg = F.bf16_to_f64(g["G"])
    rows = np.repeat(np.arange(t.shape[0]), t.shape[1])
    cols = t.reshape(-1)
    ok = cols >= 0
    a, b = Gg[rows[ok], cols[ok]], ref["G"][rows[ok], cols[ok]]
    assert (np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-9).all(), np.abs(a - b).max()


def test_ce_accumulate(fm):
    case("ce accumulate")
    ins = synth.ce_inputs(384, 128, 512, 2, 84)
    init = np.random.default_rng(84).standard_normal((512, 128)).astype(np.float32)
    g = run(fm, ins, [1.0, 0.5], 15.0, accumulate=True, dW_init=init)
    check(ins, g, [1.0, 0.5], 15.0, dW_add=init.astype(np.float64))


def test_ce_empty(fm):
    case("ce M=0")
    ins = synth.ce_inputs(0, 128, 256, 2, 85)
    g = run(fm, ins, [1.0, 0.5], 15.0)
    assert g["loss"] == 0.0 and (g["dW"] == 0).all()


# ------------------------------------------------------------------ FP8 head
def run_fp8(fm, ins, weights, c):
    from oracle import mlp as O
    X, W = bf16_dev(ins["X"]), bf16_dev(ins["W"])
    M, d = ins["X"].shape
    V = ins["W"].shape[0]
    Wt = torch.empty((d, V), dtype=torch.uint8, device=DEV)
    inv = torch.zeros(1, dtype=torch.float32, device=DEV)
    fm.fp8_cast_transpose(W, Wt, inv_scale_out=inv)
    sx = O.exact_scale(O.amax(F.bf16_to_f64(ins["X"])))
    t = torch.from_numpy(ins["targets"].astype(np.int32)).to(DEV)
    w = torch.tensor(weights, dtype=torch.float32, device=DEV)
    loss, lse = torch.zeros(1, device=DEV), torch.zeros(M, device=DEV)
    dX = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    dW = torch.empty((V, d), dtype=torch.float32, device=DEV)
    ws = fm.softcap_ce_fwd_bwd_fp8(X, torch.tensor([sx], dtype=torch.float32, device=DEV), Wt, inv, W, t, w, c,
                                   loss, dX, dW, lse_out=lse)
    torch.cuda.synchronize()
    return {"loss": float(loss.item()), "lse": lse.cpu().numpy().astype(np.float64),
            "G": bits(ws[:M * V * 2].view(torch.bfloat16).view(M, V)), "dX": F.bf16_to_f64(bits(dX)),
            "dW": dW.cpu().numpy().astype(np.float64), "Wt": Wt.cpu().numpy(), "inv": float(inv.item()), "sx": sx}


def check_fp8(ins, g, weights, c):
    from oracle import mlp as O
    from .test_gpu_fp8up import acc_bound
    Wt, _, inv, _ = O.cast_transpose(ins["W"])
    assert (Wt == g["Wt"]).all() and inv == g["inv"]
    Z = C.fp8_logits(ins["X"], g["sx"], Wt, inv)
    ref = C.softcap_ce(ins["X"], ins["W"], ins["targets"], weights, c if c else float("inf"), Z=Z)
    X = F.bf16_to_f64(ins["X"])
    xq = F.e4m3_decode(F.e4m3_encode(F.fl32(X * g["sx"])))
    a = O.inv_scale(g["sx"]) * inv
    ez = ((acc_bound(xq, F.e4m3_decode(Wt)) * a).max(axis=1) * 1.001 + 4 * U * np.abs(Z).max(axis=1)
          + 16 * U * (c if c else 0.0))
    V = ins["W"].shape[0]
    tiles = -(-V // 256)
    e_lse = ez + (48 + tiles) * U + 2.0 ** -22 + 2.0 ** -23 * np.abs(ref["lse"])
    assert (np.abs(g["lse"] - ref["lse"]) <= e_lse).all()
    t = ins["targets"]
    valid = (t >= 0) & (t < V)
    M = t.shape[0]
    wsum = np.where(valid, np.asarray(weights)[None, :], 0.0).sum(axis=1)
    eloss = (wsum * (e_lse + ez)).sum() / M + (256 + M / 256 + 8) * U * np.abs(ref["per_row"]).sum() / M
    assert abs(g["loss"] - ref["loss"]) <= eloss, (g["loss"], ref["loss"], eloss)
    Gg = F.bf16_to_f64(g["G"])
    assert rel_fro(Gg, ref["G"]) < 1e-2
    assert rel_fro(g["dX"], Gg @ F.bf16_to_f64(ins["W"])) < 4e-3
    assert rel_fro(g["dW"], Gg.T @ X) < 1e-4


@pytest.mark.parametrize("M,d,V,T,c", [(300, 128, 1024, 3, 15.0), (257, 256, 832, 2, 5.0), (777, 768, 4096, 3, 30.0),
                                       (64, 128, 256, 1, 0.0)])
def test_ce_fp8_head(fm, M, d, V, T, c):
    case(f"ce fp8 head M={M} d={d} V={V} T={T} c={c}")
    ins = synth.ce_inputs(M, d, V, T, 90 + M, seq=100, head_var=16.0)
    w = [1.0, 0.5, 0.25][:T]
    check_fp8(ins, run_fp8(fm, ins, w, c), w, c)
