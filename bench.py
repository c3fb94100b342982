#!/usr/bin/env python3
"""Benchmark of the fused FP8 ReLU^2 MLP block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one training pass of the MLP block over one batch of synthetic
GPT-2-small-shaped tokens (M=49152, d=768, h=3072, margin 2):
  mlp_relu2_fwd (TRAIN: up-projection + ReLU^2 + e4m3 quantisation with the
  delayed scale + partial amax, amax reduction, e4m3 down-projection),
  mlp_relu2_bwd (dgrad with sqrt(post), dX, dW1, dW2),
  fp8_cast_transpose_w2 (the W2 cache refresh that follows each update),
with the measured amax carried to the next step as its amax_prev.
Inputs are resident in HBM before timing starts; the matrix-core probe
(~20 ms of MFMA work on the workload's operands) runs first, then W warm-up
steps that are not timed; K steps are timed with HIP events between two
device synchronisations.

value = 12*M*d*h / t_step in TFLOP/s (the six GEMMs of forward + backward).
One JSON line goes to stdout; progress goes to stderr.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

M, D, H = 49152, 768, 3072
MARGIN = 2.0
PEAK_BF16 = 2500.0    # TFLOP/s, MI355X dense bf16 MFMA (published)
PEAK_FP8 = 5000.0     # TFLOP/s, MI355X dense fp8 MFMA (published)
PEAK_HBM = 8000.0     # GB/s
METRIC = "MLP fwd+bwd TFLOP/s and % of MFMA peak, M=49152 d=768 h=3072, 1 GPU"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "hbm_traffic_mlp_fwd_bwd_M49152.txt")
# GEMM kernels carry the launch site as their last template argument
KID_NAMES = {1: "up_gemm_relu2_quant", 2: "down_gemm_e4m3", 3: "down_gemm_bf16_eval", 4: "dpost_gemm_dpre",
             5: "dx_gemm", 6: "dw1_gemm", 7: "dw2_gemm", 8: "fp8_linear_gemm", 9: "up_gemm_e4m3_relu2_quant",
             10: "ce_head_gemm_stats", 11: "ce_head_gemm_grad", 12: "ce_dx_gemm", 13: "ce_dw_gemm",
             14: "ce_head_gemm_e4m3_stats", 15: "ce_head_gemm_e4m3_grad", 16: "dw_gemm"}
OTHER_NAMES = {"k_max_final": "amax_final", "k_amax_partial": "amax_partial", "k_cast_transpose": "cast_transpose",
               "k_splitk_reduce": "splitk_reduce", "k_splitk_reduce_tiles": "splitk_reduce", "k_quantize": "quantize_e4m3",
               "k_lin_panel": "fp8_linear_panel", "k_fill_zero": "fill_zero",
               "k_zero_scalar": "zero_scalar", "k_scale_from_amax": "scale_from_amax", "k_amax_small": "amax_small",
               "k_transpose_weights": "transpose_weights", "k_rmsnorm_fwd": "rmsnorm_fwd", "k_rmsnorm_bwd": "rmsnorm_bwd",
               "k_add_bf16": "add_bf16", "k_sgd_bf16": "sgd_update_bf16", "k_mfma_probe": "mfma_probe",
               "k_count_top": "count_top_codes", "k_sum_counts": "sum_counts", "k_ce_rows": "ce_rows",
               "k_ce_loss": "ce_loss"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# algorithmic work per launch of each kernel at (M, d, h): (flops, bytes, dtype peak)
def kernel_work(M, d, h):
    b16, b8, f32 = 2, 1, 4
    mdh2 = 2.0 * M * d * h
    return {
        "up_gemm_relu2_quant": (mdh2, M * d * b16 + h * d * b16 + M * h * (b16 + b8), PEAK_BF16),
        "down_gemm_e4m3": (mdh2, M * h * b8 + h * d * b8 + M * d * b16, PEAK_FP8),
        "dpost_gemm_dpre": (mdh2, M * d * b16 + d * h * b16 + 2 * M * h * b16, PEAK_BF16),
        "dx_gemm": (mdh2, M * h * b16 + h * d * b16 + M * d * b16, PEAK_BF16),
        "dw1_gemm": (mdh2, M * h * b16 + M * d * b16 + h * d * f32, PEAK_BF16),
        "dw2_gemm": (mdh2, M * d * b16 + M * h * b16 + d * h * f32, PEAK_BF16),
        # dW1 and dW2 in one launch
        "dw_gemm": (2 * mdh2, 2 * (M * h * b16 + M * d * b16 + h * d * f32), PEAK_BF16),
        "down_gemm_bf16_eval": (mdh2, M * h * b16 + h * d * b16 + M * d * b16, PEAK_BF16),
        "up_gemm_e4m3_relu2_quant": (mdh2, M * d * b8 + h * d * b8 + M * h * (b16 + b8), PEAK_FP8),
    }


# The bandwidth-bound kernels at the workload's large sizes, as --hbm-kernels
# runs them: algorithmic HBM bytes per launch.
def hbm_kernel_bytes(M, d, h):
    return {
        "amax_partial": M * h * 2,                  # max |x| over a [M, h] bf16 tensor (post-sized)
        "cast_transpose": M * h * 2 + M * h,        # [M, h] bf16 -> [h, M] e4m3, given scale
        "count_top_codes": M * h,                   # e4m3 codes at 448 in a [M, h] tensor
        "quantize_e4m3": M * d * 2 + M * d,         # X [M, d] bf16 -> e4m3 (fp8_linear's pass for K > 768)
    }


# launches that run more than one of the step's GEMMs
GEMMS_PER_LAUNCH = {"dw_gemm": 2}


def mixed_floor_us(M, d, h, fp8_gemms=1):
    """Time of the six GEMMs of a step at the published peaks, `fp8_gemms` of
    them (the down-projection; with the e4m3 up-projection two) in e4m3."""
    mdh = float(M) * d * h
    return ((12 - 2 * fp8_gemms) * mdh / (PEAK_BF16 * 1e12) + 2 * fp8_gemms * mdh / (PEAK_FP8 * 1e12)) * 1e6


# the sources the kernels of the timed step are compiled from
STEP_SOURCES = ("abi.hip", "common.h", "epilogues.h", "gemm.h", "host.h", "launch.h", "mlp_bwd.hip", "mlp_fwd.hip",
                "persist.h")


def kernel_source_hash():
    """Digest of the step's kernel sources: HBM counters are valid only for the code they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_relu_mlp_amd", "csrc")
    for f in STEP_SOURCES:
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def logical_kernel_name(raw):
    m = re.search(r"gemm\w*_kernel\d*<.*, (\d+)>\(", raw)
    if m:
        return KID_NAMES.get(int(m.group(1)), raw)
    m = re.search(r"fp8mlp::(k_\w+)", raw)
    if m:
        return OTHER_NAMES.get(m.group(1), m.group(1))
    return raw


def linear_work(M, d, n):
    """fp8_linear at M x d -> n: flops and algorithmic HBM bytes (X read once in bf16, the e4m3 weight,
    Y written in bf16) of one call."""
    return 2.0 * M * d * n, M * d * 2 + d * n + M * n * 2


LIN_CALLS, LIN_KEPT = 40, 20   # fp8_linear calls per `--linear` run; the last ones summarised


def summarize_linear(outdir):
    """profiles/kernel_trace_fp8_linear_M49152.md from rocprofv3 kernel traces of `bench.py --linear qkv`
    and `--linear o` under outdir/lin_qkv and outdir/lin_o."""
    cmd = "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/lin_{p} -o k -- python3 bench.py --linear {p}"
    lines = ["# fp8_linear kernel durations: the QKV and output projections, M=49152, K=768 (one MI355X)", "",
             "Commands (from a scratch directory, TMPDIR=/tmp):", "", "    " + cmd.format(p="qkv"),
             "    " + cmd.format(p="o"), "",
             f"Summarised with `python3 bench.py --summarize-linear OUT`.  Each run first runs the matrix-core",
             f"probe (~20 ms of e4m3 MFMA work, so the chip holds its loaded clocks), then {LIN_CALLS} calls; the",
             f"last {LIN_KEPT} are summarised.  Algorithmic bytes: X read once in bf16, the e4m3 weight, Y written",
             "in bf16.  Roofline time = max(flops / 5.0 PFLOP/s, bytes / 8 TB/s); fraction = roofline time /",
             "measured time.", "",
             "| projection | N | kernel | calls | avg us | TFLOP/s | of fp8 peak | GB/s alg. | of roofline |",
             "|---|---:|---|---:|---:|---:|---:|---:|---:|"]
    for proj, n in (("qkv", 3 * D), ("o", D)):
        files = sorted(glob.glob(os.path.join(outdir, f"lin_{proj}", "**", "*kernel_trace.csv"), recursive=True))
        if not files:
            raise SystemExit(f"no kernel trace under {os.path.join(outdir, 'lin_' + proj)}")
        with open(files[0]) as fh:
            trace = list(csv.DictReader(fh))
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                if logical_kernel_name(r["Kernel_Name"]) == "fp8_linear_panel"][-LIN_KEPT:]
        if not durs:
            raise SystemExit(f"no fp8_linear_panel dispatch in {files[0]}")
        avg = sum(durs) / len(durs)
        fl, by = linear_work(M, D, n)
        roof = max(fl / (PEAK_FP8 * 1e12), by / (PEAK_HBM * 1e9)) * 1e6
        lines.append(f"| {proj} | {n} | fp8_linear_panel | {len(durs)} | {avg:.1f} | {fl / avg / 1e6:.0f} | "
                     f"{fl / avg / 1e6 / PEAK_FP8:.3f} | {by / avg / 1e3:.0f} | {roof / avg:.3f} |")
    # counters (optional runs): HBM bytes scaled by the plain-copy calibration, matrix-core busy share
    subs = [f"lin_{p}_{c}" for p in ("qkv", "o") for c in ("fetch", "write", "mfma")] + ["cfetch", "cwrite"]
    if all(os.path.isdir(os.path.join(outdir, sub)) for sub in subs):
        ff, _ = copy_calibration(outdir, "cfetch", "FETCH_SIZE")
        wf, _ = copy_calibration(outdir, "cwrite", "WRITE_SIZE")
        pmc = "rocprofv3 --pmc {c} --output-format csv -d OUT/lin_{p}_{s} -o k -- python3 bench.py --linear {p}"
        lines += ["", "Counters per launch, one run per counter set and projection:", ""]
        for s_, c in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"), ("mfma", "MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_F8")):
            lines.append("    " + pmc.format(c=c, p="{qkv,o}", s=s_))
        lines += ["", f"HBM bytes: fetched = {ff:.3f} x FETCH_SIZE, written = {wf:.3f} x WRITE_SIZE (a plain 1 GiB",
                  "device copy under the same counters, `bench.py --copy-calibration`).  `MfmaUtil`: busy cycles of",
                  "the matrix cores over all SIMDs / (GPU active cycles x SIMDs), in per cent.", "",
                  "| projection | fetched MB | written MB | total MB | algorithmic MB | total / algorithmic | "
                  "MFMA GFLOP | MfmaUtil % |", "|---|---:|---:|---:|---:|---:|---:|---:|"]
        for proj, n in (("qkv", 3 * D), ("o", D)):
            def counter(sub, name):
                vals = [float(r["Counter_Value"]) for r in csv_rows(outdir, f"lin_{proj}_{sub}", "*counter_collection.csv")
                        if r["Counter_Name"] == name and logical_kernel_name(r["Kernel_Name"]) == "fp8_linear_panel"]
                if not vals:
                    raise SystemExit(f"no {name} of fp8_linear_panel under lin_{proj}_{sub}")
                return sum(vals) / len(vals)
            fb, wb = ff * 1024.0 * counter("fetch", "FETCH_SIZE"), wf * 1024.0 * counter("write", "WRITE_SIZE")
            gf = 512.0 * counter("mfma", "SQ_INSTS_VALU_MFMA_MOPS_F8") / 1e9
            _, by = linear_work(M, D, n)
            lines.append(f"| {proj} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | {by / 1e6:.1f} | "
                         f"{(fb + wb) / by:.2f} | {gf:.1f} | {counter('mfma', 'MfmaUtil'):.1f} |")
    with open(os.path.join(PROFILES, "kernel_trace_fp8_linear_M49152.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {PROFILES}/kernel_trace_fp8_linear_M49152.md")


def csv_rows(outdir, sub, pattern):
    """Rows of the first rocprofv3 CSV matching pattern under outdir/sub."""
    files = sorted(glob.glob(os.path.join(outdir, sub, "**", pattern), recursive=True))
    if not files:
        raise SystemExit(f"no {pattern} under {os.path.join(outdir, sub)}")
    with open(files[0]) as fh:
        return list(csv.DictReader(fh))


def copy_calibration(outdir, sub, counter, true_bytes=1 << 30):
    """(bytes per counted unit, raw bytes) from the plain 1 GiB device copy's counter run under outdir/sub."""
    vals = [float(r["Counter_Value"]) * 1024.0 for r in csv_rows(outdir, sub, "*counter_collection.csv")
            if r["Counter_Name"] == counter and "copyBuffer" in r["Kernel_Name"]]
    if not vals:
        raise SystemExit(f"no copy dispatch in {sub}")
    return true_bytes / (sum(vals) / len(vals)), sum(vals) / len(vals)


def summarize_profiles(outdir):
    """Turn the rocprofv3 runs under outdir (kt/: --kernel-trace --stats;
    fetch/, write/: --pmc FETCH_SIZE / WRITE_SIZE of this benchmark; cfetch/,
    cwrite/: the same counters for a plain 1 GiB device copy) into the text
    summaries under profiles/."""
    def rows(sub, pattern):
        return csv_rows(outdir, sub, pattern)

    cmd_bench = "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline --no-extras --no-graph"
    # kernel trace: per-dispatch durations
    trace = rows("kt", "*kernel_trace.csv")
    dur = {}
    for r in trace:
        n = logical_kernel_name(r["Kernel_Name"])
        dur.setdefault(n, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel durations: fused FP8 ReLU^2 MLP fwd+bwd, M=49152 d=768 h=3072 (one MI355X)", "",
             "Command (from a scratch directory, TMPDIR=/tmp):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/kt -o kt -- {cmd_bench}", "",
             "Summarised with `python3 bench.py --summarize-profiles OUT`.  Kernel names are the library's",
             "launch sites (GEMM kernels carry the site as a template argument).  The run includes the",
             "bootstrap forward and the warm-up steps.", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---:|---:|---:|---:|"]
    for n, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {n} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
    lines += ["", f"Kernel sources digest: `{kernel_source_hash()}`"]
    with open(os.path.join(PROFILES, "kernel_trace_mlp_fwd_bwd_M49152.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    # HBM counters, scaled by what the same counter reads for a plain copy
    def per_kernel(sub, counter):
        acc = {}
        for r in rows(sub, "*counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(logical_kernel_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sum(v) / len(v) for k, v in acc.items()}

    ff, fraw = copy_calibration(outdir, "cfetch", "FETCH_SIZE")
    wf, wraw = copy_calibration(outdir, "cwrite", "WRITE_SIZE")
    fetch, write = per_kernel("fetch", "FETCH_SIZE"), per_kernel("write", "WRITE_SIZE")
    work = kernel_work(M, D, H)
    table = {}
    lines = ["# HBM traffic per launch: fused FP8 ReLU^2 MLP fwd+bwd, M=49152 d=768 h=3072 (one MI355X)", "",
             "Commands (from a scratch directory, TMPDIR=/tmp; one counter per run):", "",
             f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/fetch -o f -- {cmd_bench}",
             f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/write -o w -- {cmd_bench}",
             "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/cfetch -o f -- python3 bench.py --copy-calibration",
             "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/cwrite -o w -- python3 bench.py --copy-calibration",
             "", "Calibration: a plain 1 GiB device-to-device copy reads "
             f"FETCH_SIZE = {fraw / 2**20:.1f} MiB and WRITE_SIZE = {wraw / 2**20:.1f} MiB, so fetched bytes = "
             f"{ff:.3f} x FETCH_SIZE and written bytes = {wf:.3f} x WRITE_SIZE.", "",
             "| kernel | fetched MB | written MB | total MB | algorithmic MB | total / algorithmic |",
             "|---|---:|---:|---:|---:|---:|"]
    for n in sorted(set(fetch) | set(write), key=lambda k: -(fetch.get(k, 0) + write.get(k, 0))):
        fb, wb = ff * fetch.get(n, 0.0), wf * write.get(n, 0.0)
        alg = work[n][1] if n in work else None
        table[n] = {"fetch_bytes": round(fb), "write_bytes": round(wb)}
        ratio = f"{(fb + wb) / alg:.2f}" if alg else ""
        algs = f"{alg / 1e6:.1f}" if alg else ""
        lines.append(f"| {n} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | {algs} | {ratio} |")
    lines += ["", f"Kernel sources digest: `{kernel_source_hash()}`"]
    with open(os.path.join(PROFILES, "hbm_traffic_mlp_fwd_bwd_M49152.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump({"src": kernel_source_hash(), "fetch_factor": ff, "write_factor": wf, "kernels": table}, fh,
                  indent=1)
        fh.write("\n")
    print(f"wrote {PROFILES}/kernel_trace_mlp_fwd_bwd_M49152.md, hbm_traffic_mlp_fwd_bwd_M49152.md, {TRAFFIC_FILE}")

    # bandwidth-bound kernels (optional run of --hbm-kernels under --kernel-trace)
    if os.path.isdir(os.path.join(outdir, "hbmk")):
        durs = {}
        for r in rows("hbmk", "*kernel_trace.csv"):
            n = logical_kernel_name(r["Kernel_Name"])
            durs.setdefault(n, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        nbytes = hbm_kernel_bytes(M, D, H)
        cmd = ("rocprofv3 --kernel-trace --stats --output-format csv -d OUT/hbmk -o k -- "
               "python3 bench.py --hbm-kernels")
        lines = ["# Bandwidth-bound kernels at the workload's sizes (one MI355X)", "",
                 "Command (from a scratch directory, TMPDIR=/tmp):", "", f"    {cmd}", "",
                 f"Sizes: M={M}, d={D}, h={H}. amax_partial: max |x| over a [M, h] bf16 tensor; cast_transpose:",
                 "[M, h] bf16 -> [h, M] e4m3 with a given scale; count_top_codes: the e4m3 codes at 448 in a",
                 "[M, h] tensor; quantize_e4m3: X [M, d] bf16 -> e4m3 (fp8_linear's conversion pass, which it",
                 "runs for K > 768: here X viewed as [M/2, 2d]; also the first step of the e4m3 up-projection). GB/s =",
                 f"algorithmic bytes per launch / average duration; peak HBM {PEAK_HBM / 1e3:.0f} TB/s.", "",
                 "| kernel | launches | avg us | algorithmic MB | GB/s | of peak |", "|---|---:|---:|---:|---:|---:|"]
        ours = set(OTHER_NAMES.values()) | set(KID_NAMES.values())
        for n in sorted((k for k in durs if k in ours), key=lambda k: -sum(durs[k]) / len(durs[k])):
            avg = sum(durs[n]) / len(durs[n])
            if n in nbytes:
                gbs = nbytes[n] / (avg * 1e-6) / 1e9
                lines.append(f"| {n} | {len(durs[n])} | {avg:.1f} | {nbytes[n] / 1e6:.1f} | {gbs:.0f} | "
                             f"{gbs / PEAK_HBM:.2f} |")
            else:
                lines.append(f"| {n} | {len(durs[n])} | {avg:.1f} |  |  |  |")
        lines += ["", f"Kernel sources digest: `{kernel_source_hash()}`"]
        with open(os.path.join(PROFILES, "kernel_trace_hbm_kernels_M49152.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"wrote {PROFILES}/kernel_trace_hbm_kernels_M49152.md")

    # matrix-core counters (optional run): executed MFMA work and busy share
    if os.path.isdir(os.path.join(outdir, "mfma")):
        acc = {}
        for r in rows("mfma", "*counter_collection.csv"):
            n = logical_kernel_name(r["Kernel_Name"])
            acc.setdefault(n, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        avg = {n: {c: sum(v) / len(v) for c, v in cs.items()} for n, cs in acc.items()}
        cmd = ("rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F8 "
               f"SQ_INSTS_VALU_MFMA_MOPS_F6F4 --output-format csv -d OUT/mfma -o m -- {cmd_bench}")
        lines = ["# Matrix-core counters per launch: fused FP8 ReLU^2 MLP fwd+bwd, M=49152 d=768 h=3072 (one MI355X)",
                 "", "Command (from a scratch directory, TMPDIR=/tmp):", "", f"    {cmd}", "",
                 "MFMA GFLOP = (SQ_INSTS_VALU_MFMA_MOPS_BF16 + _F8 + _F6F4) x 512 (the counters count multiply-",
                 "adds / 512); `MfmaUtil` = busy cycles of the matrix cores over all SIMDs / (GPU active cycles x",
                 "SIMDs), in per cent, so it folds in the clock the kernel actually ran at.", "",
                 "| kernel | MFMA GFLOP | algorithmic GFLOP | MfmaUtil % |", "|---|---:|---:|---:|"]
        for n in sorted(avg, key=lambda k: -avg[k].get("MfmaUtil", 0.0)):
            c = avg[n]
            gf = 512.0 * sum(c.get(x, 0.0) for x in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                                                      "SQ_INSTS_VALU_MFMA_MOPS_F6F4")) / 1e9
            alg = f"{work[n][0] / 1e9:.1f}" if n in work else ""
            lines.append(f"| {n} | {gf:.1f} | {alg} | {c.get('MfmaUtil', float('nan')):.1f} |")
        lines += ["", f"Kernel sources digest: `{kernel_source_hash()}`"]
        with open(os.path.join(PROFILES, "mfma_counters_mlp_fwd_bwd_M49152.md"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print(f"wrote {PROFILES}/mfma_counters_mlp_fwd_bwd_M49152.md")


def measured_traffic():
    """Per-launch HBM bytes from the committed counter summary, or {} when
    the kernels have changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return {}
    if t.get("src") != kernel_source_hash():
        return {}
    return {k: v["fetch_bytes"] + v["write_bytes"] for k, v in t.get("kernels", {}).items()}


def cpu_baseline(ins, amax_prev, gpu=None, chunk=4096):
    """The oracle (as it stands) on the whole workload: all M token rows of
    fwd (TRAIN) + bwd + the W2 cache refresh, in row chunks of ``chunk`` (the
    weight gradients summed over the chunks) to bound host memory.

    With ``gpu`` (the GPU's Y, dX, dW1, dW2 and post_q of one step from the
    same inputs and amax_prev), the oracle's outputs are also compared with
    them (relative Frobenius errors, share of differing e4m3 codes); the
    comparison time is not part of the timed baseline."""
    import numpy as np
    from oracle import formats as F
    from oracle import mlp as O
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    t_cmp = 0.0
    err = {"Y": [0.0, 0.0], "dX": [0.0, 0.0]}
    mismatch = 0

    def as_f64(a):
        a = np.asarray(a)
        return F.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    W2t, _, inv_sw, _ = O.cast_transpose(ins["W2"])
    dW1 = np.zeros((H, D))
    dW2 = np.zeros((D, H))
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        out = O.mlp_fwd(ins["X"][r0:r1], ins["W1"], W2t, inv_sw, amax_prev, MARGIN)
        bw = O.mlp_bwd(ins["dY"][r0:r1], ins["X"][r0:r1], ins["W1"], ins["W2"], F.bf16_to_f64(out["post"]))
        dW1 += bw["dW1"]
        dW2 += bw["dW2"]
        if gpu is not None:
            tc = time.perf_counter()
            for k, ref in (("Y", out["y"]), ("dX", bw["dX"])):
                r, g = as_f64(ref), as_f64(gpu[k][r0:r1])
                err[k][0] += float(np.sum((g - r) ** 2))
                err[k][1] += float(np.sum(r ** 2))
            mismatch += int(np.count_nonzero(np.asarray(out["post_q"]) != gpu["post_q"][r0:r1]))
            t_cmp += time.perf_counter() - tc
    t = time.perf_counter() - t0 - t_cmp
    parity = None
    if gpu is not None:
        rel = {k: (v[0] / v[1]) ** 0.5 if v[1] > 0 else 0.0 for k, v in err.items()}
        for k, ref in (("dW1", dW1), ("dW2", dW2)):
            rel[k] = float(np.linalg.norm(gpu[k].astype(np.float64) - ref) / np.linalg.norm(ref))
        gates = {"Y": 2e-2, "dX": 1e-2, "dW1": 1e-2, "dW2": 1e-2}
        parity = {"rel_fro": {k: round(v, 6) for k, v in rel.items()}, "gates": gates,
                  "post_q_codes_differing": mismatch / float(M * H),
                  "pass": all(rel[k] <= g for k, g in gates.items()),
                  "against": "the oracle run on its own from X, W1, W2, dY and the step's amax_prev"}
    # cores: the threads the oracle's BLAS calls ran on (its other numpy steps run on one)
    return {"value": 12.0 * M * D * H / t / 1e12, "unit": "TFLOP/s", "cores": blas, "kind": "oracle",
            "sample": f"the whole workload: all {M} token rows (d={D}, h={H}), fwd+bwd+W2 refresh, in row chunks "
                      f"of {chunk}, {t:.1f} s", "seconds": round(t, 2), "blas_threads": blas,
            "affinity_cores": cores, "parity": parity}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the FP8-linear / eval / ablation lines")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay pass (profiler runs)")
    ap.add_argument("--sustain", type=float, metavar="SECONDS",
                    help="after the warm-up, run the step back to back for SECONDS and print the rate only")
    ap.add_argument("--jsonl", metavar="PATH",
                    help="also append the record, with host cores, GPU identity and clocks, to this JSONL file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 5 times (scales the HBM byte counters)")
    ap.add_argument("--hbm-kernels", action="store_true",
                    help="only run the bandwidth-bound kernels at the workload's large sizes, 5 launches each "
                         "(for a rocprofv3 kernel trace)")
    ap.add_argument("--linear", choices=("qkv", "o"),
                    help="only run fp8_linear on the QKV or output projection (M=49152, K=768), 2 + 5 calls "
                         "(for a rocprofv3 kernel trace)")
    ap.add_argument("--summarize-linear", metavar="OUT",
                    help="write profiles/kernel_trace_fp8_linear_M49152.md from the rocprofv3 runs of --linear "
                         "under OUT/lin_qkv and OUT/lin_o (no GPU needed)")
    ap.add_argument("--summarize-profiles", metavar="OUT",
                    help="write the profiles/ summaries from the rocprofv3 runs under OUT (no GPU needed)")
    args = ap.parse_args()
    if args.summarize_linear:
        summarize_linear(args.summarize_linear)
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the multi-GPU data-parallel path is "
              "not implemented, so there is no figure for more than one GPU", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 5}))
        return

    import fp8_relu_mlp_amd as fm
    from fp8_relu_mlp_amd import synth

    dev = torch.device("cuda:0")
    fm.lib()
    if args.hbm_kernels:
        # post-sized bf16 values >= 0, their e4m3 codes and a bf16 X, generated on the device
        g = torch.Generator(device=dev).manual_seed(7)
        big = torch.randn((M, H), generator=g, device=dev).square_().to(torch.bfloat16)
        xs = torch.randn((M, D), generator=g, device=dev).to(torch.bfloat16)
        f1 = lambda v=0.0: torch.full((1,), v, dtype=torch.float32, device=dev)
        amx, sc, sx, xam = f1(), f1(16.0), f1(64.0), f1()
        ws_a = torch.empty(max(1, fm.lib().amax_reduce_workspace(M * H)), dtype=torch.uint8, device=dev)
        ws_c = torch.empty(max(1, fm.lib().fp8_cast_transpose_workspace(M, H)), dtype=torch.uint8, device=dev)
        q = torch.empty((H, M), dtype=torch.uint8, device=dev)
        cnt = torch.zeros(1, dtype=torch.int64, device=dev)
        ws_t = torch.empty(max(1, fm.lib().fp8_saturation_count_workspace(M * H)), dtype=torch.uint8, device=dev)
        # fp8_linear with K = 2d > 768 runs its conversion pass over all of X, then a narrow GEMM
        wt = torch.zeros((2 * D, 64), dtype=torch.uint8, device=dev)
        winv = f1(1.0)
        yl = torch.empty((M // 2, 64), dtype=torch.bfloat16, device=dev)
        ws_l = torch.empty(max(1, fm.lib().fp8_linear_workspace(M // 2, 2 * D)), dtype=torch.uint8, device=dev)
        for _ in range(5):
            fm.amax_reduce(big, amx, workspace=ws_a)
        for _ in range(5):
            fm.fp8_cast_transpose(big, q, scale_in=sc, workspace=ws_c)
        for _ in range(5):
            fm.fp8_saturation_count(q, cnt, workspace=ws_t)
        for _ in range(5):
            fm.fp8_linear(xs.view(M // 2, 2 * D), sx, wt, winv, yl, x_amax_out=xam, workspace=ws_l)
        torch.cuda.synchronize()
        print(json.dumps({"bytes_per_launch": hbm_kernel_bytes(M, D, H), "launches": 5}))
        return
    if args.linear:
        a = synth.attn_inputs()
        xk, wk, n = ("X", "Wqkv", 3 * D) if args.linear == "qkv" else ("Xo", "Wo", D)

        def bf1(x):
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

        Xa, Wa = bf1(a[xk]), bf1(a[wk])
        Wt = torch.empty((D, n), dtype=torch.uint8, device=dev)
        f1 = lambda v=0.0: torch.full((1,), v, dtype=torch.float32, device=dev)
        inv_w, amax, sx = f1(), f1(), f1()
        fm.fp8_cast_transpose(Wa, Wt, inv_scale_out=inv_w)
        fm.amax_reduce(Xa, amax)
        fm.fp8_scale_from_amax(amax, 1.0, sx)
        Ya = torch.empty((Xa.shape[0], n), dtype=torch.bfloat16, device=dev)
        wsl = torch.empty(max(1, fm.lib().fp8_linear_workspace(Xa.shape[0], D)), dtype=torch.uint8, device=dev)
        # the chip to the clocks it holds under matrix work first (as before the step's warm-up)
        sink = torch.empty(fm.PROBE_BLOCKS * 256, dtype=torch.float32, device=dev)
        fm.mfma_probe(fm.MFMA_E4M3, Wt, Wt, 20000, sink)
        for _ in range(LIN_CALLS):
            fm.fp8_linear(Xa, sx, Wt, inv_w, Ya, workspace=wsl)
        torch.cuda.synchronize()
        print(json.dumps({"projection": args.linear, "M": int(Xa.shape[0]), "K": D, "N": n, "calls": LIN_CALLS}))
        return
    log("generating inputs")
    ins = synth.mlp_inputs(M, D, H, synth.WORKLOADS["fwdbwd"][3], with_dy=True)

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    X, W1, W2, dY = bf(ins["X"]), bf(ins["W1"]), bf(ins["W2"]), bf(ins["dY"])
    blk = fm.Relu2MLP(W1, W2, margin=MARGIN, amax_init=1.0)
    post = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    post_q = torch.empty((M, H), dtype=torch.uint8, device=dev)
    Y = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, D), dtype=torch.bfloat16, device=dev)
    dW1 = torch.empty((H, D), dtype=torch.float32, device=dev)
    dW2 = torch.empty((D, H), dtype=torch.float32, device=dev)
    L = fm.lib()
    ws_f = torch.empty(max(1, L.mlp_relu2_fwd_workspace(M, D, H)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, L.mlp_relu2_bwd_workspace(M, D, H)), dtype=torch.uint8, device=dev)
    ws_c = torch.empty(max(1, L.fp8_cast_transpose_workspace(D, H)), dtype=torch.uint8, device=dev)

    def step():
        blk.forward(X, post=post, post_q=post_q, Y=Y, workspace=ws_f)
        blk.backward(dY, X, post, dX, dW1, dW2, workspace=ws_b)
        blk.refresh_w2_cache(workspace=ws_c)

    blk.forward(X, post=post, post_q=post_q, Y=Y, workspace=ws_f)   # bootstrap amax_prev
    torch.cuda.synchronize()

    # matrix-core rate on the workload's own operands (the clock under a dense
    # MFMA load depends on the data; the published peaks assume 2.4 GHz).  It
    # runs before the warm-up: its ~20 ms of dense matrix work bring the chip
    # to the clocks it holds under this load, which an idle chip takes some
    # 20 steps to reach (those steps run up to 10 % slower).
    log("matrix-core rate probe")
    sink = torch.empty(fm.PROBE_BLOCKS * 256, dtype=torch.float32, device=dev)

    def probe_rate(dtype, a, b, iters=20000):
        fm.mfma_probe(dtype, a, b, iters // 10, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fl = fm.mfma_probe(dtype, a, b, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        return fl / (e0.elapsed_time(e1) * 1e-3) / 1e12

    probe = {"bf16_tflops": round(probe_rate(fm.MFMA_BF16, X, W1), 1),
             "e4m3_tflops": round(probe_rate(fm.MFMA_E4M3, post_q, blk.W2t_q), 1),
             "operands": "X and W1 (bf16), post_q and W2t_q (e4m3) of this workload"}

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    if args.sustain:
        # the warm step back to back for a while (for sampling the socket power beside it)
        t0, n = time.time(), 0
        while time.time() - t0 < args.sustain:
            for _ in range(50):
                step()
            n += 50
            torch.cuda.synchronize()
        dt = time.time() - t0
        print(json.dumps({"sustain_s": round(dt, 2), "steps": n, "us_per_step": round(1e6 * dt / n, 1)}))
        return

    log(f"timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 12.0 * M * D * H
    value = flops / (ms * 1e-3) / 1e12
    floor_us = mixed_floor_us(M, D, H)
    log(f"{ms:.3f} ms/step, {value:.1f} TFLOP/s")

    # per-kernel durations: the same steps again with every launch bracketed by events
    log("per-kernel timing pass")
    with fm.KernelTimer(64 * args.steps) as kt:
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    per = {}
    for name, t in kt.records():
        per.setdefault(name, []).append(t)
    work = kernel_work(M, D, H)
    traffic = measured_traffic()
    kernels = {}
    for name, ts in per.items():
        avg_us = 1e3 * sum(ts) / len(ts)
        entry = {"launches_per_step": len(ts) / args.steps, "avg_us": round(avg_us, 2)}
        if name in work:
            fl, by, peak = work[name]
            entry.update(tflops=round(fl / (avg_us * 1e-6) / 1e12, 1), frac_mfma=round(fl / (avg_us * 1e-6) / 1e12 / peak, 4),
                         hbm_gbs_alg=round(by / (avg_us * 1e-6) / 1e9, 1))
        if name in traffic:
            entry["hbm_bytes_measured"] = traffic[name]
        kernels[name] = entry
    gemms = [n for n in kernels if n in work]
    # the dominant contraction: a launch that runs several GEMMs counts per GEMM
    dom = max(gemms, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches_per_step"] / GEMMS_PER_LAUNCH.get(n, 1))
    fl, by, peak = work[dom]
    achieved = fl / (kernels[dom]["avg_us"] * 1e-6) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": traffic.get(dom),
                "algorithmic_flops_per_launch": fl, "algorithmic_bytes_per_launch": by}

    # the same step replayed from a HIP graph (two steps per graph, so the
    # forward's amax buffer swap comes back to the captured roles); no entry
    # point allocates, synchronises or reads a device value, so capture holds
    graph_ms = None
    if not args.no_graph:
        graph_ms = graph_replay_ms(torch, step, args.steps)
        log(f"graph replay: {graph_ms:.3f} ms/step")

    roofline["probe_peak"] = probe["bf16_tflops"] if peak == PEAK_BF16 else probe["e4m3_tflops"]
    roofline["frac_of_probe_peak"] = round(achieved / roofline["probe_peak"], 4)

    power = None
    if not args.no_extras:
        log("socket power while the step runs back to back")
        power = socket_power(torch, step)
    extras = {}
    if not args.no_extras:
        log("extra measurements")
        extras = extra_measurements(fm, torch, dev, X, W1, W2, dY, blk, post, post_q, Y, dX, dW1, dW2, ws_f, ws_b,
                                    ws_c)

    cpu = None
    if not args.no_cpu_baseline:
        # one more step whose outputs the oracle's are compared with
        amax_used = float(blk.amax_prev.item())
        blk.forward(X, post=post, post_q=post_q, Y=Y, workspace=ws_f)
        blk.backward(dY, X, post, dX, dW1, dW2, workspace=ws_b)
        torch.cuda.synchronize()
        u16 = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
        gpu_out = {"Y": u16(Y), "dX": u16(dX), "dW1": dW1.cpu().numpy(), "dW2": dW2.cpu().numpy(),
                   "post_q": post_q.cpu().numpy()}
        log("cpu baseline (the oracle on the whole workload)")
        cpu = cpu_baseline(ins, amax_used, gpu_out)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16+e4m3 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": "relu2_mlp_fwd_bwd_gpt2_small", "M": M, "d": D, "h": H, "margin": MARGIN,
                   "step": "fwd(train)+bwd+W2 cache refresh"},
        "pct_mixed_mfma_peak": round(100.0 * floor_us / (ms * 1e3), 2),
        "graph_replay": None if graph_ms is None else {
            "ms_per_step": round(graph_ms, 4), "value": round(flops / (graph_ms * 1e-3) / 1e12, 2),
            "pct_mixed_mfma_peak": round(100.0 * floor_us / (graph_ms * 1e3), 2),
            "steps": 2 * max(1, args.steps // 2), "how": "fwd+bwd+W2 refresh, two steps per captured HIP graph"},
        "mixed_mfma_floor_us": round(floor_us, 1),
        "roofline": roofline,
        "mfma_probe": probe,
        "power": power,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)
    if args.jsonl:
        rec = dict(out, time_utc=time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()), host=host_info(),
                   gpu=gpu_info(torch))
        with open(args.jsonl, "a") as fh:
            fh.write(json.dumps(rec) + "\n")


def host_info():
    info = {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "python": sys.version.split()[0]}
    try:
        from threadpoolctl import threadpool_info
        info["blas_threads"] = max([p.get("num_threads", 1) for p in threadpool_info()
                                    if p.get("user_api") == "blas"] or [1])
    except Exception:
        pass
    return info


def gpu_info(torch):
    """Identity of GPU 0 and its shader-clock levels as the driver lists them
    (sysfs pp_dpm_sclk, the current level marked *), where readable."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1), "torch": torch.__version__,
            "hip": getattr(torch.version, "hip", None)}
    for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(f) as fh:
                info["sclk_levels"] = [ln.strip() for ln in fh if ln.strip()]
            break
        except OSError:
            continue
    return info


def socket_power(torch, step, seconds=3.0):
    """Median socket power (amd-smi) while the step runs back to back for
    `seconds`, sampled from a thread after the first second; None when
    amd-smi is not there or reports nothing."""
    import shutil
    import subprocess
    import threading
    if shutil.which("amd-smi") is None:
        return None
    samples, stop = [], threading.Event()

    def sample():
        t0 = time.time()
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "--power"], capture_output=True, text=True, timeout=10)
                m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", r.stdout)
                if m and time.time() - t0 > 1.0:
                    samples.append(float(m.group(1)))
            except (OSError, subprocess.SubprocessError):
                return
            time.sleep(0.25)

    th = threading.Thread(target=sample, daemon=True)
    t0, n = time.time(), 0
    th.start()
    while time.time() - t0 < seconds:
        for _ in range(20):
            step()
        n += 20
        torch.cuda.synchronize()
    dt = time.time() - t0
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None
    samples.sort()
    return {"socket_w_median": samples[len(samples) // 2], "socket_w_max": samples[-1], "samples": len(samples),
            "us_per_step": round(1e6 * dt / n, 1),
            "how": f"amd-smi metric --power every ~0.3 s while the step ran back to back for {seconds:.0f} s"}


def graph_replay_ms(torch, step, steps):
    """The step replayed from a HIP graph: two steps per graph, so the
    forward's amax buffer swap comes back to the captured roles; no entry
    point allocates, synchronises or reads a device value, so capture holds."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
        step()
    torch.cuda.synchronize()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    reps = max(1, steps // 2)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (2 * reps)
    del graph
    return ms


def extra_measurements(fm, torch, dev, X, W1, W2, dY, blk, post, post_q, Y, dX, dW1, dW2, ws_f, ws_b, ws_c,
                       reps=20):
    """Side measurements (not part of `value`): forward-only TRAIN vs EVAL
    (bf16 down-projection ablation), the W2 cache refresh, the step with the
    up-projection in e4m3 as well (mlp_relu2_fwd_fp8up, both weight caches
    refreshed after the update), the step that keeps only the e4m3 copy of
    post (mlp_relu2_bwd_fp8post), the layer-stack
    workload (12 layers x 8 SGD steps at M=65536, with the share of e4m3
    post codes at the top code per layer and step, counted by the library)
    and the FP8 attention projections."""
    import numpy as np
    from fp8_relu_mlp_amd import synth

    def timed(fn, reps=reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {}
    mdh2 = 2.0 * M * D * H
    t_tr = timed(lambda: blk.forward(X, post=post, post_q=post_q, Y=Y, carry=False, workspace=ws_f))
    t_ev = timed(lambda: blk.forward(X, mode=fm.EVAL_BF16, post=post, Y=Y, carry=False, workspace=ws_f))
    out["fwd_train_fp8_ms"] = round(t_tr, 4)
    out["fwd_eval_bf16_ms"] = round(t_ev, 4)
    out["fwd_train_tflops"] = round(2 * mdh2 / (t_tr * 1e-3) / 1e12, 1)
    ws_c = torch.empty(max(1, fm.lib().fp8_cast_transpose_workspace(D, H)), dtype=torch.uint8, device=dev)
    t_w2 = timed(lambda: fm.fp8_cast_transpose_w2(W2, blk.W2t_q, blk.w2_scale, blk.w2_inv_scale, blk.w2_amax,
                                                  workspace=ws_c))
    out["w2_refresh_us"] = round(t_w2 * 1e3, 2)
    out["w2_refresh_gbs_alg"] = round((D * H * 2 * 2 + D * H) / (t_w2 * 1e-3) / 1e9, 1)

    # the naive unfused forward the pages warn about: the up-projection stores
    # only post, a separate pass rescans it for amax, another quantises it,
    # then the FP8 down-projection (fp8_linear = quantise pass + e4m3 GEMM);
    # summed kernel durations, against the fused forward's
    amx, sxn = torch.zeros(1, dtype=torch.float32, device=dev), torch.zeros(1, dtype=torch.float32, device=dev)
    ws_a = torch.empty(max(1, fm.lib().amax_reduce_workspace(M * H)), dtype=torch.uint8, device=dev)
    ws_l = torch.empty(max(1, fm.lib().fp8_linear_workspace(M, H)), dtype=torch.uint8, device=dev)

    def naive():
        blk.forward(X, mode=fm.EVAL_BF16, post=post, Y=Y, carry=False, workspace=ws_f)
        fm.amax_reduce(post, amx, workspace=ws_a)
        fm.fp8_scale_from_amax(amx, MARGIN, sxn)
        fm.fp8_linear(post, sxn, blk.W2t_q, blk.w2_inv_scale, Y, workspace=ws_l)

    def kernel_sums(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        with fm.KernelTimer(256 * reps) as kt:
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        acc = {}
        for name, t in kt.records():
            acc[name] = acc.get(name, 0.0) + 1e3 * t / reps
        return acc

    kn = kernel_sums(naive)
    kf = kernel_sums(lambda: blk.forward(X, post=post, post_q=post_q, Y=Y, carry=False, workspace=ws_f))
    naive_parts = {k: round(v, 1) for k, v in kn.items() if k != "down_gemm_bf16_eval"}
    out["naive_unfused_fwd_us"] = round(sum(naive_parts.values()), 1)
    out["naive_unfused_fwd_parts_us"] = naive_parts
    out["fused_fwd_kernels_us"] = round(sum(kf.values()), 1)
    del ws_l

    # cast-transpose and amax at large sizes (HBM-bound): [49152, 3072] bf16
    Wbig = post.view(M, H)
    Wt_big = torch.empty((H, M), dtype=torch.uint8, device=dev)
    ws_big = torch.empty(max(1, fm.lib().fp8_cast_transpose_workspace(M, H)), dtype=torch.uint8, device=dev)
    t_cb = timed(lambda: fm.fp8_cast_transpose(Wbig, Wt_big, scale_in=sxn, workspace=ws_big))
    out["cast_transpose_49152x3072_us"] = round(t_cb * 1e3, 1)
    out["cast_transpose_49152x3072_gbs"] = round((M * H * 3) / (t_cb * 1e-3) / 1e9, 1)
    t_ab = timed(lambda: fm.amax_reduce(post, amx, workspace=ws_a))
    out["amax_reduce_post_us"] = round(t_ab * 1e3, 1)
    out["amax_reduce_post_gbs"] = round((M * H * 2) / (t_ab * 1e-3) / 1e9, 1)
    del Wt_big, ws_big, ws_a

    # the same step with both forward GEMMs in e4m3
    blk8 = fm.Relu2MLP(W1, W2, margin=MARGIN, amax_init=1.0, fp8_up=True)
    ws_8 = torch.empty(max(1, fm.lib().mlp_relu2_fwd_fp8up_workspace(M, D, H)), dtype=torch.uint8, device=dev)
    blk8.forward(X, post=post, post_q=post_q, Y=Y, workspace=ws_8)        # bootstrap both amaxes

    def step8():
        blk8.forward(X, post=post, post_q=post_q, Y=Y, workspace=ws_8)
        blk8.backward(dY, X, post, dX, dW1, dW2, workspace=ws_b)
        blk8.refresh_caches(workspace=ws_c)

    t_f8 = timed(lambda: blk8.forward(X, post=post, post_q=post_q, Y=Y, carry=False, workspace=ws_8))
    t_s8 = timed(step8)
    out["fp8up_fwd_ms"] = round(t_f8, 4)
    out["fp8up_fwd_tflops"] = round(2 * mdh2 / (t_f8 * 1e-3) / 1e12, 1)
    out["fp8up_step_ms"] = round(t_s8, 4)
    out["fp8up_step_tflops"] = round(6 * mdh2 / (t_s8 * 1e-3) / 1e12, 1)
    out["fp8up_step_pct_mixed_mfma_peak"] = round(100.0 * mixed_floor_us(M, D, H, 2) / (t_s8 * 1e3), 2)
    with fm.KernelTimer(64 * reps) as kt:
        for _ in range(reps):
            step8()
    torch.cuda.synchronize()
    ts = [t for name, t in kt.records() if name == "up_gemm_e4m3_relu2_quant"]
    if ts:
        us = 1e3 * sum(ts) / len(ts)
        out["fp8up_up_gemm_us"] = round(us, 2)
        out["fp8up_up_gemm_tflops"] = round(mdh2 / (us * 1e-6) / 1e12, 1)
        out["fp8up_up_gemm_frac_fp8_peak"] = round(mdh2 / (us * 1e-6) / 1e12 / PEAK_FP8, 4)
    xq = [t for name, t in kt.records() if name == "quantize_e4m3"]
    if xq:
        out["fp8up_quantize_x_us"] = round(1e3 * sum(xq) / len(xq), 2)
    del blk8, ws_8

    # the step without the bf16 post: the backward runs on the e4m3 copy
    blkq = fm.Relu2MLP(W1, W2, margin=MARGIN, amax_init=1.0, keep_post=False)
    blkq.forward(X, post_q=post_q, Y=Y, workspace=ws_f)

    def stepq():
        blkq.forward(X, post_q=post_q, Y=Y, workspace=ws_f)
        blkq.backward(dY, X, None, dX, dW1, dW2, workspace=ws_b, post_q=post_q)
        blkq.refresh_w2_cache(workspace=ws_c)

    t_fq = timed(lambda: blkq.forward(X, post_q=post_q, Y=Y, carry=False, workspace=ws_f))
    t_sq = timed(stepq)
    out["fp8post_fwd_ms"] = round(t_fq, 4)
    out["fp8post_step_ms"] = round(t_sq, 4)
    out["fp8post_step_tflops"] = round(6 * mdh2 / (t_sq * 1e-3) / 1e12, 1)
    out["fp8post_step_pct_mixed_mfma_peak"] = round(100.0 * mixed_floor_us(M, D, H) / (t_sq * 1e3), 2)
    with fm.KernelTimer(64 * reps) as kt:
        for _ in range(reps):
            stepq()
    torch.cuda.synchronize()
    perq = {}
    for name, t in kt.records():
        perq.setdefault(name, []).append(t)
    out["fp8post_kernels_us"] = {k: round(1e3 * sum(v) / len(v), 2) for k, v in perq.items()
                                 if k in ("up_gemm_relu2_quant", "dpost_gemm_dpre", "dw2_gemm")}
    del blkq

    # both variants together: e4m3 up-projection, no bf16 post
    blkb = fm.Relu2MLP(W1, W2, margin=MARGIN, amax_init=1.0, fp8_up=True, keep_post=False)
    ws_b8 = torch.empty(max(1, fm.lib().mlp_relu2_fwd_fp8up_workspace(M, D, H)), dtype=torch.uint8, device=dev)
    blkb.forward(X, post_q=post_q, Y=Y, workspace=ws_b8)

    def stepb():
        blkb.forward(X, post_q=post_q, Y=Y, workspace=ws_b8)
        blkb.backward(dY, X, None, dX, dW1, dW2, workspace=ws_b, post_q=post_q)
        blkb.refresh_caches(workspace=ws_c)

    t_sb = timed(stepb)
    out["fp8up_fp8post_step_ms"] = round(t_sb, 4)
    out["fp8up_fp8post_step_tflops"] = round(6 * mdh2 / (t_sb * 1e-3) / 1e12, 1)
    out["fp8up_fp8post_step_pct_mixed_mfma_peak"] = round(100.0 * mixed_floor_us(M, D, H, 2) / (t_sb * 1e3), 2)
    del blkb, ws_b8

    # layer-stack workload: 12 layers x 8 SGD steps at M=65536 (state carry per layer)
    from fp8_relu_mlp_amd.stack import Relu2Stack
    Ms, ds, hs, seed_s = synth.WORKLOADS["stack"]
    Ls, steps_s = synth.STACK["layers"], synth.STACK["steps"]

    def bfd(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    wts = synth.stack_weights(Ls, ds, hs, seed_s)
    batches = [synth.stack_batch(Ms, ds, seed_s, t) for t in range(steps_s)]
    Xs = [bfd(b["X"]) for b in batches]
    dYs = [bfd(b["dY"]) for b in batches]

    def stack_run(top=None, **opts):
        stk = Relu2Stack([bfd(w1) for w1, _ in wts], [bfd(w2) for _, w2 in wts], lr=synth.STACK["lr"],
                         telemetry=top is not None, **opts)
        stk.step(Xs[0], dYs[0])            # allocation + the bootstrap step, untimed
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for t in range(steps_s):
            stk.step(Xs[t], dYs[t])
            if top is not None:
                # fp8_saturation_count of every layer's e4m3 post copy (the library's count kernel)
                top.append(stk.saturated.double().cpu().numpy() / (Ms * hs))
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    t_stack = stack_run()
    top = []
    stack_run(top)
    fl_stack = 12.0 * Ms * ds * hs * Ls * steps_s
    floor_stack = steps_s * Ls * mixed_floor_us(Ms, ds, hs) / 1e3
    out["stack_12x8_ms"] = round(t_stack, 2)
    out["stack_12x8_tflops"] = round(fl_stack / (t_stack * 1e-3) / 1e12, 1)
    out["stack_12x8_mixed_floor_ms"] = round(floor_stack, 2)
    # share of e4m3 post codes at the top code (448) per layer and step: an
    # upper bound on the clipped share, 0 when nothing came near the limit
    out["stack_top_code_rate_max"] = float(np.max(top))
    out["stack_top_code_nonzero_layer_steps"] = int(np.count_nonzero(np.stack(top)))
    t_stack8 = stack_run(fp8_up=True)
    out["stack_12x8_fp8up_ms"] = round(t_stack8, 2)
    out["stack_12x8_fp8up_tflops"] = round(fl_stack / (t_stack8 * 1e-3) / 1e12, 1)
    t_stackq = stack_run(keep_post=False)
    out["stack_12x8_fp8post_ms"] = round(t_stackq, 2)
    t_stackb = stack_run(fp8_up=True, keep_post=False)
    out["stack_12x8_fp8up_fp8post_ms"] = round(t_stackb, 2)
    out["stack_12x8_fp8up_fp8post_tflops"] = round(fl_stack / (t_stackb * 1e-3) / 1e12, 1)

    # margin / window sweep with the top-code telemetry (share of e4m3 post
    # codes at 448 per layer and step, bootstrap step excluded)
    sweep = []
    for margin, window in ((1.0, 1), (1.25, 1), (2.0, 1), (4.0, 1), (1.25, 4)):
        stk = Relu2Stack([bfd(w1) for w1, _ in wts], [bfd(w2) for _, w2 in wts], lr=synth.STACK["lr"],
                         margin=margin, amax_window=window, telemetry=True)
        stk.step(Xs[0], dYs[0])
        rates = []
        for t in range(steps_s):
            stk.step(Xs[t], dYs[t])
            rates.append(stk.saturated.double().cpu().numpy() / (Ms * hs))
        r = np.stack(rates)
        sweep.append({"margin": margin, "window": window, "top_code_rate_max": float(r.max()),
                      "top_code_rate_mean": float(r.mean()),
                      "layer_steps_with_top_codes": int(np.count_nonzero(r))})
        del stk
    out["margin_sweep"] = sweep
    del Xs, dYs

    # fused softcapped cross-entropy over the head: M=49152, d=768, V=50304, 3 targets
    ce = synth.CE
    ci = synth.ce_inputs(ce["M"], ce["d"], ce["V"], ce["T"], ce["seed"], seq=ce["seq"])
    Xc, Wc = bfd(ci["X"]), bfd(ci["W"])
    tc = torch.from_numpy(ci["targets"].astype(np.int32)).to(dev)
    wc = torch.tensor(ce["weights"], dtype=torch.float32, device=dev)
    lossc = torch.zeros(1, device=dev)
    dXc = torch.empty_like(Xc)
    dWc = torch.empty((ce["V"], ce["d"]), dtype=torch.float32, device=dev)
    wsc = torch.empty(fm.lib().softcap_ce_workspace(ce["M"], ce["V"], ce["d"], ce["T"]), dtype=torch.uint8,
                      device=dev)
    run_ce = lambda: fm.softcap_ce_fwd_bwd(Xc, Wc, tc, wc, ce["softcap"], lossc, dXc, dWc, workspace=wsc)
    t_ce = timed(run_ce, reps=5)
    fl_ce = 4 * 2.0 * ce["M"] * ce["d"] * ce["V"]
    out["ce_fwd_bwd_ms"] = round(t_ce, 3)
    out["ce_fwd_bwd_tflops"] = round(fl_ce / (t_ce * 1e-3) / 1e12, 1)
    out["ce_frac_bf16_peak"] = round(fl_ce / (t_ce * 1e-3) / 1e12 / PEAK_BF16, 4)
    with fm.KernelTimer(64) as kt:
        run_ce()
    torch.cuda.synchronize()
    out["ce_kernels_us"] = {n: round(1e3 * t, 1) for n, t in kt.records()}
    out["ce_loss"] = round(float(lossc.item()), 5)
    del wsc
    # the FP8 head: e4m3 X (exact scale) and the transposed e4m3 W cache
    Wtc = torch.empty((ce["d"], ce["V"]), dtype=torch.uint8, device=dev)
    invc = torch.zeros(1, dtype=torch.float32, device=dev)
    fm.fp8_cast_transpose(Wc, Wtc, inv_scale_out=invc)
    amc = torch.zeros(1, dtype=torch.float32, device=dev)
    fm.amax_reduce(Xc, amc)
    sxc = torch.zeros(1, dtype=torch.float32, device=dev)
    fm.fp8_scale_from_amax(amc, 1.0, sxc)
    wsc8 = torch.empty(fm.lib().softcap_ce_fp8_workspace(ce["M"], ce["V"], ce["d"], ce["T"]), dtype=torch.uint8,
                       device=dev)
    run_ce8 = lambda: fm.softcap_ce_fwd_bwd_fp8(Xc, sxc, Wtc, invc, Wc, tc, wc, ce["softcap"], lossc, dXc, dWc,
                                                workspace=wsc8)
    t_ce8 = timed(run_ce8, reps=5)
    out["ce_fp8_fwd_bwd_ms"] = round(t_ce8, 3)
    out["ce_fp8_fwd_bwd_tflops"] = round(fl_ce / (t_ce8 * 1e-3) / 1e12, 1)
    with fm.KernelTimer(64) as kt:
        run_ce8()
    torch.cuda.synchronize()
    out["ce_fp8_kernels_us"] = {n: round(1e3 * t, 1) for n, t in kt.records()}
    out["ce_fp8_loss"] = round(float(lossc.item()), 5)
    del Xc, Wc, tc, wsc8, dXc, dWc, Wtc

    # FP8 attention projections: QKV [49152,768]x[768,2304], O [49152,768]x[768,768]
    a = synth.attn_inputs()

    def bf(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    for tag, xk, wk, n in (("qkv", "X", "Wqkv", 2304), ("o", "Xo", "Wo", 768)):
        Xa, Wa = bf(a[xk]), bf(a[wk])
        Wt = torch.empty((D, n), dtype=torch.uint8, device=dev)
        inv_w = torch.zeros(1, dtype=torch.float32, device=dev)
        fm.fp8_cast_transpose(Wa, Wt, inv_scale_out=inv_w)
        amax = torch.zeros(1, dtype=torch.float32, device=dev)
        fm.amax_reduce(Xa, amax)
        sx = torch.zeros(1, dtype=torch.float32, device=dev)
        fm.fp8_scale_from_amax(amax, 1.0, sx)
        Ya = torch.empty((Xa.shape[0], n), dtype=torch.bfloat16, device=dev)
        wsl = torch.empty(max(1, fm.lib().fp8_linear_workspace(Xa.shape[0], D)), dtype=torch.uint8, device=dev)
        t = timed(lambda: fm.fp8_linear(Xa, sx, Wt, inv_w, Ya, workspace=wsl))
        fl, by = linear_work(Xa.shape[0], D, n)
        roof_ms = max(fl / (PEAK_FP8 * 1e12), by / (PEAK_HBM * 1e9)) * 1e3
        out[f"fp8_linear_{tag}_us"] = round(t * 1e3, 2)
        out[f"fp8_linear_{tag}_frac_roofline"] = round(roof_ms / t, 4)
        out[f"fp8_linear_{tag}_tflops"] = round(fl / (t * 1e-3) / 1e12, 1)
        out[f"fp8_linear_{tag}_frac_fp8_peak"] = round(fl / (t * 1e-3) / 1e12 / PEAK_FP8, 4)
        out[f"fp8_linear_{tag}_hbm_gbs_alg"] = round(by / (t * 1e-3) / 1e9, 1)
    return out


if __name__ == "__main__":
    main()
