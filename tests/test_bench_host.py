"""Host logic of bench.py (no GPU): the algorithmic work it divides by, the
published-peak floor, the kernel-name mapping of rocprofv3 traces, the
counter summaries and the one-GPU guard.

The expected figures are computed by hand for this workload (M=49152,
d=768, h=3072): per-kernel HBM bytes 533.2 / 228.9 / 684.2 /
386.9 / 386.9 / 382.2 MB, 1.3916 TFLOP per fwd+bwd, the mixed floor 506.9 us
at 256 CU x 2.4 GHz peaks; fp8_linear QKV 173.9 GFLOP and 303.8 MB, O 58.0
GFLOP and 151.6 MB.
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

M, D, H = 49152, 768, 3072


def test_step_work_matches_the_hand_computed_table():
    w = bench.kernel_work(M, D, H)
    mb = {k: v[1] / 1e6 for k, v in w.items()}
    assert mb["up_gemm_relu2_quant"] == pytest.approx(533.2, abs=0.05)
    assert mb["down_gemm_e4m3"] == pytest.approx(228.9, abs=0.05)
    assert mb["dpost_gemm_dpre"] == pytest.approx(684.2, abs=0.05)
    assert mb["dw1_gemm"] == pytest.approx(386.9, abs=0.05)
    assert mb["dw2_gemm"] == pytest.approx(386.9, abs=0.05)
    assert mb["dx_gemm"] == pytest.approx(382.2, abs=0.05)
    assert mb["dw_gemm"] == pytest.approx(2 * 386.9, abs=0.1)
    step = ("up_gemm_relu2_quant", "down_gemm_e4m3", "dpost_gemm_dpre", "dx_gemm", "dw_gemm")
    assert sum(w[k][0] for k in step) / 1e12 == pytest.approx(1.3916, abs=1e-4)
    assert sum(w[k][1] for k in step) / 1e9 == pytest.approx(2.60, abs=0.005)
    # the e4m3 GEMMs are priced at the fp8 peak, the others at bf16
    assert w["down_gemm_e4m3"][2] == bench.PEAK_FP8 and w["up_gemm_relu2_quant"][2] == bench.PEAK_BF16


def test_mixed_floor(monkeypatch):
    # at peaks from 256 CU x 2.4 GHz (2516.6 / 5033.2 TFLOP/s) the floor is
    # 506.9 us; at the rounded published 2.5 / 5.0 PFLOP/s it is 510.2 us
    monkeypatch.setattr(bench, "PEAK_BF16", 2516.6)
    monkeypatch.setattr(bench, "PEAK_FP8", 5033.2)
    assert bench.mixed_floor_us(M, D, H) == pytest.approx(506.9, abs=0.05)
    monkeypatch.undo()
    assert bench.mixed_floor_us(M, D, H) == pytest.approx(510.2, abs=0.05)
    # both forward GEMMs in e4m3: 8 bf16 + 4 fp8 GEMM-halves of M d h
    assert bench.mixed_floor_us(M, D, H, fp8_gemms=2) == pytest.approx(463.9, abs=0.05)


def test_linear_work():
    fl, by = bench.linear_work(M, D, 3 * D)
    assert fl / 1e9 == pytest.approx(173.9, abs=0.05) and by / 1e6 == pytest.approx(303.8, abs=0.05)
    fl, by = bench.linear_work(M, D, D)
    assert fl / 1e9 == pytest.approx(58.0, abs=0.05) and by / 1e6 == pytest.approx(151.6, abs=0.05)


# kernel names as rocprofv3 reports them for this library
TRACE_NAMES = {
    "void fp8mlp::gemm_pp_kernel<fp8mlp::GemmCfg<2, 256, 256, 128, 2, 1, 0, 0, 0, 8, 0, 3>, "
    "fp8mlp::EpiRelu2QuantT<false>, 1>(fp8mlp::GemmArgs, fp8mlp::EpiRelu2QuantT<false>)": "up_gemm_relu2_quant",
    "void fp8mlp::gemm_pp_kernel<fp8mlp::GemmCfg<1, 192, 384, 128, 2, 1, 0, 1, 0, 8, 0, 2>, fp8mlp::EpiBf16Out, 2>"
    "(fp8mlp::GemmArgs, fp8mlp::EpiBf16Out)": "down_gemm_e4m3",
    "void fp8mlp::gemm_pp_persist_kernel<fp8mlp::GemmCfg<2, 256, 256, 128, 2, 1, 0, 0, 0, 8, 0, 3>, "
    "fp8mlp::EpiDpreWP, 4>(fp8mlp::GemmArgs, fp8mlp::EpiDpreWP, int)": "dpost_gemm_dpre",
    "void fp8mlp::gemm_pp_kernel<fp8mlp::GemmCfg<2, 192, 256, 128, 2, 1, 0, 0, 0, 8, 0, 3>, fp8mlp::EpiBf16Out, 5>"
    "(fp8mlp::GemmArgs, fp8mlp::EpiBf16Out)": "dx_gemm",
    "void fp8mlp::gemm_pp_kernel2<fp8mlp::GemmCfg<2, 256, 256, 128, 2, 1, 1, 1, 0, 8, 0, 3>, fp8mlp::EpiF32Part, 16>"
    "(fp8mlp::GemmArgs, fp8mlp::EpiF32Part, fp8mlp::GemmArgs, fp8mlp::EpiF32Part, int, int)": "dw_gemm",
    "void fp8mlp::k_splitk_reduce_tiles<fp8mlp::GemmCfg<2, 256, 256, 128, 2, 1, 1, 1, 0, 8, 0, 3> >"
    "(fp8mlp::RedProb, fp8mlp::RedProb, int, long, int)": "splitk_reduce",
    "fp8mlp::k_transpose_weights(unsigned short const*, unsigned short const*, long, long, unsigned short*, "
    "unsigned short*)": "transpose_weights",
    "void fp8mlp::k_amax_partial<1>(void const*, long, unsigned int*)": "amax_partial",
    "fp8mlp::k_cast_transpose(unsigned short const*, long, long, unsigned char*, float const*, unsigned int const*, "
    "int, float*, float*, float*)": "cast_transpose",
}


def test_logical_kernel_names():
    for raw, name in TRACE_NAMES.items():
        assert bench.logical_kernel_name(raw) == name, raw
    other = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >(int)"
    assert bench.logical_kernel_name(other) == other


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summaries_from_synthetic_counters(tmp_path, monkeypatch):
    """Counters in KiB; a 1 GiB copy that reports 512 MiB fetched and 1 GiB
    written gives the factors 2 and 1, and a kernel's bytes are the factor
    times its counter, averaged over its dispatches."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(prof / "traffic.txt"))
    out = tmp_path / "out"
    up, dx = [k for k, v in TRACE_NAMES.items() if v == "up_gemm_relu2_quant"][0], \
        [k for k, v in TRACE_NAMES.items() if v == "dx_gemm"][0]
    trace_hdr = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    _write_csv(str(out / "kt" / "kt_kernel_trace.csv"), trace_hdr,
               [[up, 1000, 251000], [up, 300000, 550000], [dx, 600000, 800000]])
    cnt_hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(str(out / "cfetch" / "f_counter_collection.csv"), cnt_hdr,
               [["__amd_rocclr_copyBuffer", "FETCH_SIZE", 512 * 1024]])
    _write_csv(str(out / "cwrite" / "w_counter_collection.csv"), cnt_hdr,
               [["__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024 * 1024]])
    # up: fetched 2 x (200000, 216000) KiB averaged, written 1 x 440000 KiB
    _write_csv(str(out / "fetch" / "f_counter_collection.csv"), cnt_hdr,
               [[up, "FETCH_SIZE", 200000], [up, "FETCH_SIZE", 216000], [dx, "FETCH_SIZE", 300000]])
    _write_csv(str(out / "write" / "w_counter_collection.csv"), cnt_hdr,
               [[up, "WRITE_SIZE", 440000], [dx, "WRITE_SIZE", 74000]])
    bench.summarize_profiles(str(out))
    t = json.loads((prof / "traffic.txt").read_text())
    assert t["fetch_factor"] == pytest.approx(2.0) and t["write_factor"] == pytest.approx(1.0)
    assert t["kernels"]["up_gemm_relu2_quant"] == {"fetch_bytes": 2 * 208000 * 1024, "write_bytes": 440000 * 1024}
    assert t["kernels"]["dx_gemm"] == {"fetch_bytes": 2 * 300000 * 1024, "write_bytes": 74000 * 1024}
    md = (prof / "kernel_trace_mlp_fwd_bwd_M49152.md").read_text()
    assert "| up_gemm_relu2_quant | 2 | 250.0 | 250.0 | 250.0 |" in md
    assert "| dx_gemm | 1 | 200.0 |" in md
    traffic_md = (prof / "hbm_traffic_mlp_fwd_bwd_M49152.md").read_text()
    up_total = (2 * 208000 + 440000) * 1024 / 1e6
    assert f"| up_gemm_relu2_quant | {2 * 208000 * 1024 / 1e6:.1f} |" in traffic_md
    up_alg = bench.kernel_work(bench.M, bench.D, bench.H)["up_gemm_relu2_quant"][1] / 1e6
    assert traffic_md.split("up_gemm_relu2_quant")[1].splitlines()[0].endswith(f"| {up_total / up_alg:.2f} |")
    # the summary is tied to the sources it was taken on
    assert bench.measured_traffic()["dx_gemm"] == (2 * 300000 + 74000) * 1024
    t["src"] = "0" * 16
    (prof / "traffic.txt").write_text(json.dumps(t))
    assert bench.measured_traffic() == {}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
