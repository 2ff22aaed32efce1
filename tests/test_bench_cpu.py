"""Host logic of bench.py, on the CPU: the rocprofv3 summaries that feed the
JSON line's roofline (per-launch traffic averaged over the step's own launches,
copy calibration taken after the library's kernels, clock from busy cycles),
the kernel-symbol lookup, and the one-GPU guard."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMM = "void mx::(anonymous namespace)::pipe::k_gemm_pipe<2, 2, true, 0>(mx::GemmArgs)"
ROWS = "void mx::(anonymous namespace)::k_quantize_rows<2, true, true>(x)"
DUAL = "void mx::(anonymous namespace)::k_quantize_transpose<2, true, true, 2, false>(x)"
FLUSH = "void at::native::reduce_kernel<512, 1>(x)"
CONVERT = "void at::native::vectorized_elementwise_kernel<copy>(x)"
CALIB = "__amd_rocclr_copyBuffer"

# (dispatch, kernel, FETCH_SIZE KiB, WRITE_SIZE KiB, duration ns)
RUN = [
    (1, ROWS, 100.0, 50.0, 20000),     # the step: quantizer at one size
    (2, GEMM, 1000.0, 500.0, 400000),  # the step's GEMM
    (3, ROWS, 300.0, 150.0, 30000),    # quantizer at another size
    (4, GEMM, 1000.0, 500.0, 400000),
    (5, FLUSH, 0.0, 0.0, 90000),       # first cache fill: the step ends here
    (6, GEMM, 1000.0, 500.0, 450000),  # lone launch
    (7, CONVERT, 999999.0, 999999.0, 200000),  # a big dtype conversion (not the calibration)
    (8, GEMM, 5000.0, 10.0, 900000),   # the same kernel at another shape (extra record)
    (9, DUAL, 200.0, 120.0, 80000),    # a kernel only the extra records run
    (10, CALIB, 131072.0, 262144.0, 60000),  # 256 MiB calibration copies
    (11, CALIB, 131072.0, 262144.0, 60000),
]
CMDS = ("trace --steps 2 --warmup 0", "fetch", "write", "clock --steps 2 --warmup 0",
        "mfma --steps 2 --warmup 0", "lds --steps 2 --warmup 0")


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


@pytest.fixture()
def profile_dirs(tmp_path):
    t0 = 1000000
    trace, counters = [], {"FETCH_SIZE": [], "WRITE_SIZE": [], "GRBM_GUI_ACTIVE": []}
    for d, k, fk, wk, dt in RUN:
        s, e = t0 + d * 10 ** 7, t0 + d * 10 ** 7 + dt
        trace.append([d, k, s, e])
        counters["FETCH_SIZE"].append([d, k, "FETCH_SIZE", fk, s, e])
        counters["WRITE_SIZE"].append([d, k, "WRITE_SIZE", wk, s, e])
        # busy cycles of a 2.0 GHz clock summed over the dies
        counters["GRBM_GUI_ACTIVE"].append([d, k, "GRBM_GUI_ACTIVE", 2.0 * bench.XCDS * dt, s, e])
    stats = {}
    for d, k, _, _, dt in RUN:
        stats.setdefault(k, []).append(dt)
    _write(str(tmp_path / "trace" / "t_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    _write(str(tmp_path / "trace" / "t_kernel_stats.csv"),
           ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "TotalDurationNs"],
           [[k, len(v), sum(v) / len(v), min(v), max(v), sum(v)] for k, v in stats.items()])
    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    for name, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write"), ("GRBM_GUI_ACTIVE", "clock")):
        _write(str(tmp_path / sub / ("x_counter_collection.csv")), head, counters[name])
    # MfmaUtil: 40 and 50 % for the step's two GEMM launches, 0 for the quantizer
    mf = [[d, k, "MfmaUtil", (40.0 + 10.0 * (d == 4)) if k == GEMM else 0.0, 0, 1] for d, k, _, _, _ in RUN]
    _write(str(tmp_path / "mfma" / "x_counter_collection.csv"), head, mf)
    # LDS: the GEMM's two step launches busy 1000 and 3000 cycles with 10 and 50 conflict cycles;
    # the quantizer uses no LDS
    lds = []
    for d, k, _, _, _ in RUN:
        if k == GEMM:
            act, con = (1000.0, 10.0) if d == 2 else (3000.0, 50.0)
        else:
            act, con = 0.0, 0.0
        lds += [[d, k, "SQ_LDS_IDX_ACTIVE", act, 0, 1], [d, k, "SQ_LDS_BANK_CONFLICT", con, 0, 1]]
    _write(str(tmp_path / "lds" / "x_counter_collection.csv"), head, lds)
    return tmp_path


def test_summaries(profile_dirs):
    out = profile_dirs / "out"
    bench.summarize_profiles(*(str(profile_dirs / d) for d in ("trace", "fetch", "write", "clock")),
                             command=CMDS, out_dir=str(out))
    data = json.load(open(out / "traffic.json"))
    assert data["source_sha"] == bench.kernel_source_sha()
    # calibration: the copies after the last library kernel, not the larger conversion
    assert data["fetch_scale"] == pytest.approx(2.0) and data["write_scale"] == pytest.approx(1.0)
    k = data["kernels"]
    # the step's two GEMM launches only (not the lone launch, not the other shape)
    assert k[GEMM]["read_bytes"] == pytest.approx(1000.0 * 2 * 1024)
    assert k[GEMM]["write_bytes"] == pytest.approx(500.0 * 1024)
    # a kernel the step runs at two sizes: the mean over those
    assert k[ROWS]["read_bytes"] == pytest.approx(200.0 * 2 * 1024)
    # a kernel only the extra records run: its own launches
    assert k[DUAL]["bytes_per_launch"] == pytest.approx(200.0 * 2 * 1024 + 120.0 * 1024)
    # clock: 2.0 GHz for the GEMM; the 20-30 us quantizer launches are left out
    assert data["sclk_ghz"] == {GEMM: pytest.approx(2.0)}
    for name in ("kernel_trace_%s.md", "hbm_traffic_%s.md", "sclk_%s.md"):
        text = open(out / (name % bench.WORKLOAD)).read()
        assert "Command" in text or "Commands" in text
    assert "| 2 | 400.0 |" in open(out / ("kernel_trace_%s.md" % bench.WORKLOAD)).read()


def test_kernel_symbols():
    assert bench.kernel_symbol("llama31_8b_gateup_fprop_mxfp4/Y mx_gemm e2m1xe2m1") == GEMM
    assert bench.kernel_symbol("llama31_8b_wgrad_mxfp4_hadamard/dW mx_gemm_layout e2m1xe2m1") == \
        "void mx::(anonymous namespace)::pipe::k_gemm_pipe<2, 2, false, 0>(mx::GemmArgs)"
    assert bench.kernel_symbol("llama31_8b_qkv_fprop_mxfp8/Y mx_gemm e4m3xe4m3") == \
        "void mx::(anonymous namespace)::pipe::k_gemm_pipe<0, 0, true, 1>(mx::GemmArgs)"


def test_quant_bytes():
    assert bench.quant_bytes(32, 64, "e4m3") == 32 * 64 * (2 + 1 + 1 / 32)
    assert bench.quant_bytes(32, 64, "e2m1") == 32 * 64 * (2 + 0.5 + 1 / 32)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_mfma_summary(profile_dirs):
    out = profile_dirs / "out2"
    bench.summarize_profiles(*(str(profile_dirs / d) for d in ("trace", "fetch", "write", "clock")),
                             command=CMDS, out_dir=str(out), mfma_dir=str(profile_dirs / "mfma"))
    data = json.load(open(out / "traffic.json"))
    # the mean over the step's two GEMM launches (40 and 50); kernels reading 0 are left out
    assert data["mfma_util_pct"] == {GEMM: pytest.approx(45.0)}
    assert "| 2 | 45.0 |" in open(out / ("mfma_util_%s.md" % bench.WORKLOAD)).read()


def test_lds_summary(profile_dirs):
    out = profile_dirs / "out3"
    bench.summarize_profiles(*(str(profile_dirs / d) for d in ("trace", "fetch", "write", "clock")),
                             command=CMDS, out_dir=str(out), mfma_dir=str(profile_dirs / "mfma"),
                             lds_dir=str(profile_dirs / "lds"))
    data = json.load(open(out / "traffic.json"))
    # (10 + 50) / (1000 + 3000) over the step's two GEMM launches; the quantizer (no LDS) is left out
    assert data["lds_conflict_pct"] == {GEMM: pytest.approx(1.5)}
    assert "| 2 | 0.00 | 0.000 | 1.50% |" in open(out / ("lds_bank_conflicts_%s.md" % bench.WORKLOAD)).read()


def test_ablation_summary(tmp_path):
    abl = {"shape": "dW[2x2]", "metric": "rel", "plain": 0.25,
           "random": {"mean": 0.2, "min": 0.1, "max": 0.3, "error_of_the_8_step_average": 0.05}}
    path = tmp_path / "abl.md"
    bench.write_ablation_summary(abl, str(path), 0)
    text = open(path).read()
    assert "--ablation --seed 0" in text and "| plain | 0.2500 |" in text and "| 0.1000 / 0.3000 | 0.0500 |" in text
