"""CPU tests of the benchmark's host arithmetic and its command line."""

from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("nq,nk", [(1, 1), (5, 5), (7, 3), (3, 7), (1, 9), (9, 1), (64, 100), (100, 64)])
def test_visible_pairs_brute_force(nq, nk):
    mask = np.arange(nk)[None, :] <= (np.arange(nq) + nk - nq)[:, None]
    assert bench.visible_pairs(nq, nk, True) == int(mask.sum())
    assert bench.visible_pairs(nq, nk, False) == nq * nk


def test_workload_figures():
    fl = bench.attention_flops(2, 16, 4096, 4096, 128, True)
    assert fl["fwd"] == 137_472_507_904                      # 4 d B H N(N+1)/2
    assert fl["dkdv"] + fl["dq"] == 343_681_269_760          # 2.5 x forward
    assert bench.attention_flops(1, 16, 16384, 16384, 128, True)["fwd"] == 1_099_578_736_640
    assert bench.attention_flops(4, 8, 1024, 1024, 64, False)["fwd"] == 8_589_934_592
    assert bench.decode_bytes(8, 32, 8, 32768, 128, 2) == 1_073_939_488


def test_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def _counter_csv(path, rows):
    """A rocprofv3-style counter CSV: rows of (dispatch, kernel, counter, value, start, end)."""
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for r in rows:
            w.writerow(r)


def test_util_from_reads_the_last_launch_of_each_kernel(tmp_path):
    fwd = "fa::fwd_kernel<bf16>"
    rows = []
    # Two launches of the forward: 1000 ns at half MFMA busy, then 500 ns fully busy.
    # GRBM_GUI_ACTIVE sums 8 XCDs; MFMA busy cycles sum 1024 SIMDs.
    for disp, start, end, grbm_xcd, busy in ((1, 0, 1000, 2000, 0.5), (2, 2000, 2500, 1200, 1.0)):
        rows += [(disp, fwd, "GRBM_GUI_ACTIVE", 8 * grbm_xcd, start, end),
                 (disp, fwd, "SQ_VALU_MFMA_BUSY_CYCLES", busy * grbm_xcd * 1024, start, end),
                 (disp, fwd, "SQ_LDS_BANK_CONFLICT", 10, start, end),
                 (disp, fwd, "SQ_LDS_IDX_ACTIVE", 110, start, end)]
    _counter_csv(tmp_path / "c.csv", rows)
    rec = bench.util_from(str(tmp_path / "c.csv"), out_dir=str(tmp_path))
    assert rec["fwd"]["mfma_busy"] == 1.0
    assert rec["fwd"]["clock_ghz"] == 2.4                    # 1200 cycles in 500 ns
    assert rec["fwd"]["lds_bank_conflicts_per_access"] == 0.1
    assert rec["fwd"]["us"] == 0.5
    assert os.path.exists(tmp_path / "mfma_util.json")


def test_util_from_drops_counters_of_launches_shorter_than_the_window(tmp_path):
    """GRBM cycles beyond duration x 2.4 GHz mean the counter window outlasted
    the launch: busy fraction and clock are then not reported."""
    prep = "fa::bwd_prep_kernel<bf16>"
    rows = [(1, prep, "GRBM_GUI_ACTIVE", 8 * 3934, 0, 1000),   # 3.934 GHz over 1 us: impossible
            (1, prep, "SQ_VALU_MFMA_BUSY_CYCLES", 0, 0, 1000),
            (1, prep, "SQ_LDS_BANK_CONFLICT", 0, 0, 1000),
            (1, prep, "SQ_LDS_IDX_ACTIVE", 10, 0, 1000)]
    _counter_csv(tmp_path / "c.csv", rows)
    rec = bench.util_from(str(tmp_path / "c.csv"), out_dir=str(tmp_path))
    assert rec["prep"]["mfma_busy"] is None and rec["prep"]["clock_ghz"] is None
    assert rec["prep"]["lds_bank_conflicts_per_access"] == 0.0


def test_traffic_from_scales_by_the_calibration_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    gib_kib = bench.COPY_BYTES // 1024
    # The counters read the copy at half its true bytes; the decode's split and
    # reduce kernels are summed per launch, averaged over launches.
    fetch = [(1, copy, "FETCH_SIZE", gib_kib / 2, 0, 1),
             (2, "decode_split_kernel<bf16>", "FETCH_SIZE", 100, 0, 1),
             (3, "decode_reduce_kernel<bf16>", "FETCH_SIZE", 10, 0, 1),
             (4, "decode_split_kernel<bf16>", "FETCH_SIZE", 300, 0, 1)]
    write = [(1, copy, "WRITE_SIZE", gib_kib, 0, 1),
             (2, "decode_split_kernel<bf16>", "WRITE_SIZE", 4, 0, 1),
             (3, "decode_reduce_kernel<bf16>", "WRITE_SIZE", 1, 0, 1)]
    _counter_csv(tmp_path / "f.csv", fetch)
    _counter_csv(tmp_path / "w.csv", write)
    rec = bench.traffic_from(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), out_dir=str(tmp_path))
    assert rec["_calibration"]["fetch_factor"] == 2.0 and rec["_calibration"]["write_factor"] == 1.0
    assert rec["decode"]["fetch_bytes"] == (200 + 10) * 1024 * 2
    assert rec["decode"]["write_bytes"] == (4 + 1) * 1024
    assert os.path.exists(tmp_path / "traffic.json") and os.path.exists(tmp_path / "hbm_traffic_mha_bf16_4k_decode_fp8.md")


def test_trace_summary_labels_dispatches_by_leg(tmp_path):
    """Dispatches are assigned to legs in LEG_ORDER by their counts."""
    import csv
    steps, warmup = 2, 1
    rows, t = [], 0
    names = {"fwd": "_ZN2fa12_GLOBAL__N_110fwd_kernelIDF16bLi128ELb1ELb0ELi8EEEvNS0_9FwdParamsEPKiS4_",
             "other": "at::native::elementwise_kernel"}
    for leg, per_step in bench.LEG_ORDER:
        passes = 2 if leg in bench.TWO_PASS_LEGS else 1
        for _ in range((steps * passes + warmup) * per_step):
            rows.append((names["fwd"], t, t + 1000 if leg != "mha_bf16_4k" else t + 3000))
            t += 5000
    rows.append((names["other"], t, t + 500))
    with open(tmp_path / "trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writerows(rows)
    text = bench.trace_summary(str(tmp_path / "trace.csv"), steps, warmup)
    line = [l for l in text.splitlines() if l.startswith("| mha_bf16_4k |")][0]
    calls = (2 * steps + warmup) * dict(bench.LEG_ORDER)["mha_bf16_4k"]
    assert "`fwd_kernel<bf16, 128, 1, 0, 8>`" in line and f"| {calls} | 3.00 | 3.00 |" in line
    assert any(l.startswith("| (torch / runtime) |") for l in text.splitlines())


def test_trace_summary_knows_every_library_kernel():
    """Every __global__ kernel in the library's HIP sources is one that the
    trace summary counts as an attention dispatch (a kernel it did not know
    would be filed under torch / runtime and shift every later leg)."""
    import glob
    import re
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "exact_io_aware_47_amd", "csrc")
    names = set()
    for path in glob.glob(os.path.join(csrc, "*.hip")):
        text = open(path).read()
        for m in re.finditer(r"__global__", text):
            k = re.search(r"\b(\w+_kernel)\s*\(", text[m.end():m.end() + 400])
            assert k, f"no kernel name after __global__ in {path}"
            names.add(k.group(1))
    assert {"fwd_kernel", "bwd_dkdv16_kernel", "bwd_dq_kernel", "decode_split_kernel"} <= names
    for n in sorted(names):
        mangled = f"_ZN2fa12_GLOBAL__N_1{len(n)}{n}IDF16bLi128EEEvv"
        assert any(k in mangled for k in bench.ATTENTION_KERNEL), n
