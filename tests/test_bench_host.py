"""CPU checks of bench.py's host logic: the profiler-summary bookkeeping that
feeds `roofline.traffic` (scaling by the reference copy, per-workload records,
staleness by source hash), the matrix-core and copy-overlap summaries, and the
single-GPU guard.  No GPU is touched.
"""
import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FETCH_KIB_COPY = 524288.0   # a 1 GiB copy reads half its bytes in FETCH_SIZE units on this counter
WRITE_KIB_COPY = 1048576.0


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    """A copy of the kernel sources and an empty profiles/ folder, with bench.ROOT pointing at it."""
    csrc = tmp_path / "long_context_exact_ring_amd" / "csrc"
    shutil.copytree(os.path.join(ROOT, "long_context_exact_ring_amd", "csrc"), csrc)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def _summarize(root, workload, fetch_kib, write_kib):
    kern = "void ra::bwd_dkdv_bf16_kernel<128, 32, 8, true, true>(ra::BwdArgs)"
    copy = "__amd_rocclr_copyBuffer"
    fetch = root / "fetch.csv"
    write = root / "write.csv"
    stats = root / "stats.csv"
    # two dispatches of the kernel (averaged), a small host upload and the 1 GiB reference copy
    _counter_csv(fetch, [(kern, "FETCH_SIZE", fetch_kib - 10), (kern, "FETCH_SIZE", fetch_kib + 10),
                         (copy, "FETCH_SIZE", 64.0), (copy, "FETCH_SIZE", FETCH_KIB_COPY)])
    _counter_csv(write, [(kern, "WRITE_SIZE", write_kib), (kern, "WRITE_SIZE", write_kib),
                         (copy, "WRITE_SIZE", 128.0), (copy, "WRITE_SIZE", WRITE_KIB_COPY)])
    with open(stats, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "TotalDurationNs", "Percentage"])
        w.writeheader()
        w.writerow({"Name": kern, "Calls": 2, "AverageNs": 2.0e6, "TotalDurationNs": 4.0e6, "Percentage": 100})
    bench.summarize_profiles(str(stats), str(fetch), str(write), 1024, workload)


def test_traffic_is_scaled_by_the_largest_copy_and_kept_per_workload(fake_root, capsys):
    _summarize(fake_root, "causal_128k_h32_d128", fetch_kib=1000.0, write_kib=300.0)
    capsys.readouterr()
    # FETCH scaled by 1 GiB / 512 MiB = 2, WRITE by 1; KiB -> bytes
    expect = round(1000.0 * 2 * 1024 + 300.0 * 1024)
    assert bench.profiled_traffic("bwd_dkdv", 128, "bf16", "causal_128k_h32_d128") == expect
    # another workload, head_dim or dtype has no record
    assert bench.profiled_traffic("bwd_dkdv", 128, "bf16", "bwd_causal_32k_h32_d128") is None
    assert bench.profiled_traffic("bwd_dkdv", 64, "bf16", "causal_128k_h32_d128") is None
    assert bench.profiled_traffic("bwd_dkdv", 128, "f32", "causal_128k_h32_d128") is None
    # a second workload's summary leaves the first one in place
    _summarize(fake_root, "bwd_causal_32k_h32_d128", fetch_kib=10.0, write_kib=3.0)
    capsys.readouterr()
    rec = json.load(open(fake_root / "profiles" / "traffic.json"))
    assert set(rec["workloads"]) == {"causal_128k_h32_d128", "bwd_causal_32k_h32_d128"}
    assert bench.profiled_traffic("bwd_dkdv", 128, "bf16", "causal_128k_h32_d128") == expect


def test_traffic_goes_stale_when_the_kernel_source_changes(fake_root, capsys):
    _summarize(fake_root, "causal_128k_h32_d128", fetch_kib=1000.0, write_kib=300.0)
    capsys.readouterr()
    assert bench.profiled_traffic("bwd_dkdv", 128, "bf16", "causal_128k_h32_d128") is not None
    # an unrelated kernel's source does not matter ...
    with open(fake_root / "long_context_exact_ring_amd" / "csrc" / "ffn.hip", "a") as f:
        f.write("\n// edit\n")
    assert bench.profiled_traffic("bwd_dkdv", 128, "bf16", "causal_128k_h32_d128") is not None
    # ... its own source or a shared header does
    with open(fake_root / "long_context_exact_ring_amd" / "csrc" / "kernels.h", "a") as f:
        f.write("\n// edit\n")
    assert bench.profiled_traffic("bwd_dkdv", 128, "bf16", "causal_128k_h32_d128") is None


def test_kernel_sources_cover_each_kernels_file():
    assert "bwd_bf16.hip" in bench.kernel_sources("ra::bwd_dkdv_bf16_kernel<128, 32, 8, true, true>")
    assert "ffn.hip" in bench.kernel_sources("ra::gemm_bt_kernel<2, 4, 4, 2, true>")
    assert "decode.hip" in bench.kernel_sources("ra::decode_partial_kernel<128, 2>")
    assert "fwd_step.hip" in bench.kernel_sources("ra::fwd_bf16_kernel<128, 64, 8, 1>")
    for name in ("ra::fwd_bf16_kernel<128, 64, 8, 1>", "something::else"):
        srcs = bench.kernel_sources(name)
        assert "kcommon.h" in srcs and "kernels.h" in srcs
        for f in srcs:
            assert os.path.exists(os.path.join(ROOT, "long_context_exact_ring_amd", "csrc", f)), f


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_mfma_busy_is_normalised_to_four_simds(tmp_path, capsys):
    path = tmp_path / "sq.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for d, (k, busy_cu, mfma) in enumerate((("ra::mfma_rate_kernel(int, float*)", 100.0, 400.0),
                                                ("void ra::fwd_bf16_kernel<128, 64, 8, 1>(ra::FwdArgs)", 100.0, 200.0))):
            for c, v in (("SQ_BUSY_CU_CYCLES", busy_cu), ("SQ_VALU_MFMA_BUSY_CYCLES", mfma), ("SQ_WAVE_CYCLES", 1000.0),
                         ("SQ_WAIT_ANY", 400.0), ("SQ_ACTIVE_INST_ANY", 300.0)):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})
    bench.summarize_mfma(str(path))
    out = capsys.readouterr().out
    assert "| `ra::mfma_rate_kernel` | 1 | 1.00 | 0.40 | 0.30 |" in out
    assert "| `ra::fwd_bf16_kernel<128, 64, 8, 1>` | 1 | 0.50 |" in out


def test_copy_overlap_counts_only_device_copies_under_kernels(tmp_path, capsys):
    kern = tmp_path / "k.csv"
    with open(kern, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for a, b in ((0, 100), (50, 150), (300, 400)):  # union: [0,150) and [300,400)
            w.writerow({"Kernel_Name": "k", "Start_Timestamp": a, "End_Timestamp": b})
    copy = tmp_path / "c.csv"
    with open(copy, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Direction", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerow({"Direction": "MEMORY_COPY_DEVICE_TO_DEVICE", "Start_Timestamp": 100, "End_Timestamp": 200})
        w.writerow({"Direction": "MEMORY_COPY_DEVICE_TO_DEVICE", "Start_Timestamp": 250, "End_Timestamp": 350})
        w.writerow({"Direction": "MEMORY_COPY_HOST_TO_DEVICE", "Start_Timestamp": 500, "End_Timestamp": 900})
    frac = bench.summarize_overlap(str(kern), str(copy))
    capsys.readouterr()
    # copy 1: [100,150) under kernels of 100; copy 2: [300,350) of 100 -> 100 of 200
    assert frac == pytest.approx(0.5)
