"""Host-side logic of bench.py (no GPU): the prefill's work count, the counter summary
behind `roofline.traffic`, and the single-GPU guard."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("L,window,sinks", [(1, 4, 2), (7, 4, 2), (40, 8, 4), (40, 8, 0),
                                            (13, 64, 4), (100, 1, 1)])
def test_prefill_pairs_counts_the_attended_keys(L, window, sinks):
    # the flop count of the prefill roofline (4 * d per pair) against the key sets the
    # oracle attends, position by position
    for retrieval in (True, False):
        brute = sum(len(oracle.prefill_rows(t, retrieval, window, sinks)) for t in range(L))
        assert bench.prefill_pairs(L, retrieval, window, sinks) == brute


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_summarize_pmc_scales_by_the_copy(tmp_path):
    # FETCH_SIZE reads half of the copy's 1 MiB (scale 2), WRITE_SIZE all of it (scale 1);
    # each kernel's mean is taken over its dispatches, the largest copy is the calibration
    a = "void rtp::(anonymous namespace)::k_stage_a<512, _Float16>(rtp::StageAParams)"
    b = "void rtp::(anonymous namespace)::k_stage_b<2, 8, _Float16>(rtp::StageBParams)"
    copy = "void at::native::vectorized_elementwise_kernel<neg_kernel>(int)"
    f, w, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _pmc_csv(f, "FETCH_SIZE", [(a, 100.0), (a, 300.0), (b, 40.0), (copy, 512.0), (copy, 2.0)])
    _pmc_csv(w, "WRITE_SIZE", [(a, 50.0), (a, 50.0), (b, 4.0), (copy, 1024.0)])
    bench.summarize_pmc(str(f), str(w), "c4", 2 ** 20, str(out))
    res = json.loads(out.read_text())
    assert res["scale"]["FETCH_SIZE"]["factor"] == 2.0 and res["scale"]["WRITE_SIZE"]["factor"] == 1.0
    ka, kb = res["kernels"]["k_stage_a"], res["kernels"]["k_stage_b"]
    assert ka["FETCH_SIZE"]["bytes_per_launch"] == 200 * 1024 * 2
    assert ka["WRITE_SIZE"]["bytes_per_launch"] == 50 * 1024
    assert ka["bytes_per_launch"] == 200 * 1024 * 2 + 50 * 1024
    assert kb["bytes_per_launch"] == 40 * 1024 * 2 + 4 * 1024
    assert res["source_sha256"] == bench.source_sha256()


def test_summarize_pmc_needs_the_copy_and_every_kernel(tmp_path):
    f, w, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _pmc_csv(f, "FETCH_SIZE", [("k_stage_a", 1.0), ("k_stage_b", 1.0)])  # no copy kernel
    _pmc_csv(w, "WRITE_SIZE", [("k_stage_a", 1.0), ("k_stage_b", 1.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(f), str(w), "c4", 2 ** 20, str(out))
    assert not out.exists()
    copy = "vectorized_elementwise_kernel<neg_kernel>"
    _pmc_csv(f, "FETCH_SIZE", [("k_stage_a", 1.0), (copy, 8.0)])       # no stage-B reading
    _pmc_csv(w, "WRITE_SIZE", [("k_stage_a", 1.0), (copy, 8.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(f), str(w), "c4", 2 ** 20, str(out))
    assert not out.exists()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
    assert not r.stdout.strip()


@pytest.mark.parametrize("argv,msg", [
    (["--context", "4096", "--workload", "c1"], "--context applies to the c3 and c4 workloads"),
    (["--dense", "--topk", "64"], "--dense is the c4 shape alone"),
    (["--dense", "--workload", "c2"], "--dense is the c4 shape alone"),
])
def test_bench_rejects_options_it_cannot_honour(argv, msg):
    # checked before any device work: the run ends with the message and no result line
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and msg in r.stderr
    assert not r.stdout.strip()


def test_context_label():
    import bench
    assert bench.context_label(1 << 20) == "1M"
    assert bench.context_label(65536) == "64K"
    assert bench.context_label(131072) == "128K"
    assert bench.context_label(1 << 24) == "16M"
    assert bench.context_label(3 << 19) == "1.5M"
    assert bench.context_label(4096) == "4K"
    assert bench.context_label(5000) == "5000"


def test_decode_metric_label():
    import bench
    assert bench.decode_metric(1 << 20) == \
        "decode attention us/step and achieved HBM GB/s (% of peak) at 1M context"
    assert bench.decode_metric(65536).endswith("at 64K context")

