"""Host-side logic of bench.py: the algorithmic work counts, the counter
summaries (scaling by the calibration reads) and the one-GPU contract."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import make_workload  # noqa: E402


def test_work_counts_closed_form():
    # two sequences, causal s_q = 2: query i sees L - 1 + i keys
    w = make_workload(seqlens=[5, 1], s_q=2, num_heads_q=4, causal=True, seed=1)
    flops, kv, alg = bench.work_counts(w)
    visible = (4 + 5) + (0 + 1)
    assert flops == 2 * 4 * (576 + 512) * visible
    assert kv == (5 + 1) * 1 * 576 * 2
    assert alg == kv + 2 * 2 * 4 * (576 * 2 + 512 * 2 + 4)
    # an e4m3 query halves the q bytes; an fp8 cache halves the cache bytes
    _, _, alg8 = bench.work_counts(w, q_elem=1)
    assert alg - alg8 == 2 * 2 * 4 * 576
    w8 = make_workload(seqlens=[5, 1], num_heads_q=4, kv_dtype="fp8_e4m3fn", seed=1)
    assert bench.work_counts(w8)[1] == 6 * 576


def _counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_pmc_summary_scales_each_kernel_by_its_calibration(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_json", lambda cfg: str(tmp_path / f"decode_c{cfg}_hbm_traffic.json"))
    mib = 256
    # calibrations: the copy's read shows half its bytes, its write all; the
    # LDS-DMA read a quarter (so the decode fetch is scaled by 4, not 2)
    _counters(tmp_path / "cf", [(1, "copy_kernel", "FETCH_SIZE", mib * 1024 / 2)])
    _counters(tmp_path / "cw", [(1, "copy_kernel", "WRITE_SIZE", mib * 1024)])
    _counters(tmp_path / "lf", [(1, "lds_dma_read_kernel", "FETCH_SIZE", mib * 1024 / 4)])
    # two dispatches of each kernel, counters split over two instances
    _counters(tmp_path / "f", [(7, "mla_decode_kernel<...>", "FETCH_SIZE", 100.0),
                               (7, "mla_decode_kernel<...>", "FETCH_SIZE", 100.0),
                               (9, "mla_decode_kernel<...>", "FETCH_SIZE", 300.0),
                               (8, "mla_combine_kernel<...>", "FETCH_SIZE", 10.0),
                               (10, "mla_combine_kernel<...>", "FETCH_SIZE", 30.0)])
    _counters(tmp_path / "w", [(7, "mla_decode_kernel<...>", "WRITE_SIZE", 50.0),
                               (9, "mla_decode_kernel<...>", "WRITE_SIZE", 70.0),
                               (8, "mla_combine_kernel<...>", "WRITE_SIZE", 5.0),
                               (10, "mla_combine_kernel<...>", "WRITE_SIZE", 5.0)])
    bench.pmc_summary(1, str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                      mib, ["cmd"], lds_fetch_dir=str(tmp_path / "lf"))
    rec = json.load(open(tmp_path / "decode_c1_hbm_traffic.json"))
    assert rec["decode_fetch_kib_per_dispatch"] == 250.0        # (200 + 300) / 2 dispatches
    assert rec["fetch_factor"] == 2.0 and rec["lds_dma_fetch_factor"] == 4.0 and rec["write_factor"] == 1.0
    assert rec["decode_fetch_bytes"] == int(250 * 1024 * 4)
    assert rec["decode_write_bytes"] == int(60 * 1024)
    assert rec["combine_fetch_bytes"] == int(20 * 1024 * 2)
    assert rec["combine_write_bytes"] == int(5 * 1024)
    assert rec["hbm_bytes_per_call"] == rec["hbm_bytes_per_launch"] + int(20 * 1024 * 2) + int(5 * 1024)
    assert rec["decode_source_hash"] == bench.decode_source_hash()
    assert os.path.exists(tmp_path / "decode_c1_hbm_traffic.md")


def test_measured_traffic_needs_the_current_sources(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    monkeypatch.setattr(bench, "traffic_json", lambda cfg: str(path))
    path.write_text(json.dumps({"decode_source_hash": bench.decode_source_hash(), "hbm_bytes_per_call": 123}))
    assert bench.measured_traffic(2) == 123
    path.write_text(json.dumps({"decode_source_hash": "stale", "hbm_bytes_per_call": 123}))
    assert bench.measured_traffic(2) is None


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "DECODE_SOURCES", ["a.hip"])
    a.write_text("int f() { return 1; }  // one\n/* block\n comment */\n")
    h0 = bench.decode_source_hash()
    a.write_text("// other words\nint f()   {\n return 1; }\n")
    assert bench.decode_source_hash() == h0
    a.write_text("int f() { return 2; }\n")
    assert bench.decode_source_hash() != h0


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.gpu
def test_bench_line_carries_the_contract_fields(gpu_lib):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "3",
                        "--fwd-iters", "3", "--no-cpu-baseline"], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in rec, k
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 3 and rec["dtype"] == "bf16"
    roof = rec["roofline"]
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in roof, k
    assert roof["bound"] == "hbm" and roof["peak"] == 8000.0 and 0.0 < roof["frac"] < 1.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert rec["config"]["workload"].startswith("standard MLA decode")


@pytest.mark.gpu
def test_bench_line_for_one_gpus_batch_share(gpu_lib):
    """--batch-share N: the line describes the share (B/N sequences) and
    carries no counter traffic (the committed counters are for the whole
    batch)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--batch-share", "8", "--steps", "3",
                        "--warmup", "3", "--fwd-iters", "3", "--no-cpu-baseline"], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    rec = json.loads([l for l in r.stdout.splitlines() if l.strip()][-1])
    assert rec["config"]["batch"] == 8 and rec["config"]["batch_share_of_gpus"] == 8
    assert "share of the batch over 8 GPUs" in rec["config"]["workload"]
    assert rec["roofline"]["traffic"] is None and rec["n_gpus"] == 1
