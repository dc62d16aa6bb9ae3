"""bench.py: its byte accounting and the JSON line it prints.

The byte count is pinned to the per-layer figure of the tiny workload worked out
by hand from the formula (K and V rows of every attended token, q and output,
table entries and lengths, the appended rows read and written); the JSON line is
checked for the fields the benchmark contract names, on a short run of the tiny
workload (GPU)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import get_config  # noqa: E402


def test_algorithmic_bytes_of_the_tiny_workload():
    cfg = get_config("c1a")  # 4 sequences, 12 query / 2 KV heads, D 128, B 16, fp16
    lengths = np.array([5, 16, 37, 64])
    entries = sum(-(-int(n) // 16) for n in lengths)  # 1 + 1 + 3 + 4 blocks
    b = bench.algorithmic_bytes(cfg, lengths, entries)
    kv = 122 * 2 * 2 * 128 * 2      # 122 attended tokens, K and V, 2 heads, 128 dims, 2 bytes
    qo = 2 * 4 * 12 * 128 * 2       # q read + output written, 4 x 12 heads
    meta = 4 * 9 + 4 * 4            # 9 table entries + 4 lengths, int32
    append = 2 * 4 * 2 * 128 * 2 * 2  # new K and V rows of 4 sequences x 2 heads, read + written
    assert b["decode"] == kv + qo + meta == 149_556
    assert b["layer"] == kv + qo + meta + append == 157_748  # about 158 KB per layer


def test_shared_prefix_rows_count_once():
    cfg = get_config("c1a")
    lengths = np.array([5, 16, 37, 64])
    full = bench.algorithmic_bytes(cfg, lengths, 9)
    shared = bench.algorithmic_bytes(cfg, lengths, 9, shared_tokens=10)
    assert full["decode"] - shared["decode"] == 10 * 2 * 2 * 128 * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


@pytest.mark.gpu
def test_bench_line_carries_the_contract_fields():
    print("[gpu] bench.py --config c1a (short run)", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config", "c1a",
                        "--steps", "3", "--warmup", "1", "--cpu-seconds", "1"],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    b = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in b, key
    assert b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1
    assert b["value"] > 0 and b["ms_per_step"] > 0 and b["higher_is_better"] is True
    assert "workload" in b["config"]
    roof = b["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = b["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert b["parity_vs_oracle"]["within_tolerance"] is True
    assert set(cpu["single_thread"]) == {"c1a", "c4"} and cpu["affinity_cpus"] >= cpu["cores"]
    assert b["hbm_read_reference"]["gbps"] > 0
