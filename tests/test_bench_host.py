"""bench.py's host-side pieces on the CPU: the algorithmic byte counts, the
one-GPU guard, and the oracle baseline's sharded timing run (no GPU)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_algorithmic_bytes_of_the_benchmark_step():
    # 32768 tokens x 2048, 16 q / 8 kv heads of 128, intermediate 6144, bf16: one read and
    # one write of every row (rmsnorm), two of each (add_rmsnorm), q and k in place plus 12
    # position bytes a token (mrope), gate and up read and the product written (swiglu)
    T, H, I, s = 32768, 2048, 6144, 2
    assert bench.algorithmic_bytes("rmsnorm", T, H, I, 16, 8, 128, s) == 2 * T * H * s + H * s
    assert bench.algorithmic_bytes("add_rmsnorm", T, H, I, 16, 8, 128, s) == 4 * T * H * s + H * s
    assert bench.algorithmic_bytes("mrope", T, H, I, 16, 8, 128, s) == 2 * 24 * 128 * s * T + 12 * T
    assert bench.algorithmic_bytes("swiglu", T, H, I, 16, 8, 128, s) == 3 * T * I * s
    assert sum(bench.algorithmic_bytes(op, T, H, I, 16, 8, 128, s)
               for op in ("rmsnorm", "add_rmsnorm", "mrope", "swiglu")) == 2416320512


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_cpu_baseline_shards_cover_the_sample():
    w = W.sweep(dtype="bf16", hidden=256, head_dim=64, tokens=37)
    r = bench.cpu_baseline(w, 37, threads=3)
    assert r["kind"] == "oracle" and r["cores"] == 3 and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["single_thread"]["value"] > 0
    assert set(r["per_op_ms"]) == {"rmsnorm", "add_rmsnorm", "mrope", "swiglu"}
    assert "3 host threads" in r["sample"]
