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


def test_stream_mix_matches_the_algorithmic_bytes():
    # the calibration kernel moves the op's bytes less the once-per-launch weights and the
    # position/index bytes, in the op's read/write mix
    T, H, I, nq, nkv, D = 32768, 2048, 6144, 16, 8, 128
    for s in (2, 4):
        for op, extra in (("rmsnorm", H * s), ("add_rmsnorm", H * s), ("mrope", 12 * T),
                          ("swiglu", 0), ("layernorm", 2 * H * s), ("add_layernorm", 2 * H * s),
                          ("mrope_kv_append", 20 * T)):
            nr, nw, nb = bench.stream_mix(op, T, H, I, nq, nkv, D, s)
            assert (nr + nw) * nb + extra == bench.algorithmic_bytes(op, T, H, I, nq, nkv, D, s), op


def test_rotation_covers_a_gibibyte():
    for nbytes in (1, 16 << 20, 100_000_000, 1 << 30, 5 << 30):
        nb = bench.rotation(nbytes)
        assert nb * nbytes >= 1 << 30 and (nb - 1) * nbytes < 1 << 30


def test_bar_summary_lists_pairs_below_the_bar():
    rec = lambda f, c: {"frac_of_peak": f, "frac_of_ceiling": c, "ceiling_GB_s": 6600.0}
    configs = [{"workload": "a", "rmsnorm": rec(0.79, 0.96), "swiglu": rec(0.82, 0.99)},
               {"workload": "b", "mrope": rec(0.5, 0.9), "mrope_head_dim64": rec(0.81, 0.97)}]
    s = bench.bar_summary(configs)
    assert s["pairs"] == 4 and s["pairs_below_bar"] == 2
    assert {(b["workload"], b["op"]) for b in s["below"]} == {("a", "rmsnorm"), ("b", "mrope")}
    assert s["lowest_frac_of_ceiling"] == {"workload": "b", "op": "mrope", "frac_of_ceiling": 0.9}


def test_config_cases_cover_every_bandwidth_bound_workload():
    names = [n for n, _ in bench.config_cases("cpu")]
    assert names[:2] == ["prefill_bf16", "ragged_bf16"]
    assert {f"sweep_{dt}_h{h}" for dt in ("bf16", "f32") for h in (512, 1024, 1536, 2048, 4096)} \
        == set(names[2:])


def test_row_ceiling_matches_the_norm_rows():
    assert bench.row_ceiling_bytes("rmsnorm", 2048, 2) == 4096
    assert bench.row_ceiling_bytes("add_layernorm", 4096, 4) == 16384
    assert bench.row_ceiling_bytes("add_rmsnorm", 1536, 2) == 3072
    assert bench.row_ceiling_bytes("rmsnorm", 2560, 2) == 0          # 5 KiB rows are not built
    assert bench.row_ceiling_bytes("mrope", 2048, 2) == 0
    assert bench.row_ceiling_bytes("swiglu", 2048, 2) == 0
