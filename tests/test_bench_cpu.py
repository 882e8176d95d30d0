"""CPU checks of bench.py's host side: the one-GPU guard, the CPU-baseline leg on
a small workload, and the lookup of stored traffic counters."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baseline_times_the_oracle_on_whole_groups():
    from attention_fa_fwd_05_amd import workloads as wl
    w = wl.WORKLOADS["mha_fp32_T128_d64"]
    out = bench.cpu_baseline(w, wl.make_inputs(w), 0.01)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s" and out["value"] > 0
    assert out["cores"] >= 1 and out["host_cores"] >= 1 and out["cpu_model"]
    assert out["sample"].startswith("1 of 1 (batch, K/V head) groups")


def test_source_hash_and_stored_traffic():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    assert bench.stored_traffic("no_such_workload", "fwd_kernel") is None
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    entry = rec["gqa_bf16_T4096_d128_causal"]["dkdv_pair_kernel"]
    got = bench.stored_traffic("gqa_bf16_T4096_d128_causal", "dkdv_pair_kernel")
    # counters are reported only while they were taken on the current kernel sources
    assert got == (entry["bytes_per_launch"] if entry["source_hash"] == h else None)


def test_varlen_decode_batches():
    """The variable-length decode batches of bench.py --varlen-decode: 16 key counts each, from
    a seeded generator; "prefix" holds one 8032-key prefix and 15 counts of 32-600 keys."""
    import numpy as np
    prefix = bench.VARLEN_DECODE["prefix"](np.random.default_rng(20260))
    uniform = bench.VARLEN_DECODE["uniform"](np.random.default_rng(20260))
    assert len(prefix) == len(uniform) == 16
    assert prefix[0] == 8032 and all(32 <= n <= 600 for n in prefix[1:])
    assert all(1000 <= n <= 8032 for n in uniform)
    assert prefix == bench.VARLEN_DECODE["prefix"](np.random.default_rng(20260))
