#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = the whole path over one batch: forward (O, L) then the backward
(preprocess, dK/dV pass, dQ pass) with a fixed cotangent dO.  Inputs are
seeded synthetic tensors already resident in HBM; outputs and the workspace
are allocated once, outside the timed region.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
    python bench.py --decode        # key-split forward, 32 queries against 8032 keys
    python bench.py --mask 0.5      # forward + backward under a random boolean mask
    python bench.py --varlen-decode prefix   # variable-length key-split forward

Prints one JSON line: whole-step throughput in counted TFLOP/s (4*Tq*Tk*d
forward + 10*Tq*Tk*d backward per query head, halved when causal), the
roofline of the dominant kernel (its counted FLOPs per launch over its average
launch time, from HIP events recorded on the stream the kernels run on), and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s & % bf16 MFMA peak, d=128 T=4096 GQA causal"
# MI355X dense matrix peaks (TFLOP/s): 256 CUs x 2.4 GHz x 4096 bf16 flop/clk/CU.
PEAK = {"bf16": 2516.6, "fp32": 157.3}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ["fa_common.h", "fa_kernels.h", "fa_fwd.hip", "fa_bwd.hip", "fa_dkdv.hip", "fa_paged.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_fa_fwd_05_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if still current."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload, {}).get(kernel)
    if not entry or entry.get("source_hash") != kernel_source_hash():
        return None
    return entry["bytes_per_launch"]


def cpu_baseline(w, inp, budget_s: float):
    """Time the fp64 oracle on whole (batch, K/V head) groups until the budget is used."""
    import numpy as np
    import oracle.attention as oa
    blas, threads = "unknown", None
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            threads = max(p.get("num_threads", 1) for p in pools)
            blas = ", ".join(sorted({f"{p.get('internal_api')} {p.get('version')}" for p in pools}))
    except Exception:
        pass
    host_cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cores = threads if threads else host_cores
    groups = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    rng = np.random.default_rng(0)
    rng.shuffle(groups)
    done, t0 = 0, time.perf_counter()
    for b, g in groups:
        oa.group_forward_backward(inp.q, inp.k, inp.v, inp.do, b, g, w.causal, w.scale, window=w.window)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    elapsed = time.perf_counter() - t0
    from attention_fa_fwd_05_amd import accounting
    if w.window > 0:
        f = sum(accounting.window_flops(1, w.G, w.Tq, w.Tk, w.d, w.causal, w.window)) * done
    else:
        f = (4.0 + 10.0) * w.G * w.Tq * w.Tk * w.d * (0.5 if w.causal else 1.0) * done
    return {"value": f / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of {len(groups)} (batch, K/V head) groups ({done * w.G} query heads), "
                      f"dense fp64 forward+backward, {elapsed:.1f} s",
            "host_cores": int(host_cores), "cpu_model": cpu_model(), "blas": blas}


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def decode_bench(args, fa, accounting, wl):
    """Forward only, split over key slices and merged (fa_fwd_splitk, automatic
    slice count), for few query rows against a long key prefix.  HBM-bound:
    the roofline is the algorithmic bytes (Q, K, V read; O, L written) over the
    launch pair's time against 8 TB/s."""
    import torch
    w = wl.WORKLOADS[args.workload or "gqa_bf16_B16_Tq32_Tk8032_d128_causal"]
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    code = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F32
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Tq, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, fa.splitk_workspace_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, code, 0)),
                     dtype=torch.uint8, device="cuda")

    def step():
        fa.forward_splitk(q, k, v, w.causal, w.scale, window=w.window, workspace=ws, out=o, lse=lse)

    for _ in range(args.warmup):
        step()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for _ in range(args.steps):
        step()
    ev[1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    if w.window > 0:
        f_fwd, _ = accounting.window_flops(w.B, w.Hq, w.Tq, w.Tk, w.d, w.causal, w.window)
    else:
        f_fwd = 4.0 * w.d * w.B * w.Hq * accounting.visible_pairs(w.Tq, w.Tk, w.causal, w.window)
    e = 2 if w.dtype == "bf16" else 4
    algo_bytes = e * (2 * w.B * w.Hq * w.Tq * w.d + 2 * w.B * w.Hkv * w.Tk * w.d) + 4 * w.B * w.Hq * w.Tq
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    out = {"metric": "decode-shaped forward (key-split, merged): TFLOP/s and HBM GB/s",
           "value": round(f_fwd / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": "synthetic (seeded N(0,1) inputs, rounded to bf16)",
           "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Tq": w.Tq, "Tk": w.Tk,
                      "d": w.d, "causal": w.causal, "window": w.window, "nsplit": "auto",
                      "workspace_bytes": ws.numel()},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                        "frac": round(gbs / 8000.0, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": algo_bytes, "avg_launch_ms": round(ms, 4)}}
    print(json.dumps(out), flush=True)
    return 0


def mask_bench(args, fa, accounting, wl):
    """Forward and backward under a boolean mask (fa_fwd_mask, fa_bwd_mask) on
    the headline shape: each batch entry gets its own seeded random mask of the
    given density, on top of the causal bound.  Counted work is 4d (forward)
    and 10d (backward) per visible (query, key) pair, the pairs counted exactly
    from the mask; the backward's roofline is its matrix work (14d per pair:
    8d in the dK/dV pass, 6d in the dQ pass) over the whole fa_bwd_mask call."""
    import numpy as np
    import torch
    w = wl.WORKLOADS[args.workload or wl.HEADLINE]
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    rng = np.random.default_rng(1000 + w.seed)
    mask = rng.random((w.B, w.Tq, w.Tk), dtype=np.float32) < args.mask
    if w.causal:
        mask &= np.arange(w.Tk)[None, :] <= np.arange(w.Tq)[:, None] + (w.Tk - w.Tq)
    pairs = int(mask.sum()) * w.Hq                   # visible pairs over all (entry, query head)
    bits = fa.pack_mask(torch.from_numpy(mask).cuda())
    del mask
    code = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F32
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Tq, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stride = w.Tq * fa.load_library().fa_mask_row_words(w.Tk) if w.B > 1 else 0
    ws = torch.empty(max(1, fa.load_library().fa_bwd_mask_workspace_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d,
                                                                           code, stride)),
                     dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.forward_masked(q, k, v, bits, w.causal, w.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record()
        fa.backward_masked(q, k, v, o, lse, do, bits, w.causal, w.scale, workspace=ws, dq=dq, dk=dk, dv=dv)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_fwd = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    ms_bwd = sum(e[1].elapsed_time(e[2]) for e in events) / args.steps
    f_fwd, f_bwd = 4.0 * w.d * pairs, 10.0 * w.d * pairs
    ms_step = elapsed / args.steps * 1e3
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    peak = PEAK[w.dtype]
    bwd_mm = 14.0 * w.d * pairs / (ms_bwd * 1e-3) / 1e12
    out = {"metric": "attention fwd+bwd under a boolean mask: TFLOP/s on the exactly counted visible pairs",
           "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
           "data": f"synthetic (seeded N(0,1) inputs and cotangent; seeded random mask, density {args.mask})",
           "config": {"workload": f"{w.name}_mask{args.mask}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Tq": w.Tq,
                      "Tk": w.Tk, "d": w.d, "causal": w.causal, "mask_density": args.mask,
                      "visible_pairs": pairs, "parallelism": "single GPU"},
           "pct_peak": round(100.0 * value / peak, 2),
           "roofline": {"bound": "mfma", "kernel": "fa_bwd_mask (dQ with the -D, L2 rows; mask transpose; dK/dV)",
                        "achieved": round(bwd_mm, 2), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(bwd_mm / peak, 4), "traffic": None,
                        "flops_per_launch": 14.0 * w.d * pairs, "avg_launch_ms": round(ms_bwd, 4)},
           "breakdown_ms": {"fwd_mask": round(ms_fwd, 4), "bwd_mask": round(ms_bwd, 4)},
           "fwd_tflops": round(f_fwd / (ms_fwd * 1e-3) / 1e12, 2),
           "bwd_tflops": round(f_bwd / (ms_bwd * 1e-3) / 1e12, 2),
           "workspace_bytes": ws.numel()}
    print(json.dumps(out), flush=True)
    return 0


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling rocprofv3 byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


# Variable-length decode batches: 32 new positions per sequence against key
# counts drawn from a seeded generator (Hq = 32, Hkv = 8, d = 128, bf16,
# end-aligned causal).  "prefix": one 8032-key prefix among 15 sequences of
# 32-600 keys; "uniform": 16 sequences of 1000-8032 keys.
VARLEN_DECODE = {"prefix": lambda rng: [8032] + [int(x) for x in rng.integers(32, 601, 15)],
                 "uniform": lambda rng: [int(x) for x in rng.integers(1000, 8033, 16)]}


def varlen_decode_bench(args, fa, accounting):
    """Forward only over a variable-length batch of decode blocks: the key-split
    call (fa_fwd_varlen_splitk, automatic slice count) timed beside the unsplit
    one (fa_fwd_varlen).  HBM-bound: the roofline is the algorithmic bytes (Q,
    K, V read; O, L written) over the split call's time against 8 TB/s."""
    import numpy as np
    import torch
    rng = np.random.default_rng(20260)
    tk = VARLEN_DECODE[args.varlen_decode](rng)
    Hq, Hkv, d, tq1 = 32, 8, 128, 32
    B, tq = len(tk), [tq1] * len(tk)
    g = torch.Generator().manual_seed(20261)
    mk = lambda *shape: torch.randn(*shape, generator=g).to(torch.bfloat16).cuda()
    q, k, v = mk(Hq, sum(tq), d), mk(Hkv, sum(tk), d), mk(Hkv, sum(tk), d)
    cq = torch.tensor(np.concatenate([[0], np.cumsum(tq)]).astype(np.int32)).cuda()
    ck = torch.tensor(np.concatenate([[0], np.cumsum(tk)]).astype(np.int32)).cuda()
    o, o1 = torch.empty_like(q), torch.empty_like(q)
    lse, lse1 = (torch.empty(Hq, sum(tq), dtype=torch.float32, device="cuda") for _ in range(2))
    lib = fa.load_library()
    need = int(lib.fa_fwd_varlen_splitk_workspace_bytes(B, Hq, Hkv, sum(tq), sum(tk), max(tq), max(tk), d,
                                                        fa.FA_DTYPE_BF16, 0, 0))
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    rows = Hq * sum(tq)
    nsplit = max(1, round(need / (rows * (d + 1) * 4))) if need else 1
    scale = d ** -0.5

    def split():
        fa.forward_varlen_splitk(q, k, v, cq, ck, max(tq), max(tk), True, scale, nsplit=0, workspace=ws, out=o,
                                 lse=lse)

    def unsplit():
        fa.forward_varlen(q, k, v, cq, ck, max(tq), max(tk), True, scale, out=o1, lse=lse1)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for _ in range(args.steps):
            fn()
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / args.steps, (time.perf_counter() - t0) / args.steps * 1e3

    ms_unsplit, _ = timed(unsplit)
    ms, wall_ms = timed(split)
    flops = 4.0 * d * Hq * sum(accounting.visible_pairs(a, b, True) for a, b in zip(tq, tk))
    algo_bytes = 2 * (2 * Hq * sum(tq) * d + 2 * Hkv * sum(tk) * d) + 4 * Hq * sum(tq)
    gbs = algo_bytes / (ms * 1e-3) / 1e9
    out = {"metric": "variable-length decode forward (key-split, merged): TFLOP/s and HBM GB/s",
           "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) inputs rounded to bf16; seeded key counts)",
           "config": {"workload": f"varlen_decode_{args.varlen_decode}", "B": B, "Hq": Hq, "Hkv": Hkv,
                      "Tq_per_seq": tq1, "key_counts": tk, "d": d, "causal": True, "nsplit_auto": nsplit,
                      "workspace_bytes": ws.numel()},
           "unsplit_ms": round(ms_unsplit, 4), "speedup_vs_unsplit": round(ms_unsplit / ms, 2),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                        "frac": round(gbs / 8000.0, 4), "traffic": None,
                        "algorithmic_bytes_per_launch": algo_bytes, "avg_launch_ms": round(ms, 4)}}
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the CPU oracle baseline (0 disables it)")
    ap.add_argument("--decode", action="store_true",
                    help="time the key-split forward on a decode-shaped workload instead")
    ap.add_argument("--mask", type=float, default=0.0, metavar="DENSITY",
                    help="time the boolean-mask forward and backward with a random mask of this density")
    ap.add_argument("--varlen-decode", choices=sorted(VARLEN_DECODE), default=None,
                    help="time the variable-length key-split forward on a batch of decode blocks instead")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="run only a device copy of BYTES bytes (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the attention path here has no multi-GPU mode", file=sys.stderr)
        return 2

    import torch

    import attention_fa_fwd_05_amd as fa
    from attention_fa_fwd_05_amd import accounting
    from attention_fa_fwd_05_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return 0

    fa.load_library()
    if args.decode:
        return decode_bench(args, fa, accounting, wl)
    if args.mask > 0:
        return mask_bench(args, fa, accounting, wl)
    if args.varlen_decode:
        return varlen_decode_bench(args, fa, accounting)
    w = wl.WORKLOADS[args.workload or wl.HEADLINE]
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    code = fa.FA_DTYPE_BF16 if w.dtype == "bf16" else fa.FA_DTYPE_F32
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.Tq, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(1, fa.workspace_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, code)),
                     dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.forward(q, k, v, w.causal, w.scale, out=o, lse=lse, window=w.window)
        if ev is not None:
            ev[1].record()
        # fa_bwd's order: the dQ pass (which also forms every row's -D and L2
        # for the next pass), then the dK/dV pass.
        for i, stage in enumerate((fa.STAGE_DQ, fa.STAGE_DKDV)):
            fa.backward(q, k, v, o, lse, do, w.causal, w.scale, workspace=ws, dq=dq, dk=dk, dv=dv,
                        stages=stage, window=w.window)
            if ev is not None:
                ev[2 + i].record()

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    def avg_ms(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in events) / len(events)

    ms_fwd, ms_dq, ms_dkdv = avg_ms(0, 1), avg_ms(1, 2), avg_ms(2, 3)
    if w.window > 0:
        f_fwd, f_bwd = accounting.window_flops(w.B, w.Hq, w.Tq, w.Tk, w.d, w.causal, w.window)
    else:
        f_fwd, f_bwd = accounting.flops(w.B, w.Hq, w.Tq, w.Tk, w.d, w.causal)
    ms_step = elapsed / args.steps * 1e3
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    peak = PEAK[w.dtype]
    # Each kernel's own matrix work per visible (query, key) pair: forward 4d
    # (S, PV), dK/dV pass 8d (S, dP, dV, dK), dQ pass 6d (S, dP, dQ).
    # bf16 runs the dK/dV pass on wave pairs (dkdv_pair_kernel), fp32 on dkdv_kernel.
    kf = accounting.kernel_flops(w.B, w.Hq, w.Tq, w.Tk, w.d, w.causal, w.window)
    dkdv_name = "dkdv_pair_kernel" if w.dtype == "bf16" else "dkdv_kernel"
    kernels = {"fwd_kernel": (kf["fwd_kernel"], ms_fwd), dkdv_name: (kf["dkdv_kernel"], ms_dkdv),
               "dq_kernel": (kf["dq_kernel"], ms_dq)}
    dom = max(kernels, key=lambda n: kernels[n][1])
    dom_flops, dom_ms = kernels[dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    ret = accounting.retained_bytes_recompute(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, w.dtype)
    dense = accounting.retained_bytes_dense(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, w.dtype)
    out = {
        "metric": METRIC if w.name == wl.HEADLINE else
                  f"attention fwd+bwd TFLOP/s & % {w.dtype} MFMA peak ({w.name})",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs and cotangent, rounded to bf16)" if w.dtype == "bf16"
                else "synthetic (seeded N(0,1) inputs and cotangent)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Tq": w.Tq, "Tk": w.Tk,
                   "d": w.d, "causal": w.causal, "window": w.window, "scale": w.scale,
                   "parallelism": "single GPU"},
        "pct_peak": round(100.0 * value / peak, 2),
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": stored_traffic(w.name, dom),
                     "flops_per_launch": dom_flops, "avg_launch_ms": round(dom_ms, 4)},
        "breakdown_ms": {"fwd_kernel": round(ms_fwd, 4), "dq_kernel": round(ms_dq, 4),
                         dkdv_name: round(ms_dkdv, 4)},
        "breakdown_note": "the dQ pass runs first and also forms every query row's -D and log2-domain L "
                          "for the dK/dV pass (no separate preprocessing pass)",
        "fwd_tflops": round(f_fwd / (ms_fwd * 1e-3) / 1e12, 2),
        "bwd_tflops": round(f_bwd / ((ms_dkdv + ms_dq) * 1e-3) / 1e12, 2),
        "fwd_pct_peak": round(100.0 * f_fwd / (ms_fwd * 1e-3) / 1e12 / peak, 2),
        "bwd_pct_peak": round(100.0 * f_bwd / ((ms_dkdv + ms_dq) * 1e-3) / 1e12 / peak, 2),
        "retained_bytes": {"recompute_qkvoL": ret, "dense_qkv_plus_P": dense,
                           "ratio": round(dense / ret, 2)},
        "workspace_bytes": ws.numel(),
    }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
