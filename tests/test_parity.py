"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance: maximum relative Frobenius error over O, L, dQ, dK, dV of 1e-4 for
fp32 storage and 2e-2 for bf16 storage with fp32 accumulation.  L rows that
are -inf in the oracle must be -inf on the GPU.

Every comparison also bounds the error of each row on its own
(tests/parity_tools.py), so one wrong row cannot hide in a large tensor.

Small and medium workloads are compared in full.  The three large bf16
workloads run at full size in the launch configuration the benchmark times,
and every (batch, K/V head) group is compared with the oracle run on that
group (every output), plus the exact invariants on every output.
"""

import math

import numpy as np
import pytest

import oracle.attention as oa
from attention_fa_fwd_05_amd import workloads as wl
from parity_tools import Accum, errors, log
from parity_tools import check as check_errs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def run_gpu(fa, w, inp):
    import torch
    q, k, v, do = wl.to_device(inp, w.dtype)
    o, lse = fa.forward(q, k, v, w.causal, w.scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, w.causal, w.scale)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in
            (("O", o), ("L", lse), ("dQ", dq), ("dK", dk), ("dV", dv))}


def errors_full(w, inp, out):
    O, L, dQ, dK, dV = oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale)
    return errors(out, {"O": O, "L": L, "dQ": dQ, "dK": dK, "dV": dV})


def check(w, errs):
    check_errs(w.name, w.dtype, errs)


def custom(name, B, Hq, Hkv, Tq, Tk, d, dtype, causal, seed=7, sigma=1.0):
    return wl.Workload(name, B, Hq, Hkv, Tq, Tk, d, dtype, causal, seed, sigma)


# ------------------------------------------------------------- full comparison

SMALL = [wl.WORKLOADS[n] for n in (
    "mha_fp32_T128_d64", "mha_fp32_T1000_d64", "mha_fp32_T1000_d64_causal",
    "mha_fp32_T1000_d64_sigma3", "mha_fp32_T1000_d64_sigma3_causal")] + [
    # several tiles plus ragged tails, GQA, both head dims, both dtypes
    custom("gqa_bf16_T300_d128", 2, 4, 2, 300, 300, 128, "bf16", False),
    custom("gqa_bf16_T300_d128_causal", 2, 4, 2, 300, 300, 128, "bf16", True),
    custom("gqa_bf16_T300_d64_causal", 1, 8, 1, 300, 300, 64, "bf16", True),
    custom("mha_bf16_T257_d64", 2, 2, 2, 257, 257, 64, "bf16", False),
    custom("gqa_fp32_T200_d128_causal", 1, 4, 2, 200, 200, 128, "fp32", True),
    custom("gqa_fp32_T130_d128", 2, 2, 1, 130, 130, 128, "fp32", False),
    # end-aligned causal with Tq != Tk, including rows that see no key
    custom("gqa_bf16_Tq200_Tk333_causal", 1, 4, 2, 200, 333, 128, "bf16", True),
    custom("gqa_bf16_Tq333_Tk200_causal", 1, 4, 2, 333, 200, 128, "bf16", True),
    custom("mha_fp32_Tq150_Tk40_causal", 1, 2, 2, 150, 40, 64, "fp32", True),
    custom("mha_fp32_Tq40_Tk150", 1, 2, 2, 40, 150, 64, "fp32", False),
    # a single query row
    custom("mha_fp32_Tq1_Tk77_d64", 1, 2, 1, 1, 77, 64, "fp32", False),
    custom("mha_bf16_Tq1_Tk300_d128", 1, 2, 1, 1, 300, 128, "bf16", False),
    # large score spread (frequent running-max rescales) in bf16
    custom("gqa_bf16_T512_d128_sigma3_causal", 1, 4, 1, 512, 512, 128, "bf16", True, 9, 3.0),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_parity_full(fa, w):
    log(f"case {w.name}")
    inp = wl.make_inputs(w)
    out = run_gpu(fa, w, inp)
    check(w, errors_full(w, inp, out))


def test_non_default_scale(fa):
    import torch
    w = custom("gqa_bf16_T200_d128_causal_scale0.3", 1, 4, 2, 200, 200, 128, "bf16", True)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    o, lse = fa.forward(q, k, v, True, 0.3)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, True, 0.3)
    torch.cuda.synchronize()
    names = ("O", "L", "dQ", "dK", "dV")
    got = {n: t.float().cpu().numpy() for n, t in zip(names, (o, lse, dq, dk, dv))}
    ref = dict(zip(names, oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, True, 0.3)))
    check(w, errors(got, ref))


@pytest.mark.parametrize("w", [
    custom("mha_bf16_T1_d128_causal", 1, 2, 2, 1, 1, 128, "bf16", True),
    custom("mha_bf16_Tq70_Tk1_d128", 1, 4, 4, 70, 1, 128, "bf16", False),
    custom("gqa_fp32_Tq70_Tk1_d64", 2, 4, 2, 70, 1, 64, "fp32", False),
], ids=lambda w: w.name)
def test_single_key_closed_form(fa, w):
    """One visible key per row: O = V_0, L = scale q.k_0, dV_0 = sum dO and dQ = dK = 0.

    dQ and dK vanish exactly, so their error is measured against the size of
    the terms that cancel: scale * |dO| |V_0| |K_0| (Frobenius norms).
    """
    inp = wl.make_inputs(w)
    out = run_gpu(fa, w, inp)
    O, L, dQ, dK, dV = oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale)
    assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12
    errs = errors(out, {"O": O, "L": L, "dV": dV})
    size = w.scale * np.linalg.norm(inp.do) * np.linalg.norm(inp.v) * np.linalg.norm(inp.k)
    errs["dQ"] = (float(np.linalg.norm(out["dQ"]) / size), 0.0)
    errs["dK"] = (float(np.linalg.norm(out["dK"]) / size), 0.0)
    check(w, errs)


# ------------------------------------------------------------- empty inputs

@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_no_keys(fa, dtype):
    import torch
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q = torch.randn(1, 4, 70, 64, device="cuda").to(tdt)
    k = torch.empty(1, 2, 0, 64, device="cuda", dtype=tdt)
    v = torch.empty(1, 2, 0, 64, device="cuda", dtype=tdt)
    o, lse = fa.forward(q, k, v, False)
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))
    do = torch.randn_like(q)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, False)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_no_queries(fa, dtype):
    import torch
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    q = torch.empty(2, 4, 0, 128, device="cuda", dtype=tdt)
    k = torch.randn(2, 2, 130, 128, device="cuda").to(tdt)
    v = torch.randn(2, 2, 130, 128, device="cuda").to(tdt)
    o, lse = fa.forward(q, k, v, True)
    assert o.numel() == 0 and lse.numel() == 0
    dk0 = torch.full_like(k, 7.0)
    dv0 = torch.full_like(v, 7.0)
    dq, dk, dv = fa.backward(q, k, v, o, lse, torch.empty_like(q), True, dk=dk0, dv=dv0)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


# ------------------------------------------------------------- large workloads

LARGE = [wl.WORKLOADS[n] for n in ("mha_bf16_T2048_d128_causal", "gqa_bf16_T4096_d128_causal",
                                   "gqa_bf16_T8000x8032_d128")]


@pytest.mark.parametrize("w", LARGE, ids=[w.name for w in LARGE])
def test_parity_large_every_group(fa, w):
    """Every (batch, K/V head) group at full size against the oracle run on that group alone
    (its G query heads' O, L, dQ and the group's dK, dV), accumulated into whole-tensor
    relative Frobenius errors and per-row bounds; then the exact invariants on every output."""
    log(f"case {w.name}: generating inputs")
    inp = wl.make_inputs(w)
    out = run_gpu(fa, w, inp)
    log(f"case {w.name}: GPU done")
    for name, arr in out.items():
        fin = np.isfinite(arr) if name != "L" else ~np.isnan(arr)
        assert fin.all(), f"{name} has non-finite values"
    G = w.G
    acc = Accum()
    for b in range(w.B):
        for g in range(w.Hkv):
            ref = oa.group_forward_backward(inp.q, inp.k, inp.v, inp.do, b, g, w.causal, w.scale)
            got = {"O": out["O"][b, g * G:(g + 1) * G], "L": out["L"][b, g * G:(g + 1) * G],
                   "dQ": out["dQ"][b, g * G:(g + 1) * G], "dK": out["dK"][b, g], "dV": out["dV"][b, g]}
            for n in ("O", "L", "dQ", "dK", "dV"):
                acc.add(n, got[n], ref[n])
                acc.add_rows(n, got[n], ref[n])
    check(w.with_(name=f"{w.name}[all {w.B * w.Hkv} groups]"), acc.result())
    # exact invariants on every output: dK sums to zero over keys; dV sums to the
    # group's summed cotangent (all rows see at least one key here)
    dk_sum = out["dK"].sum(axis=2)
    assert np.abs(dk_sum).max() <= 2e-2 * np.abs(out["dK"]).sum(axis=2).max()
    do_sum = inp.do.astype(np.float64).reshape(w.B, w.Hkv, G, w.Tq, w.d).sum(axis=(2, 3))
    dv_sum = out["dV"].astype(np.float64).sum(axis=2)
    assert oa.relative_frobenius(dv_sum, do_sum) <= 2e-2


# ------------------------------------------------------------- long sequence

def test_parity_long_sequence(fa):
    """32768 causal positions, GQA 8/2: hundreds of key tiles per row and of query
    blocks per key block.  Sampled query rows of every head are compared with the
    oracle for O, L and dQ (a dQ row needs only its own row of P); dK and dV are
    checked everywhere with the exact invariants."""
    w = custom("gqa_bf16_T32768_d128_causal", 1, 8, 2, 32768, 32768, 128, "bf16", True, seed=13)
    log(f"case {w.name}: generating inputs")
    inp = wl.make_inputs(w)
    out = run_gpu(fa, w, inp)
    log(f"case {w.name}: GPU done")
    for name, arr in out.items():
        fin = np.isfinite(arr) if name != "L" else ~np.isnan(arr)
        assert fin.all(), f"{name} has non-finite values"
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, w.Tq - 1], rng.integers(0, w.Tq, 5)]))
    G = w.G
    got = {"O": [], "L": [], "dQ": []}
    ref = {"O": [], "L": [], "dQ": []}
    for h in range(w.Hq):
        q, k, v, do = inp.q[0, h], inp.k[0, h // G], inp.v[0, h // G], inp.do[0, h]
        o, lse, p = oa.head_forward(q[rows], k, v, True, w.scale, rows=rows, Tq=w.Tq)
        dq, _, _ = oa.head_backward(q[rows], k, v, do[rows], o, p, w.scale)
        for n, x in (("O", o), ("L", lse), ("dQ", dq)):
            ref[n].append(x)
        for n in got:
            got[n].append(out[n][0, h, rows])
    check(w.with_(name=f"{w.name}[rows]"),
          errors({n: np.stack(got[n]) for n in got}, {n: np.stack(ref[n]) for n in ref}))
    dk_sum = out["dK"].astype(np.float64).sum(axis=2)
    assert np.abs(dk_sum).max() <= 2e-2 * np.abs(out["dK"]).sum(axis=2).max()
    do_sum = inp.do.astype(np.float64).reshape(w.B, w.Hkv, G, w.Tq, w.d).sum(axis=(2, 3))
    dv_sum = out["dV"].astype(np.float64).sum(axis=2)
    assert oa.relative_frobenius(dv_sum, do_sum) <= 2e-2


# ------------------------------------------------------------- library behaviour

def test_outputs_are_bitwise_reproducible(fa):
    """No kernel uses atomics and every summation order is fixed, so repeated calls give
    identical bits: plain, sliding-window, boolean-mask and key-split paths."""
    import torch
    w = custom("gqa_bf16_T700_d128_causal", 2, 8, 2, 700, 700, 128, "bf16", True)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    mask = torch.from_numpy(np.random.default_rng(5).random((2, 700, 700)) < 0.6).cuda()
    runs = {
        "plain": lambda: (*fa.forward(q, k, v, True), *fa.backward(q, k, v, *fa.forward(q, k, v, True), do, True)),
        "window": lambda: (*fa.forward(q, k, v, True, window=150),
                           *fa.backward(q, k, v, *fa.forward(q, k, v, True, window=150), do, True, window=150)),
        "mask": lambda: (*fa.forward_masked(q, k, v, mask, True),
                         *fa.backward_masked(q, k, v, *fa.forward_masked(q, k, v, mask, True), do, mask, True)),
        "split": lambda: fa.forward_splitk(q[:, :, :32].contiguous(), k, v, True, nsplit=4),
        "mask_split": lambda: fa.forward_masked(q, k, v, mask, True, nsplit=3),
    }
    for name, run in runs.items():
        first = run()
        second = run()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(first, second)):
            assert torch.equal(x, y), f"{name}: output {i} differs between two calls"


def test_library_allocates_nothing(fa):
    import torch
    w = custom("gqa_bf16_T256_d128", 1, 4, 2, 256, 256, 128, "bf16", True)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    o, lse = torch.empty_like(q), torch.empty(1, 4, 256, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.workspace_bytes(1, 4, 2, 256, 256, 128, fa.FA_DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fa.forward(q, k, v, True, out=o, lse=lse)
    fa.backward(q, k, v, o, lse, do, True, workspace=ws, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before


def test_workspace_too_small_is_rejected(fa):
    import torch
    q = torch.randn(1, 2, 64, 128, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 2, 64, 128, device="cuda").to(torch.bfloat16)
    o, lse = fa.forward(q, k, k, False)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    do = torch.randn_like(q)
    with pytest.raises(ValueError, match="needed"):          # the binding refuses first
        fa.backward(q, k, k, o, lse, do, False, workspace=ws)
    dq, dk = torch.empty_like(q), torch.empty_like(k)        # the library refuses on its own
    st = fa.load_library().fa_bwd(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dk.data_ptr(), ws.data_ptr(), 16,
                                  1, 2, 2, 64, 64, 128, 0, 128 ** -0.5, fa.FA_DTYPE_BF16, None)
    assert st == 7


def test_autograd_wrapper_retains_linear_state(fa):
    import torch
    w = custom("mha_bf16_T512_d128", 1, 2, 2, 512, 512, 128, "bf16", True)
    inp = wl.make_inputs(w)
    q, k, v, do = (t.clone().requires_grad_(i < 3) for i, t in enumerate(wl.to_device(inp, w.dtype)))
    saved = []

    def pack(t):
        saved.append((t.data_ptr(), t.numel() * t.element_size()))
        return t

    with torch.autograd.graph.saved_tensors_hooks(pack, lambda t: t):
        o = fa.attention(q, k, v, True)
    (o.float() * do.detach().float()).sum().backward()
    total = sum(b for _, b in dict(saved).items())
    from attention_fa_fwd_05_amd import accounting
    assert total == accounting.retained_bytes_recompute(1, 2, 2, 512, 512, 128, "bf16")
    O, L, dQ, dK, dV = oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, True, w.scale)
    assert oa.relative_frobenius(q.grad.float().cpu().numpy(), dQ) <= 2e-2
