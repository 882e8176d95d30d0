"""GPU parity of the sliding-window entry points (fa_fwd_window, fa_bwd_window)
against the fp64 oracle with the same window.

Tolerance as for the other parity tests: maximum relative Frobenius error over
O, L, dQ, dK, dV of 1e-4 (fp32 storage) and 2e-2 (bf16 storage); L rows that
are -inf in the oracle (queries whose window holds no key) must be -inf.

Small shapes are compared in full: windows of one key, windows that cut
inside a tile and across tile edges, a window wider than the sequence, the
window without the causal bound, Tq != Tk in both directions, fp32 at both
head dims, and ragged tails.  The article's sliding-window shape (8000 queries
against 8032 keys, 32 query heads over 8 key/value heads, 2080 keys per query)
runs at full size and is compared on one whole (batch, K/V head) group,
sampled query rows of every head (O, L, dQ), and exact invariants.
"""

import numpy as np
import pytest

import oracle.attention as oa
from attention_fa_fwd_05_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def log(msg):
    print(msg, flush=True)


def case(name, B, Hq, Hkv, Tq, Tk, d, dtype, causal, window, seed=21):
    return wl.Workload(name, B, Hq, Hkv, Tq, Tk, d, dtype, causal, seed, window=window)


def run_gpu(fa, w, inp):
    import torch
    q, k, v, do = wl.to_device(inp, w.dtype)
    o, lse = fa.forward(q, k, v, w.causal, w.scale, window=w.window)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, w.causal, w.scale, window=w.window)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in
            (("O", o), ("L", lse), ("dQ", dq), ("dK", dk), ("dV", dv))}


def check(w, errs):
    log(f"{w.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[w.dtype]}
    assert not bad, f"{w.name}: over tolerance {TOL[w.dtype]}: {bad}"


SMALL = [
    case("mha_fp32_T300_d64_causal_w1", 1, 2, 2, 300, 300, 64, "fp32", True, 1),
    case("mha_fp32_T300_d64_causal_w37", 1, 2, 1, 300, 300, 64, "fp32", True, 37),
    case("mha_fp32_T300_d64_causal_w128", 1, 2, 2, 300, 300, 64, "fp32", True, 128),
    case("mha_fp32_T300_d64_causal_w129", 1, 2, 2, 300, 300, 64, "fp32", True, 129),
    case("mha_fp32_T300_d64_causal_w1000", 1, 2, 2, 300, 300, 64, "fp32", True, 1000),
    case("mha_fp32_T1000_d64_causal_w256", 2, 4, 4, 1000, 1000, 64, "fp32", True, 256),
    case("gqa_fp32_T200_d128_causal_w100", 1, 4, 2, 200, 200, 128, "fp32", True, 100),
    case("gqa_fp32_T130_d128_w40", 1, 2, 1, 130, 130, 128, "fp32", False, 40),
    case("gqa_bf16_T300_d128_causal_w64", 2, 4, 2, 300, 300, 128, "bf16", True, 64),
    case("gqa_bf16_T300_d128_causal_w100", 2, 4, 2, 300, 300, 128, "bf16", True, 100),
    case("gqa_bf16_T600_d128_causal_w257", 1, 8, 2, 600, 600, 128, "bf16", True, 257),
    case("mha_bf16_T257_d64_w50", 2, 2, 2, 257, 257, 64, "bf16", False, 50),
    case("gqa_bf16_T300_d64_causal_w3", 1, 8, 1, 300, 300, 64, "bf16", True, 3),
    case("gqa_bf16_Tq200_Tk333_causal_w70", 1, 4, 2, 200, 333, 128, "bf16", True, 70),
    case("gqa_bf16_Tq333_Tk200_causal_w90", 1, 4, 2, 333, 200, 128, "bf16", True, 90),
    case("mha_fp32_Tq40_Tk150_w30", 1, 2, 2, 40, 150, 64, "fp32", False, 30),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_window_parity_full(fa, w):
    log(f"case {w.name}")
    inp = wl.make_inputs(w)
    out = run_gpu(fa, w, inp)
    O, L, dQ, dK, dV = oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale,
                                                     window=w.window)
    errs = {"O": oa.relative_frobenius(out["O"], O),
            "L": oa.relative_frobenius(out["L"], L, finite_only=True),
            "dQ": oa.relative_frobenius(out["dQ"], dQ),
            "dK": oa.relative_frobenius(out["dK"], dK),
            "dV": oa.relative_frobenius(out["dV"], dV)}
    if w.window == 1:
        # One key per row: dQ and dK vanish exactly, so their error is measured
        # against the size of the cancelling terms, scale |dO| |V| |K|.
        assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12
        size = w.scale * np.linalg.norm(inp.do) * np.linalg.norm(inp.v) * np.linalg.norm(inp.k)
        errs["dQ"] = float(np.linalg.norm(out["dQ"]) / size)
        errs["dK"] = float(np.linalg.norm(out["dK"]) / size)
    check(w, errs)


def test_window_zero_is_the_plain_call(fa):
    """window <= 0 through the window entry points equals fa_fwd / fa_bwd bit for bit."""
    import torch
    w = case("gqa_bf16_T300_d128_causal", 1, 4, 2, 300, 300, 128, "bf16", True, 0)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    lib = fa.load_library()
    o1, l1 = fa.forward(q, k, v, True, w.scale)
    o2, l2 = torch.empty_like(q), torch.empty_like(l1)
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.fa_fwd_window(P(q), P(k), P(v), P(o2), P(l2), 1, 4, 2, 300, 300, 128, 1, -5, w.scale, 1,
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_window_sliding_window_shape_sampled(fa):
    w = wl.WORKLOADS["gqa_bf16_T8000x8032_d128_causal_window2080"]
    log(f"case {w.name}: generating inputs")
    inp = wl.make_inputs(w)
    out = run_gpu(fa, w, inp)
    log(f"case {w.name}: GPU done")
    for name, arr in out.items():
        fin = np.isfinite(arr) if name != "L" else ~np.isnan(arr)
        assert fin.all(), f"{name} has non-finite values"
    G = w.G
    b, g = 0, w.Hkv - 1
    ref = oa.group_forward_backward(inp.q, inp.k, inp.v, inp.do, b, g, True, w.scale, window=w.window)
    check(w.with_(name=f"{w.name}[b={b},g={g}]"),
          {"O": oa.relative_frobenius(out["O"][b, g * G:(g + 1) * G], ref["O"]),
           "L": oa.relative_frobenius(out["L"][b, g * G:(g + 1) * G], ref["L"], finite_only=True),
           "dQ": oa.relative_frobenius(out["dQ"][b, g * G:(g + 1) * G], ref["dQ"]),
           "dK": oa.relative_frobenius(out["dK"][b, g], ref["dK"]),
           "dV": oa.relative_frobenius(out["dV"][b, g], ref["dV"])})
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, w.Tq - 1], rng.integers(0, w.Tq, 5)]))
    got = {"O": [], "L": [], "dQ": []}
    exp = {"O": [], "L": [], "dQ": []}
    for h in range(w.Hq):
        q, k, v, do = inp.q[0, h], inp.k[0, h // G], inp.v[0, h // G], inp.do[0, h]
        o, lse, p = oa.head_forward(q[rows], k, v, True, w.scale, rows=rows, Tq=w.Tq, window=w.window)
        dq, _, _ = oa.head_backward(q[rows], k, v, do[rows], o, p, w.scale)
        for n, x in (("O", o), ("L", lse), ("dQ", dq)):
            exp[n].append(x)
            got[n].append(out[n][0, h, rows])
    check(w.with_(name=f"{w.name}[rows]"),
          {n: oa.relative_frobenius(np.stack(got[n]), np.stack(exp[n]), finite_only=(n == "L"))
           for n in got})
    # every query sees at least one key: dK sums to zero over keys, dV to the
    # group's summed cotangent
    dk_sum = out["dK"].astype(np.float64).sum(axis=2)
    assert np.abs(dk_sum).max() <= 2e-2 * np.abs(out["dK"]).sum(axis=2).max()
    do_sum = inp.do.astype(np.float64).reshape(w.B, w.Hkv, G, w.Tq, w.d).sum(axis=(2, 3))
    assert oa.relative_frobenius(out["dV"].astype(np.float64).sum(axis=2), do_sum) <= 2e-2
