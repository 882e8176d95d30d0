"""GPU parity of head dim 32 (the measured configuration of "What Ordinary
Autograd Saves: Tiling the Forward Pass Is Only Half the Algorithm", section
"The implementation under test": d = dv = 32, fp32), in fp32 and in bf16 (64-
byte rows, the 4-chunk swizzle; the bf16 dK/dV pass splits each block's Q and
dO loads between its two wave kinds), against the fp64 oracle: O, L, dQ, dK,
dV at relative Frobenius error 1e-4 (fp32) / 2e-2 (bf16), plus the per-row
bound of parity_tools.

Cases: the article's single-head lengths 128, 256, 512 and 1024 (one head,
inputs drawn with the recipe); grouped-query heads with the causal bound; a
ragged length; Tq != Tk both ways; a sliding window; a boolean mask (forward
and backward); a key-split forward; for bf16 also the packed decode-shape
forward (32 queries against 1000 keys).
"""

import numpy as np
import pytest

import oracle.attention as oa
from attention_fa_fwd_05_amd import workloads as wl
from parity_tools import ROW_TOL, row_error

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def log(msg):
    print(msg, flush=True)


def case(name, B, Hq, Hkv, Tq, Tk, causal, seed=51, window=0, dtype="fp32"):
    return wl.Workload(name, B, Hq, Hkv, Tq, Tk, 32, dtype, causal, seed, window=window)


CASES = [
    case("mha_fp32_T128_d32", 1, 1, 1, 128, 128, False, 0),
    case("mha_fp32_T256_d32", 1, 1, 1, 256, 256, False, 0),
    case("mha_fp32_T512_d32", 1, 1, 1, 512, 512, False, 0),
    case("mha_fp32_T1024_d32", 1, 1, 1, 1024, 1024, False, 0),
    case("gqa_fp32_T1000_d32_causal", 2, 8, 2, 1000, 1000, True),
    case("gqa_fp32_Tq130_Tk333_d32_causal", 1, 4, 2, 130, 333, True),
    case("gqa_fp32_Tq333_Tk130_d32", 1, 4, 1, 333, 130, False),
    case("gqa_fp32_T300_d32_causal_w50", 1, 4, 2, 300, 300, True, window=50),
    case("mha_bf16_T128_d32", 1, 1, 1, 128, 128, False, 0, dtype="bf16"),
    case("mha_bf16_T1024_d32", 1, 1, 1, 1024, 1024, False, 0, dtype="bf16"),
    case("gqa_bf16_T1000_d32_causal", 2, 8, 2, 1000, 1000, True, dtype="bf16"),
    case("gqa_bf16_Tq130_Tk333_d32_causal", 1, 4, 2, 130, 333, True, dtype="bf16"),
    case("gqa_bf16_Tq333_Tk130_d32", 1, 4, 1, 333, 130, False, dtype="bf16"),
    case("gqa_bf16_T600_d32_causal_w100", 1, 8, 2, 600, 600, True, window=100, dtype="bf16"),
    case("gqa_bf16_T2048_d32_causal", 1, 4, 1, 2048, 2048, True, 54, dtype="bf16"),
]


def errs_of(out, ref):
    return {n: oa.relative_frobenius(out[n], ref[n], finite_only=(n == "L")) for n in ref}


def check(name, errs, dtype="fp32", out=None, ref=None):
    log(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"{name}: over tolerance {TOL[dtype]}: {bad}"
    if out is not None:
        rows = {n: row_error(out[n], ref[n], is_L=(n == "L")) for n in ref}
        bad = {k: v for k, v in rows.items() if not v <= ROW_TOL[dtype]}
        assert not bad, f"{name}: a row over {ROW_TOL[dtype]}: {bad}"


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_d32_parity_full(fa, w):
    import torch
    log(f"case {w.name}")
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    o, lse = fa.forward(q, k, v, w.causal, w.scale, window=w.window)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, w.causal, w.scale, window=w.window)
    torch.cuda.synchronize()
    out = {n: t.float().cpu().numpy() for n, t in (("O", o), ("L", lse), ("dQ", dq), ("dK", dk), ("dV", dv))}
    ref = dict(zip(("O", "L", "dQ", "dK", "dV"),
                   oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale,
                                                 window=w.window)))
    check(w.name, errs_of(out, ref), w.dtype, out, ref)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_d32_mask_and_split(fa, dtype):
    import torch
    w = case(f"gqa_{dtype}_T260_d32_mask", 2, 4, 2, 260, 260, True, 52, dtype=dtype)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    mask = np.random.default_rng(53).random((2, 260, 260)) < 0.5
    m = torch.from_numpy(mask).cuda()
    o, lse = fa.forward_masked(q, k, v, m, True, w.scale)
    dq, dk, dv = fa.backward_masked(q, k, v, o, lse, do, m, True, w.scale)
    o2, l2 = fa.forward_splitk(q, k, v, True, w.scale, nsplit=3)
    torch.cuda.synchronize()
    out = {n: t.float().cpu().numpy() for n, t in (("O", o), ("L", lse), ("dQ", dq), ("dK", dk), ("dV", dv))}
    ref = dict(zip(("O", "L", "dQ", "dK", "dV"),
                   oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, True, w.scale, mask=mask)))
    check(w.name, errs_of(out, ref), dtype, out, ref)
    O, L = oa.attention_forward(inp.q, inp.k, inp.v, True, w.scale)
    check(w.name + " split", {"O": oa.relative_frobenius(o2.float().cpu().numpy(), O),
                              "L": oa.relative_frobenius(l2.cpu().numpy(), L, finite_only=True)}, dtype)


def test_d32_bf16_decode_shape(fa):
    """32 queries per head against 1000 keys: the packed 4-wave decode-shape forward, split."""
    import torch
    w = case("gqa_bf16_B4_Tq32_Tk1000_d32_causal", 4, 8, 2, 32, 1000, True, 55, dtype="bf16")
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    O, L = oa.attention_forward(inp.q, inp.k, inp.v, True, w.scale)
    for ns in (0, 1, 3):
        o, lse = fa.forward_splitk(q, k, v, True, w.scale, nsplit=ns)
        torch.cuda.synchronize()
        check(f"{w.name} nsplit={ns}", {"O": oa.relative_frobenius(o.float().cpu().numpy(), O),
                                        "L": oa.relative_frobenius(lse.cpu().numpy(), L, finite_only=True)},
              "bf16")
