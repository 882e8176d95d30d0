"""GPU parity of a value head dim different from the query/key head dim
(fa_fwd_dv, fa_bwd_dv): (d, dv) = (128, 64) and (64, 128) in bf16 and fp32,
causal and not, GQA, ragged tails, a window, against the fp64 oracle (which
takes V of width dv).  Tolerance 2e-2 (bf16) / 1e-4 (fp32) relative Frobenius
error over O, L, dQ, dK, dV; -inf rows of L must match.
"""

import numpy as np
import pytest

import oracle.attention as oa
from attention_fa_fwd_05_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def case(name, B, Hq, Hkv, Tq, Tk, d, dv, causal, window=0, seed=41, dtype="bf16"):
    return wl.Workload(name, B, Hq, Hkv, Tq, Tk, d, dtype, causal, seed, window=window, dv=dv)


TOL = {"bf16": 2e-2, "fp32": 1e-4}


CASES = [
    case("gqa_bf16_T300_d128_dv64_causal", 2, 4, 2, 300, 300, 128, 64, True),
    case("gqa_bf16_T300_d64_dv128_causal", 2, 4, 2, 300, 300, 64, 128, True),
    case("gqa_bf16_T257_d128_dv64", 1, 4, 1, 257, 257, 128, 64, False),
    case("gqa_bf16_T257_d64_dv128", 1, 4, 1, 257, 257, 64, 128, False),
    case("gqa_bf16_Tq200_Tk333_d128_dv64_causal", 1, 4, 2, 200, 333, 128, 64, True),
    case("gqa_bf16_Tq333_Tk200_d64_dv128_causal", 1, 4, 2, 333, 200, 64, 128, True),
    case("gqa_bf16_T600_d128_dv64_causal_w100", 1, 8, 2, 600, 600, 128, 64, True, 100),
    case("gqa_bf16_T1024_d64_dv128_causal", 2, 8, 2, 1024, 1024, 64, 128, True),
    case("gqa_fp32_T300_d128_dv64_causal", 2, 4, 2, 300, 300, 128, 64, True, dtype="fp32"),
    case("gqa_fp32_T257_d64_dv128", 1, 4, 1, 257, 257, 64, 128, False, dtype="fp32"),
    case("gqa_fp32_Tq200_Tk333_d64_dv128_causal_w70", 1, 4, 2, 200, 333, 64, 128, True, 70, dtype="fp32"),
    case("gqa_fp32_Tq333_Tk200_d128_dv64", 1, 2, 1, 333, 200, 128, 64, False, dtype="fp32"),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_dv_parity(fa, w):
    import torch
    print(f"case {w.name}", flush=True)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    o, lse = fa.forward(q, k, v, w.causal, w.scale, window=w.window)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, w.causal, w.scale, window=w.window)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (w.B, w.Hq, w.Tq, w.dv) and tuple(dv.shape) == (w.B, w.Hkv, w.Tk, w.dv)
    O, L, dQ, dK, dV = oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale,
                                                     window=w.window)
    got = {n: t.float().cpu().numpy() for n, t in (("O", o), ("L", lse), ("dQ", dq), ("dK", dk), ("dV", dv))}
    errs = {"O": oa.relative_frobenius(got["O"], O),
            "L": oa.relative_frobenius(got["L"], L, finite_only=True),
            "dQ": oa.relative_frobenius(got["dQ"], dQ),
            "dK": oa.relative_frobenius(got["dK"], dK),
            "dV": oa.relative_frobenius(got["dV"], dV)}
    print(f"{w.name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(e <= TOL[w.dtype] for e in errs.values()), errs


def test_dv_unsupported_pairs_are_rejected(fa):
    import torch
    q = torch.zeros(1, 2, 8, 128, dtype=torch.float32, device="cuda")
    k = torch.zeros(1, 2, 8, 128, dtype=torch.float32, device="cuda")
    v = torch.zeros(1, 2, 8, 32, dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError, match="HEAD_DIM"):
        fa.forward(q, k, v)                        # (128, 32) is not a supported pair
