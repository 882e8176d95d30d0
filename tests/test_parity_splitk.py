"""GPU parity of the key-split forward (fa_fwd_splitk) and of the packed
forward (all query heads of a K/V group in one workgroup, used by fa_fwd when
a group's rows fit) against the fp64 oracle.

Shapes are decode-like (1, 32 or 64 new query rows against long key
prefixes, end-aligned causal, as one block of new positions attends to the
prefix plus itself) and a few ordinary ones; slice counts 1, 3, 16 and the
automatic choice; windows; both dtypes and head dims; ragged key ends.
Tolerance: relative Frobenius error 1e-4 (fp32) / 2e-2 (bf16) on O and L;
-inf rows of L must match.
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


def case(name, B, Hq, Hkv, Tq, Tk, d, dtype, causal, window=0, seed=31):
    return wl.Workload(name, B, Hq, Hkv, Tq, Tk, d, dtype, causal, seed, window=window)


CASES = [
    case("gqa_bf16_Tq32_Tk8032_d128_causal", 1, 32, 8, 32, 8032, 128, "bf16", True),
    case("gqa_bf16_Tq1_Tk8032_d128_causal", 2, 8, 2, 1, 8032, 128, "bf16", True),
    case("gqa_bf16_Tq64_Tk1000_d128", 2, 8, 2, 64, 1000, 128, "bf16", False),
    case("gqa_bf16_Tq32_Tk3000_d64_causal_w700", 1, 8, 2, 32, 3000, 64, "bf16", True, 700),
    case("gqa_fp32_Tq32_Tk2049_d64_causal", 1, 4, 1, 32, 2049, 64, "fp32", True),
    case("gqa_fp32_Tq16_Tk999_d128", 1, 4, 2, 16, 999, 128, "fp32", False),
    case("mha_fp32_Tq5_Tk300_d64_causal", 2, 2, 2, 5, 300, 64, "fp32", True),
    case("gqa_bf16_T300_d128_causal", 1, 4, 2, 300, 300, 128, "bf16", True),       # not packed
    case("gqa_bf16_Tq333_Tk200_causal", 1, 4, 2, 333, 200, 128, "bf16", True),     # rows without keys
]


def errs(w, inp, o, lse):
    O, L = oa.attention_forward(inp.q, inp.k, inp.v, w.causal, w.scale, window=w.window)
    return {"O": oa.relative_frobenius(o.float().cpu().numpy(), O),
            "L": oa.relative_frobenius(lse.cpu().numpy(), L, finite_only=True)}


def check(name, dtype, e):
    print(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in e.items()), flush=True)
    assert all(v <= TOL[dtype] for v in e.values()), (name, e)


@pytest.mark.parametrize("nsplit", [0, 1, 3, 16])
@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_splitk_parity(fa, w, nsplit):
    import torch
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    o, lse = fa.forward_splitk(q, k, v, w.causal, w.scale, window=w.window, nsplit=nsplit)
    torch.cuda.synchronize()
    check(f"{w.name}[nsplit={nsplit}]", w.dtype, errs(w, inp, o, lse))


@pytest.mark.parametrize("w", CASES[:7], ids=[w.name for w in CASES[:7]])
def test_packed_forward_parity(fa, w):
    """fa_fwd / fa_fwd_window on the decode shapes take the packed layout."""
    import torch
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    o, lse = fa.forward(q, k, v, w.causal, w.scale, window=w.window)
    torch.cuda.synchronize()
    check(f"{w.name}[packed]", w.dtype, errs(w, inp, o, lse))


def test_splitk_workspace_rules(fa):
    import torch
    w = CASES[0]
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    need = fa.splitk_workspace_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, fa.FA_DTYPE_BF16, 4)
    assert need >= 4 * w.B * w.Hq * w.Tq * (w.d + 1) * 4      # 4 slices of fp32 O and L
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="needed"):          # the binding refuses first
        fa.forward_splitk(q, k, v, True, w.scale, nsplit=4, workspace=small)
    o = torch.empty_like(q)                                  # the library refuses on its own
    lse = torch.empty(w.B, w.Hq, w.Tq, device="cuda")
    st = fa.load_library().fa_fwd_splitk(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                         small.data_ptr(), need - 256, w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, 1, 0,
                                         w.scale, fa.FA_DTYPE_BF16, 4, None)
    assert st == 7
    assert fa.splitk_workspace_bytes(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.d, fa.FA_DTYPE_BF16, 5000) == 0
