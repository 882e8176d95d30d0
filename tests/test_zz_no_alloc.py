"""fa_bwd_noalloc (the backward for callers that cannot allocate) against fa_bwd.

Both run the same kernels; fa_bwd_noalloc only keeps its per-row scratch in the
library's fixed per-device array instead of a caller's workspace, so its
gradients must equal fa_bwd's bit for bit.  Two calls in a row, the second on a
smaller problem, check that the shared scratch left by the first call does not
leak into the second; a third call repeats the first shape.  The call itself
must not change torch's allocated device memory.
"""

import numpy as np
import pytest

from attention_fa_fwd_05_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


CASES = [
    wl.Workload("gqa_bf16_T700_d128_causal", 2, 8, 2, 700, 700, 128, "bf16", True, 31),
    wl.Workload("gqa_bf16_Tq200_Tk333_d64", 1, 4, 1, 200, 333, 64, "bf16", False, 32),
    wl.Workload("gqa_fp32_T130_d64_causal", 1, 2, 1, 130, 130, 64, "fp32", True, 33),
]


def run_pair(fa, w):
    import torch
    print(f"case {w.name}", flush=True)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    o, lse = fa.forward(q, k, v, w.causal, w.scale)
    ref = fa.backward(q, k, v, o, lse, do, w.causal, w.scale)
    dq, dk, dv = torch.full_like(q, 7.0), torch.full_like(k, 7.0), torch.full_like(v, 7.0)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = fa.backward_noalloc(q, k, v, o, lse, do, w.causal, w.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before, "the no-alloc backward changed allocated memory"
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(g, r), f"{w.name}: {name} differs from fa_bwd"
        assert torch.isfinite(g.float()).all()
    return got


def test_noalloc_matches_fa_bwd_on_consecutive_calls(fa):
    first = run_pair(fa, CASES[0])
    run_pair(fa, CASES[1])            # smaller: reads only what it rewrote
    run_pair(fa, CASES[2])
    again = run_pair(fa, CASES[0])
    for a, b in zip(first, again):
        assert np.array_equal(a.float().cpu().numpy(), b.float().cpu().numpy())


def test_noalloc_rejects_a_problem_beyond_its_scratch(fa):
    import torch
    cap = fa.load_library().fa_bwd_noalloc_scratch_bytes()
    heads = cap // 8 // 4096 + 1
    q = torch.empty(1, heads, 4096, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(1, heads, 4096, device="cuda")
    with pytest.raises(fa.FaError) as ei:
        fa.backward_noalloc(q, k, k, q, lse, q, False)
    assert ei.value.status == 12
