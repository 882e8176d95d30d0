"""GPU parity of the backward through a page table (fa_bwd_paged) against the
fp64 page-pool oracle (oracle/paged.py).

Pools are shuffled and hold pages no entry references; the first page of
sequence 0 is shared by every sequence (a common prefix), one case also maps
two slots of one sequence to the same page, and one sequence has no keys.
Covered: decode-like blocks (16, 32 and 64 new queries) and 300-query blocks
against key counts from 0 to 2100 (tails that end inside a page, rows with no
visible key under end-aligned causal), page sizes 128 and 256, a window, GQA,
bf16 d = 32, 64, 128 and 256, fp32 d = 32, 64 and 128.  Checked: dQ and the gradient
pools, whole-tensor relative Frobenius error 1e-4 (fp32) / 2e-2 (bf16) and the
per-row bound of parity_tools; pages no entry references and pool rows no
sequence reads are exactly zero; two calls agree bit for bit.
"""

import numpy as np
import pytest

import oracle.paged as op
from parity_tools import check, errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def bf16_round(x):
    b = x.astype(np.float32).view(np.uint32)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.view(np.float32)


CASES = [
    # name, dtype, Hq, Hkv, d, Tq, key counts, page size, causal, window, repeat a page
    ("bf16_d128_decode32_p128", "bf16", 8, 2, 128, 32, [32, 200, 1000, 2100], 128, True, 0, False),
    ("bf16_d64_q64_p128_noncausal", "bf16", 4, 1, 64, 64, [64, 129, 700], 128, False, 0, True),
    ("bf16_d128_q300_p256_fewkeys", "bf16", 4, 2, 128, 300, [300, 100, 513], 256, True, 0, False),
    ("bf16_d128_decode32_window", "bf16", 8, 2, 128, 32, [1000, 2100], 128, True, 300, False),
    ("fp32_d32_decode32_p128", "fp32", 4, 2, 32, 32, [32, 300, 900], 128, True, 0, True),
    ("fp32_d64_decode16_noncausal", "fp32", 4, 2, 64, 16, [77, 640], 128, False, 0, False),
    ("fp32_d128_q40_empty_seq", "fp32", 2, 1, 128, 40, [0, 129, 257], 128, True, 0, False),
    ("bf16_d32_decode32_p128", "bf16", 4, 2, 32, 32, [32, 300, 900], 128, True, 0, True),
    ("bf16_d256_decode32_p128", "bf16", 4, 2, 256, 32, [32, 300, 600], 128, True, 0, False),
]


def build_case(dtype, Hq, Hkv, d, Tq, lens, P, repeat, seed=61):
    rng = np.random.default_rng(seed)
    B = len(lens)
    own = [max(1, (n + P - 1) // P) for n in lens]
    pps = max(own) + (1 if repeat else 0)
    num_pages = sum(own) + 3                                   # three pages no entry references
    order = rng.permutation(num_pages)
    table = np.full((B, pps), order[-1], dtype=np.int32)       # slots past a sequence: a spare page
    nxt = 0
    for b in range(B):
        for s in range(own[b]):
            table[b, s] = order[nxt]
            nxt += 1
    table[1:, 0] = table[0, 0]                                 # common first page
    lens = list(lens)
    if repeat:                                                 # sequence 1 reads its first page twice
        table[1, own[1]] = table[1, 0]
        lens[1] = min(lens[1], own[1] * P) + P
    q = rng.standard_normal((B, Hq, Tq, d)).astype(np.float32)
    do = rng.standard_normal((B, Hq, Tq, d)).astype(np.float32)
    kp = rng.standard_normal((num_pages, Hkv, P, d)).astype(np.float32)
    vp = rng.standard_normal((num_pages, Hkv, P, d)).astype(np.float32)
    if dtype == "bf16":
        q, do, kp, vp = (bf16_round(x) for x in (q, do, kp, vp))
    return q, kp, vp, table, np.array(lens, dtype=np.int32), do


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_backward_parity(fa, case):
    import torch
    name, dtype, Hq, Hkv, d, Tq, lens, P, causal, window, repeat = case
    print(f"case {name}", flush=True)
    q, kp, vp, table, lens, do = build_case(dtype, Hq, Hkv, d, Tq, lens, P, repeat)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda x: torch.tensor(x).to(tdt).cuda().contiguous()
    scale = 1.0 / np.sqrt(d)
    Q, KP, VP, DO = dev(q), dev(kp), dev(vp), dev(do)
    tab, sl = torch.tensor(table).cuda(), torch.tensor(lens).cuda()
    o, lse = fa.forward_paged(Q, KP, VP, tab, sl, causal, scale, window=window)
    dq, dkp, dvp = fa.backward_paged(Q, KP, VP, o, lse, DO, tab, sl, causal, scale, window=window)
    dq2, dkp2, dvp2 = fa.backward_paged(Q, KP, VP, o, lse, DO, tab, sl, causal, scale, window=window)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dkp, dkp2) and torch.equal(dvp, dvp2), "not reproducible"
    O, L, dQ, dKp, dVp = op.paged_forward_backward(q, kp, vp, table, lens, do, causal, scale, window)
    got = {"dQ": dq.float().cpu().numpy(), "dK": dkp.float().cpu().numpy(), "dV": dvp.float().cpu().numpy()}
    # rows of the pools that no sequence reads: exact zeros
    read = np.zeros(kp.shape[:3], dtype=bool)
    for b, n in enumerate(lens):
        j = np.arange(int(n))
        read[table[b, j // P], :, j % P] = True
    for k in ("dK", "dV"):
        assert not got[k][~read].any(), f"{k}: nonzero rows outside the gathered set"
    check(name, dtype, errors(got, {"dQ": dQ, "dK": dKp, "dV": dVp}))
