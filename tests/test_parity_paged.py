"""GPU parity of the paged forward (fa_fwd_paged) against the fp64 oracle run
on each sequence's keys gathered back into order.

Each sequence's K and V (its own key count) are cut into pages that are
scattered over a shuffled pool; the page table maps them back.  Covered:
decode-like blocks (1, 32 and 64 new queries) and a 300-query block against
key counts from 1 to 2100 (tails that end inside a page, a single key, empty
rows when there are fewer keys than queries under end-aligned causal), page
sizes 128 and 256, one pass and split over slices, a window, GQA, bf16 and
fp32.  Tolerance 1e-4 (fp32) / 2e-2 (bf16) relative Frobenius error on O and
L; -inf rows of L must match.
"""

import numpy as np
import pytest

import oracle.attention as oa

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-4, "bf16": 2e-2}


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
    # name, dtype, Hq, Hkv, d, Tq, key counts, page size, causal, window, nsplit
    ("bf16_decode32_p128", "bf16", 8, 2, 128, 32, [32, 200, 1000, 2100], 128, True, 0, 0),
    ("bf16_decode1_p256_split", "bf16", 8, 2, 128, 1, [1, 255, 256, 1500], 256, True, 0, 4),
    ("bf16_q64_p128_onepass", "bf16", 4, 1, 64, 64, [64, 129, 700], 128, True, 0, 1),
    ("bf16_q300_p128_fewkeys", "bf16", 4, 2, 128, 300, [300, 100, 513], 128, True, 0, 0),
    ("bf16_decode32_window", "bf16", 8, 2, 128, 32, [1000, 2100], 128, True, 300, 0),
    ("fp32_decode16_noncausal", "fp32", 4, 2, 64, 16, [77, 640], 128, False, 0, 1),
    ("fp32_d32_decode32_split", "fp32", 4, 2, 32, 32, [32, 300, 900], 128, True, 0, 0),
    ("bf16_d32_decode32_split3", "bf16", 4, 2, 32, 32, [32, 300, 900], 128, True, 0, 3),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_paged_parity(fa, case):
    import torch
    name, dtype, Hq, Hkv, d, Tq, lens, P, causal, window, nsplit = case
    print(f"case {name}", flush=True)
    rng = np.random.default_rng(55)
    B = len(lens)
    pps = max((t + P - 1) // P for t in lens)
    q = rng.standard_normal((B, Hq, Tq, d)).astype(np.float32)
    ks = [rng.standard_normal((Hkv, t, d)).astype(np.float32) for t in lens]
    vs = [rng.standard_normal((Hkv, t, d)).astype(np.float32) for t in lens]
    if dtype == "bf16":
        q = bf16_round(q); ks = [bf16_round(k) for k in ks]; vs = [bf16_round(v) for v in vs]
    num_pages = sum((t + P - 1) // P for t in lens) + 3          # a few unused pages
    order = rng.permutation(num_pages)
    kpool = rng.standard_normal((num_pages, Hkv, P, d)).astype(np.float32)   # garbage fill
    vpool = rng.standard_normal((num_pages, Hkv, P, d)).astype(np.float32)
    table = np.zeros((B, pps), dtype=np.int32)
    nxt = 0
    for b, t in enumerate(lens):
        for p in range((t + P - 1) // P):
            pg = int(order[nxt]); nxt += 1
            table[b, p] = pg
            rows = slice(p * P, min(t, (p + 1) * P))
            n = rows.stop - rows.start
            kpool[pg, :, :n] = ks[b][:, rows]
            vpool[pg, :, :n] = vs[b][:, rows]
    if dtype == "bf16":
        kpool, vpool = bf16_round(kpool), bf16_round(vpool)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda x: torch.tensor(x).to(tdt).cuda().contiguous()
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.forward_paged(dev(q), dev(kpool), dev(vpool), torch.tensor(table).cuda(),
                              torch.tensor(np.array(lens, dtype=np.int32)).cuda(), causal, scale,
                              window=window, nsplit=nsplit)
    torch.cuda.synchronize()
    O = np.zeros((B, Hq, Tq, d)); L = np.zeros((B, Hq, Tq))
    for b in range(B):
        Ob, Lb = oa.attention_forward(q[b:b + 1], ks[b][None], vs[b][None], causal, scale, window=window)
        O[b], L[b] = Ob[0], Lb[0]
    errs = {"O": oa.relative_frobenius(o.float().cpu().numpy(), O),
            "L": oa.relative_frobenius(lse.cpu().numpy(), L, finite_only=True)}
    print(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(e <= TOL[dtype] for e in errs.values()), errs
