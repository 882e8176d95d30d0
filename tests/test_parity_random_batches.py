"""GPU parity of variable-length and paged batches on seeded random configurations,
against the fp64 oracle.

Variable-length (fa_fwd_varlen / fa_bwd_varlen, and the masked pair on a third
of the cases): 16 batches of 1 to 5 sequences, each with its own query and key
counts from 0 to 300 (single rows, empty sides and Tq != Tk both ways occur),
dtype, head dim (32, 64, 128; bf16 256), group size 1, 2 or 4, causal or not,
a window on some, a boolean mask shared by the batch or per sequence on some;
the oracle runs on each sequence alone; each batch's forward also runs split
over a drawn number of key slices (automatic, 2, 3 or 7;
fa_fwd_varlen_splitk, with the batch's mask if any).  Paged (fa_fwd_paged / fa_bwd_paged):
12 pools with shuffled pages, a first page shared by every sequence and pages
no entry references, 1 to 3 sequences with 1 to 96 queries against 0 to 700
keys, page sizes 128 and 256, against oracle/paged.py.  Checked: O, L, dQ, dK,
dV (the gradient pools for paged), whole-tensor relative Frobenius error 1e-4
(fp32) / 2e-2 (bf16) and the per-row bound of parity_tools.
"""

import numpy as np
import pytest

import oracle.attention as oa
import oracle.paged as op
from attention_fa_fwd_05_amd import workloads as wl
from parity_tools import check, errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def bf16_round(x):
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.view(np.float32)


def draw_varlen(i):
    rng = np.random.default_rng(7000 + i)
    dtype = "bf16" if rng.random() < 0.7 else "fp32"
    d = int(rng.choice([32, 64, 128] + ([256] if dtype == "bf16" else [])))
    G = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.integers(1, 3))
    nb = int(rng.integers(1, 6))
    lens = []
    for _ in range(nb):
        tq = int(rng.choice([0, 1, int(rng.integers(2, 301))], p=[0.1, 0.1, 0.8]))
        tk = int(rng.choice([0, 1, int(rng.integers(2, 301))], p=[0.1, 0.1, 0.8]))
        lens.append((tq, tk))
    if max(t for t, _ in lens) == 0:
        lens[0] = (int(rng.integers(1, 200)), lens[0][1])
    if max(t for _, t in lens) == 0:
        lens[0] = (lens[0][0], int(rng.integers(1, 200)))
    return dict(dtype=dtype, d=d, Hq=G * Hkv, Hkv=Hkv, lens=lens, causal=bool(rng.random() < 0.6),
                window=int(rng.integers(1, 200)) if rng.random() < 0.3 else 0,
                masked=bool(rng.random() < 0.33), per_seq=bool(rng.random() < 0.5), seed=7000 + i)


VARLEN = [draw_varlen(i) for i in range(16)]


def vname(c):
    return (f"{c['dtype']}_d{c['d']}_H{c['Hq']}x{c['Hkv']}_{len(c['lens'])}seq{'_causal' if c['causal'] else ''}"
            f"{'_w' + str(c['window']) if c['window'] else ''}{'_mask' if c['masked'] else ''}_s{c['seed']}")


@pytest.mark.parametrize("c", VARLEN, ids=[vname(c) for c in VARLEN])
def test_random_varlen(fa, c):
    import torch
    print(f"case {vname(c)} lens {c['lens']}", flush=True)
    d, dtype, causal, window, lens = c["d"], c["dtype"], c["causal"], c["window"], c["lens"]
    max_q, max_k = max(t for t, _ in lens), max(t for _, t in lens)
    mask = None
    if c["masked"]:
        shape = (len(lens), max_q, max_k) if c["per_seq"] else (max_q, max_k)
        mask = np.random.default_rng(c["seed"] + 1).random(shape) < 0.6
    seqs, refs = [], []
    for b, (tq, tk) in enumerate(lens):
        w = wl.Workload(f"v{b}", 1, c["Hq"], c["Hkv"], tq, tk, d, dtype, causal, c["seed"] * 10 + b, window=window)
        inp = wl.make_inputs(w)
        seqs.append(inp)
        mb = None if mask is None else (mask[b] if mask.ndim == 3 else mask)[:tq, :tk]
        refs.append(oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, causal, w.scale, window=window,
                                                  mask=mb))
    pack = lambda arrs: np.concatenate(arrs, axis=1)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda x: torch.tensor(x, dtype=torch.float32).to(tdt).cuda().contiguous()
    q, k, v, do = (dev(pack([getattr(s, n)[0] for s in seqs])) for n in ("q", "k", "v", "do"))
    cq = torch.tensor(np.concatenate([[0], np.cumsum([t for t, _ in lens])]).astype(np.int32)).cuda()
    ck = torch.tensor(np.concatenate([[0], np.cumsum([t for _, t in lens])]).astype(np.int32)).cuda()
    scale = 1.0 / np.sqrt(d)
    if mask is None:
        o, lse = fa.forward_varlen(q, k, v, cq, ck, max_q, max_k, causal, scale, window=window)
        dq, dk, dv = fa.backward_varlen(q, k, v, o, lse, do, cq, ck, max_q, max_k, causal, scale, window=window)
    else:
        m = torch.from_numpy(mask).cuda()
        o, lse = fa.forward_varlen_masked(q, k, v, cq, ck, max_q, max_k, m, causal, scale, window=window)
        dq, dk, dv = fa.backward_varlen_masked(q, k, v, o, lse, do, cq, ck, max_q, max_k, m, causal, scale,
                                               window=window)
    torch.cuda.synchronize()
    got = {n: t.float().cpu().numpy() for n, t in (("O", o), ("L", lse), ("dQ", dq), ("dK", dk), ("dV", dv))}
    exp = {"O": pack([r[0][0] for r in refs]), "L": np.concatenate([r[1][0] for r in refs], axis=1),
           "dQ": pack([r[2][0] for r in refs]), "dK": pack([r[3][0] for r in refs]),
           "dV": pack([r[4][0] for r in refs])}
    check(vname(c), dtype, errors(got, exp))
    ns = int(np.random.default_rng(c["seed"] + 2).choice([0, 2, 3, 7]))
    o2, lse2 = fa.forward_varlen_splitk(q, k, v, cq, ck, max_q, max_k, causal, scale, window=window,
                                        mask=None if mask is None else torch.from_numpy(mask).cuda(), nsplit=ns)
    torch.cuda.synchronize()
    got2 = {"O": o2.float().cpu().numpy(), "L": lse2.cpu().numpy()}
    check(f"{vname(c)} split nsplit={ns}", dtype, errors(got2, {"O": exp["O"], "L": exp["L"]}))


def draw_paged(i):
    rng = np.random.default_rng(8000 + i)
    dtype = "bf16" if rng.random() < 0.7 else "fp32"
    d = int(rng.choice([32, 64, 128] + ([256] if dtype == "bf16" else [])))
    G = int(rng.choice([1, 2, 4]))
    Hkv = int(rng.integers(1, 3))
    B = int(rng.integers(1, 4))
    return dict(dtype=dtype, d=d, Hq=G * Hkv, Hkv=Hkv, B=B, Tq=int(rng.integers(1, 97)),
                lens=[int(rng.integers(0, 701)) for _ in range(B)], P=int(rng.choice([128, 256])),
                causal=bool(rng.random() < 0.6), window=int(rng.integers(1, 300)) if rng.random() < 0.3 else 0,
                seed=8000 + i)


PAGED = [draw_paged(i) for i in range(12)]


def pname(c):
    return (f"{c['dtype']}_d{c['d']}_H{c['Hq']}x{c['Hkv']}_B{c['B']}_Tq{c['Tq']}_P{c['P']}"
            f"{'_causal' if c['causal'] else ''}{'_w' + str(c['window']) if c['window'] else ''}_s{c['seed']}")


@pytest.mark.parametrize("c", PAGED, ids=[pname(c) for c in PAGED])
def test_random_paged(fa, c):
    import torch
    print(f"case {pname(c)} key counts {c['lens']}", flush=True)
    rng = np.random.default_rng(c["seed"] + 1)
    B, P, d, lens = c["B"], c["P"], c["d"], c["lens"]
    own = [max(1, (n + P - 1) // P) for n in lens]
    pps = max(own)
    num_pages = sum(own) + 2                                   # two pages no entry references
    order = rng.permutation(num_pages)
    table = np.full((B, pps), order[-1], dtype=np.int32)
    nxt = 0
    for b in range(B):
        for s in range(own[b]):
            table[b, s] = order[nxt]
            nxt += 1
    table[1:, 0] = table[0, 0]                                 # a first page shared by every sequence
    q = rng.standard_normal((B, c["Hq"], c["Tq"], d)).astype(np.float32)
    do = rng.standard_normal((B, c["Hq"], c["Tq"], d)).astype(np.float32)
    kp = rng.standard_normal((num_pages, c["Hkv"], P, d)).astype(np.float32)
    vp = rng.standard_normal((num_pages, c["Hkv"], P, d)).astype(np.float32)
    if c["dtype"] == "bf16":
        q, do, kp, vp = (bf16_round(x) for x in (q, do, kp, vp))
    seqlens = np.array(lens, dtype=np.int32)
    scale = 1.0 / np.sqrt(d)
    tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    dev = lambda x: torch.tensor(x).to(tdt).cuda().contiguous()
    Q, KP, VP, DO = dev(q), dev(kp), dev(vp), dev(do)
    tab, sl = torch.tensor(table).cuda(), torch.tensor(seqlens).cuda()
    o, lse = fa.forward_paged(Q, KP, VP, tab, sl, c["causal"], scale, window=c["window"])
    dq, dkp, dvp = fa.backward_paged(Q, KP, VP, o, lse, DO, tab, sl, c["causal"], scale, window=c["window"])
    torch.cuda.synchronize()
    O, L, dQ, dKp, dVp = op.paged_forward_backward(q, kp, vp, table, seqlens, do, c["causal"], scale, c["window"])
    got = {n: t.float().cpu().numpy() for n, t in (("O", o), ("L", lse), ("dQ", dq), ("dK", dkp), ("dV", dvp))}
    check(pname(c), c["dtype"], errors(got, {"O": O, "L": L, "dQ": dQ, "dK": dKp, "dV": dVp}))
