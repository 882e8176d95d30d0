"""GPU parity of the boolean mask combined with a sliding window, with dv != d
and with variable-length batches (fa_fwd_mask, fa_fwd_mask_splitk,
fa_bwd_mask, fa_fwd_varlen_mask, fa_bwd_varlen_mask) against the fp64 oracle
with the same mask, window and lengths.

The chunked-attention article's drafter has full layers under a block mask and
sliding-window layers ("The GQA Expansion Question", "Assumptions and
Uncertainties"); its blocks of new positions have prefixes of their own
lengths ("The Scene").  Cases: random and block-structured masks (shared and
per entry) with windows of 37 to 2080 keys, causal and not, ragged tails, GQA,
bf16 d = 64 and 128, fp32 d = 32 and 64; bf16 (d, dv) = (128, 64) and (64, 128)
under a mask, with a window and split; varlen batches with single rows, empty
sequences, Tq != Tk per sequence, a shared and a per-sequence mask, with and
without a window.  Outputs O, L, dQ, dK, dV: whole-tensor relative Frobenius
error 1e-4 (fp32) / 2e-2 (bf16) and the per-row bound of parity_tools; rows
that see no key give O = 0, L = -inf and dQ = 0.  An all-True mask must give
the unmasked window (and varlen) results bit for bit.
"""

import numpy as np
import pytest

import oracle.attention as oa
from attention_fa_fwd_05_amd import workloads as wl
from parity_tools import check, errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def random_mask(shape, seed, density):
    return np.random.default_rng(seed).random(shape) < density


def block_mask(B, Tq, Tk, seed, blk=128):
    """Per entry: every 128-query block sees a random set of 128-key blocks plus its own
    diagonal block (block-granular, as a drafter's block mask)."""
    rng = np.random.default_rng(seed)
    nb_q, nb_k = -(-Tq // blk), -(-Tk // blk)
    m = np.zeros((B, Tq, Tk), dtype=bool)
    for b in range(B):
        sel = rng.random((nb_q, nb_k)) < 0.5
        for i in range(nb_q):
            sel[i, min(nb_k - 1, (i * blk + Tk - Tq) // blk if Tk >= Tq else i)] = True
        m[b] = np.repeat(np.repeat(sel, blk, 0), blk, 1)[:Tq, :Tk]
    return m


def exact_zero_rows(name, got, ref):
    empty = np.isneginf(ref["L"])
    assert np.isneginf(got["L"][empty]).all(), f"{name}: rows without keys must have L = -inf"
    assert np.all(got["O"][empty] == 0.0), f"{name}: rows without keys must give O = 0"
    if "dQ" in got:
        assert np.all(got["dQ"][empty] == 0.0), f"{name}: rows without keys must give dQ = 0"


FIXED = [
    # name, Workload, mask maker (B, Tq, Tk) -> bool, nsplit of the forward
    ("bf16_d128_causal_window37_per_entry",
     wl.Workload("w", 2, 8, 2, 300, 300, 128, "bf16", True, 11, window=37),
     lambda B, Tq, Tk: random_mask((B, Tq, Tk), 1, 0.5), 1),
    ("bf16_d64_noncausal_window100_shared_ragged",
     wl.Workload("w", 1, 4, 1, 257, 513, 64, "bf16", False, 12, window=100),
     lambda B, Tq, Tk: random_mask((Tq, Tk), 2, 0.4), 1),
    ("fp32_d64_causal_window64", wl.Workload("w", 1, 2, 1, 200, 200, 64, "fp32", True, 13, window=64),
     lambda B, Tq, Tk: random_mask((Tq, Tk), 3, 0.5), 1),
    ("fp32_d32_causal_window50_per_entry", wl.Workload("w", 2, 2, 2, 130, 300, 32, "fp32", True, 14, window=50),
     lambda B, Tq, Tk: random_mask((B, Tq, Tk), 4, 0.6), 1),
    ("bf16_d128_block_mask_window2080", wl.Workload("w", 1, 4, 1, 2600, 2632, 128, "bf16", True, 15, window=2080),
     lambda B, Tq, Tk: block_mask(B, Tq, Tk, 5), 1),
    ("bf16_d128_decode32_window300_split3", wl.Workload("w", 2, 8, 2, 32, 1056, 128, "bf16", True, 16, window=300),
     lambda B, Tq, Tk: random_mask((B, Tq, Tk), 6, 0.5), 3),
    ("bf16_d128_dv64_causal_mask", wl.Workload("w", 1, 4, 2, 200, 333, 128, "bf16", True, 17, dv=64),
     lambda B, Tq, Tk: random_mask((Tq, Tk), 7, 0.5), 1),
    ("bf16_d64_dv128_window90_mask", wl.Workload("w", 2, 4, 1, 300, 300, 64, "bf16", True, 18, window=90, dv=128),
     lambda B, Tq, Tk: random_mask((B, Tq, Tk), 8, 0.5), 1),
    ("bf16_d128_dv64_decode_split4", wl.Workload("w", 1, 8, 2, 16, 1000, 128, "bf16", True, 19, dv=64),
     lambda B, Tq, Tk: random_mask((Tq, Tk), 9, 0.5), 4),
]


@pytest.mark.parametrize("case", FIXED, ids=[c[0] for c in FIXED])
def test_mask_window_dv_parity(fa, case):
    import torch
    name, w, make, nsplit = case
    print(f"case {name}", flush=True)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    mask = make(w.B, w.Tq, w.Tk)
    m = torch.from_numpy(mask).cuda()
    o, lse = fa.forward_masked(q, k, v, m, w.causal, w.scale, nsplit=nsplit, window=w.window)
    got = {"O": o, "L": lse}
    if nsplit == 1:
        got["dQ"], got["dK"], got["dV"] = fa.backward_masked(q, k, v, o, lse, do, m, w.causal, w.scale,
                                                             window=w.window)
    torch.cuda.synchronize()
    got = {n: t.float().cpu().numpy() for n, t in got.items()}
    O, L, dQ, dK, dV = oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale,
                                                     window=w.window, mask=mask)
    ref = {"O": O, "L": L}
    if nsplit == 1:
        ref.update(dQ=dQ, dK=dK, dV=dV)
    exact_zero_rows(name, got, ref)
    check(name, w.dtype, errors(got, ref))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_all_true_mask_with_window_is_the_window_path(fa, dtype, d):
    import torch
    w = wl.Workload("w", 2, 4, 2, 333, 400, d, dtype, True, 21, window=77)
    q, k, v, do = wl.to_device(wl.make_inputs(w), dtype)
    m = torch.ones(w.Tq, w.Tk, dtype=torch.bool, device="cuda")
    o1, l1 = fa.forward_masked(q, k, v, m, True, w.scale, window=w.window)
    o2, l2 = fa.forward(q, k, v, True, w.scale, window=w.window)
    g1 = fa.backward_masked(q, k, v, o1, l1, do, m, True, w.scale, window=w.window)
    g2 = fa.backward(q, k, v, o2, l2, do, True, w.scale, window=w.window)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


VARLEN = [
    # name, Hq, Hkv, d, dtype, causal, window, [(Tq_b, Tk_b)], per-sequence mask
    ("bf16_d128_causal_mix_per_seq", 4, 2, 128, "bf16", True, 0,
     [(1, 1), (63, 63), (300, 300), (0, 0), (129, 200), (32, 1000)], True),
    ("bf16_d128_window50_shared", 4, 1, 128, "bf16", True, 50, [(200, 333), (333, 200), (7, 31), (64, 64)], False),
    ("bf16_d64_noncausal_ragged", 4, 2, 64, "bf16", False, 0, [(200, 333), (40, 0), (0, 40), (64, 1)], True),
    ("fp32_d64_causal_window30", 2, 2, 64, "fp32", True, 30, [(5, 5), (130, 130), (77, 200)], True),
]


def pack_varlen(seqs):
    return np.concatenate(seqs, axis=1)


@pytest.mark.parametrize("case", VARLEN, ids=[c[0] for c in VARLEN])
def test_varlen_mask_parity(fa, case):
    import torch
    name, Hq, Hkv, d, dtype, causal, window, lens, per_seq = case
    print(f"case {name}", flush=True)
    B = len(lens)
    mq, mk = max(a for a, _ in lens), max(b for _, b in lens)
    full = random_mask((B, mq, mk), 31, 0.5) if per_seq else np.broadcast_to(random_mask((mq, mk), 32, 0.5),
                                                                              (B, mq, mk))
    seqs, refs = [], []
    for b, (tq, tk) in enumerate(lens):
        w = wl.Workload(f"{name}[{b}]", 1, Hq, Hkv, tq, tk, d, dtype, causal, 200 + b, window=window)
        inp = wl.make_inputs(w)
        seqs.append(inp)
        refs.append(oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, causal, w.scale, window=window,
                                                  mask=np.ascontiguousarray(full[b, :tq, :tk])))
    scale = 1.0 / np.sqrt(d)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = lambda arrs: torch.from_numpy(pack_varlen([a[0] for a in arrs])).to(tdt).cuda().contiguous()
    q, k, v, do = (dev([getattr(s, n) for s in seqs]) for n in ("q", "k", "v", "do"))
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)).cuda()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)).cuda()
    mask = torch.from_numpy(np.array(full if per_seq else full[0])).cuda()
    o, lse = fa.forward_varlen_masked(q, k, v, cu_q, cu_k, mq, mk, mask, causal, scale, window=window)
    dq, dk, dv = fa.backward_varlen_masked(q, k, v, o, lse, do, cu_q, cu_k, mq, mk, mask, causal, scale,
                                           window=window)
    torch.cuda.synchronize()
    got = {"O": o, "L": lse, "dQ": dq, "dK": dk, "dV": dv}
    got = {n: t.float().cpu().numpy() for n, t in got.items()}
    ref = {"O": pack_varlen([r[0][0] for r in refs]), "L": np.concatenate([r[1][0] for r in refs], axis=1),
           "dQ": pack_varlen([r[2][0] for r in refs]), "dK": pack_varlen([r[3][0] for r in refs]),
           "dV": pack_varlen([r[4][0] for r in refs])}
    exact_zero_rows(name, got, ref)
    check(name, dtype, errors(got, ref))


def test_all_true_varlen_mask_is_the_varlen_path(fa):
    import torch
    lens = [(100, 100), (0, 5), (37, 300), (64, 64)]
    B, Hq, Hkv, d = len(lens), 4, 2, 128
    mq, mk = 100, 300
    rng = np.random.default_rng(41)
    tq, tk = sum(a for a, _ in lens), sum(b for _, b in lens)
    mk_t = lambda *s: torch.from_numpy(rng.standard_normal(s).astype(np.float32)).to(torch.bfloat16).cuda()
    q, k, v, do = mk_t(Hq, tq, d), mk_t(Hkv, tk, d), mk_t(Hkv, tk, d), mk_t(Hq, tq, d)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)).cuda()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)).cuda()
    m = torch.ones(mq, mk, dtype=torch.bool, device="cuda")
    o1, l1 = fa.forward_varlen_masked(q, k, v, cu_q, cu_k, mq, mk, m, True, window=40)
    o2, l2 = fa.forward_varlen(q, k, v, cu_q, cu_k, mq, mk, True, window=40)
    g1 = fa.backward_varlen_masked(q, k, v, o1, l1, do, cu_q, cu_k, mq, mk, m, True, window=40)
    g2 = fa.backward_varlen(q, k, v, o2, l2, do, cu_q, cu_k, mq, mk, True, window=40)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
