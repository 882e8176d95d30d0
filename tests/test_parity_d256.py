"""GPU parity of head dim 256 (bf16) against the fp64 oracle.

The forward runs 4-wave, 128-row workgroups against 64-key tiles of 512-byte
rows (one wave per SIMD holds the 256-wide output accumulator); the dQ pass
4-wave workgroups; the dK/dV pass the 4-wave kernel with each workgroup
forming one half of the columns of dK and dV.

Cases: causal and not, GQA, ragged lengths, Tq != Tk both ways, a sliding
window (forward and backward); the key-split forward (automatic and 3 slices,
32 queries against 1000 keys); a boolean mask (forward and backward);
variable-length and paged batches (forward).  O, L, dQ, dK, dV at relative
Frobenius error 2e-2 and the per-row bound of parity_tools; rows without keys
give O = 0, L = -inf.
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


def case(name, B, Hq, Hkv, Tq, Tk, causal, seed=71, window=0):
    return wl.Workload(name, B, Hq, Hkv, Tq, Tk, 256, "bf16", causal, seed, window=window)


CASES = [
    case("gqa_bf16_T512_d256_causal", 2, 8, 2, 512, 512, True),
    case("mha_bf16_T300_d256", 1, 4, 4, 300, 300, False),
    case("gqa_bf16_Tq200_Tk333_d256_causal", 1, 4, 2, 200, 333, True),
    case("gqa_bf16_Tq333_Tk200_d256_causal", 1, 4, 1, 333, 200, True),
    case("gqa_bf16_T700_d256_causal_w100", 1, 4, 2, 700, 700, True, window=100),
]


def ref_fwd(inp, w, mask=None):
    O, L = oa.attention_forward(inp.q, inp.k, inp.v, w.causal, w.scale, window=w.window, mask=mask)
    return {"O": O, "L": L}


def got_of(o, lse):
    return {"O": o.float().cpu().numpy(), "L": lse.cpu().numpy()}


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_d256_parity(fa, w):
    import torch
    print(f"case {w.name}", flush=True)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    o, lse = fa.forward(q, k, v, w.causal, w.scale, window=w.window)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, w.causal, w.scale, window=w.window)
    torch.cuda.synchronize()
    got = got_of(o, lse)
    got.update({n: t.float().cpu().numpy() for n, t in (("dQ", dq), ("dK", dk), ("dV", dv))})
    ref = dict(zip(("O", "L", "dQ", "dK", "dV"),
                   oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale, window=w.window)))
    check(w.name, "bf16", errors(got, ref))


def test_d256_split_and_mask(fa):
    import torch
    w = case("gqa_bf16_B2_Tq32_Tk1000_d256_causal", 2, 8, 2, 32, 1000, True, 72)
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    ref = ref_fwd(inp, w)
    for ns in (0, 3):
        o, lse = fa.forward_splitk(q, k, v, True, w.scale, nsplit=ns)
        torch.cuda.synchronize()
        check(f"{w.name} nsplit={ns}", "bf16", errors(got_of(o, lse), ref))
    mask = np.random.default_rng(73).random((w.B, w.Tq, w.Tk)) < 0.5
    m = torch.from_numpy(mask).cuda()
    do = wl.to_device(inp, w.dtype)[3]
    o, lse = fa.forward_masked(q, k, v, m, True, w.scale)
    dq, dk, dv = fa.backward_masked(q, k, v, o, lse, do, m, True, w.scale)
    torch.cuda.synchronize()
    got = got_of(o, lse)
    got.update({n: t.float().cpu().numpy() for n, t in (("dQ", dq), ("dK", dk), ("dV", dv))})
    ref = dict(zip(("O", "L", "dQ", "dK", "dV"),
                   oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, True, w.scale, mask=mask)))
    check(f"{w.name} mask", "bf16", errors(got, ref))


def test_d256_varlen_and_paged(fa):
    import torch
    lens = [(1, 1), (100, 300), (0, 40), (200, 129)]
    Hq, Hkv, d = 4, 2, 256
    seqs, refs = [], []
    for b, (tq, tk) in enumerate(lens):
        w = case(f"varlen[{b}]", 1, Hq, Hkv, tq, tk, True, 80 + b)
        inp = wl.make_inputs(w)
        seqs.append(inp)
        refs.append(oa.attention_forward(inp.q, inp.k, inp.v, True, w.scale))
    dev = lambda arrs: torch.from_numpy(np.concatenate([a[0] for a in arrs], axis=1)).to(torch.bfloat16).cuda()
    q, k, v = (dev([getattr(s, n) for s in seqs]) for n in ("q", "k", "v"))
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)).cuda()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)).cuda()
    o, lse = fa.forward_varlen(q, k, v, cu_q, cu_k, 200, 300, True)
    torch.cuda.synchronize()
    ref = {"O": np.concatenate([r[0][0] for r in refs], axis=1), "L": np.concatenate([r[1][0] for r in refs], axis=1)}
    check("d256 varlen", "bf16", errors(got_of(o, lse), ref))
    # paged: 32 queries per sequence against key counts 1 .. 300, page size 128, pages shuffled
    P, B, Tq = 128, 3, 32
    klens = [1, 129, 300]
    rng = np.random.default_rng(74)
    wq = case("paged", B, Hq, Hkv, Tq, 300, True, 75)
    inp = wl.make_inputs(wq)
    pps = 3
    num_pages = B * pps + 2
    order = rng.permutation(num_pages)
    table = order[:B * pps].reshape(B, pps).astype(np.int32)
    kpool = np.zeros((num_pages, Hkv, P, d), np.float32)
    vpool = np.zeros((num_pages, Hkv, P, d), np.float32)
    for b in range(B):
        for s in range(pps):
            kpool[table[b, s]] = inp.k[b][:, s * P:(s + 1) * P] if (s + 1) * P <= 300 else np.pad(
                inp.k[b][:, s * P:300], ((0, 0), (0, (s + 1) * P - 300), (0, 0)))
            vpool[table[b, s]] = inp.v[b][:, s * P:(s + 1) * P] if (s + 1) * P <= 300 else np.pad(
                inp.v[b][:, s * P:300], ((0, 0), (0, (s + 1) * P - 300), (0, 0)))
    tb = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda().contiguous()
    o, lse = fa.forward_paged(tb(inp.q), tb(kpool), tb(vpool), torch.tensor(table).cuda(),
                              torch.tensor(np.array(klens, np.int32)).cuda(), True, wq.scale)
    torch.cuda.synchronize()
    O = np.zeros((B, Hq, Tq, d))
    L = np.zeros((B, Hq, Tq))
    for b in range(B):
        Ob, Lb = oa.attention_forward(inp.q[b:b + 1], inp.k[b:b + 1, :, :klens[b]], inp.v[b:b + 1, :, :klens[b]],
                                      True, wq.scale)
        O[b], L[b] = Ob[0], Lb[0]
    check("d256 paged", "bf16", errors(got_of(o, lse), {"O": O, "L": L}))
