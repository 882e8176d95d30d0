"""GPU parity of the boolean-mask forward and backward (fa_mask_pack,
fa_fwd_mask, fa_bwd_mask) against the fp64 oracle with the same mask.

The mask packer is integer work and is compared bit for bit with a packing
written here in numpy.  O, L, dQ, dK and dV are compared with the oracle at
the tolerance of the other parity tests: relative Frobenius error 1e-4 (fp32
storage) and 2e-2 (bf16 storage); rows that the mask leaves without a key
must have L = -inf and O = 0 exactly.

Cases: a mask shared by the batch and one per entry; with and without the
causal bound; ragged tails (Tq, Tk not multiples of the tiles); fp32 at both
head dims (d = 128 uses 64-key tiles); whole rows and whole 128-key blocks
masked; a very sparse mask (most tiles skipped by whole waves); the
prefix-plus-block layout of the chunked-attention article's drafter (32 new
positions per entry, each seeing its own prefix length and its own block);
no keys at all; and the headline shape (4096 x 4096, 32 query heads over 8
K/V heads, causal) on one whole group and sampled rows.  An all-True mask must
reproduce fa_fwd and fa_bwd bit for bit, and the autograd wrapper with a mask
the direct calls.
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


def np_pack(mask):
    """Reference packing of a bool [..., Tk] mask: 4 * ceil(Tk / 128) little-endian words per row."""
    Tk = mask.shape[-1]
    rw = 4 * ((Tk + 127) // 128)
    pad = np.zeros(mask.shape[:-1] + (rw * 32,), dtype=bool)
    pad[..., :Tk] = mask
    return np.packbits(pad, axis=-1, bitorder="little").view("<u4")


@pytest.mark.parametrize("shape", [(37, 300), (5, 128), (3, 1), (2, 129), (2, 3, 1000), (4, 0)])
def test_mask_pack_bit_exact(fa, shape):
    import torch
    m = np.random.default_rng(sum(shape)).random(shape) < 0.5
    bits = fa.pack_mask(torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    got = bits.cpu().numpy().view(np.uint32)
    assert got.shape == np_pack(m).shape
    assert np.array_equal(got, np_pack(m))


def random_mask(shape, seed, density):
    return np.random.default_rng(seed).random(shape) < density


def run(fa, w, mask_np, inp, backward=False):
    import torch
    q, k, v, do = wl.to_device(inp, w.dtype)
    m = torch.from_numpy(mask_np).cuda()
    o, lse = fa.forward_masked(q, k, v, m, w.causal, w.scale)
    out = {"O": o, "L": lse}
    if backward:
        out["dQ"], out["dK"], out["dV"] = fa.backward_masked(q, k, v, o, lse, do, m, w.causal, w.scale)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy() for n, t in out.items()}


def check_all(name, dtype, got, ref):
    errs = {n: oa.relative_frobenius(got[n], ref[n], finite_only=(n == "L")) for n in ref}
    log(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    empty = np.isneginf(ref["L"])
    assert np.all(got["O"][empty] == 0.0), f"{name}: rows without keys must give O = 0"
    if "dQ" in ref:
        assert np.all(got["dQ"][empty] == 0.0), f"{name}: rows without keys must give dQ = 0"
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"{name}: over tolerance {TOL[dtype]}: {bad}"


def check(name, dtype, O, L, Oref, Lref):
    errs = {"O": oa.relative_frobenius(O, Oref), "L": oa.relative_frobenius(L, Lref, finite_only=True)}
    log(f"{name}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    empty = np.isneginf(Lref)
    assert np.all(O[empty] == 0.0), f"{name}: rows without keys must give O = 0"
    bad = {k: v for k, v in errs.items() if not v <= TOL[dtype]}
    assert not bad, f"{name}: over tolerance {TOL[dtype]}: {bad}"


def structured_mask(Tq, Tk, seed):
    m = random_mask((Tq, Tk), seed, 0.7)
    m[::97] = False                     # whole rows without a key
    m[:, 256:384] = False               # a whole 128-key block
    return m


CASES = [
    # name, (B, Hq, Hkv, Tq, Tk, d, dtype, causal), mask maker (B, Tq, Tk) -> bool array
    ("gqa_bf16_T300_d128_shared", (2, 8, 2, 300, 300, 128, "bf16", False),
     lambda B, Tq, Tk: random_mask((Tq, Tk), 1, 0.5)),
    ("gqa_bf16_Tq257_Tk513_d128_causal_per_entry", (2, 4, 1, 257, 513, 128, "bf16", True),
     lambda B, Tq, Tk: random_mask((B, Tq, Tk), 2, 0.3)),
    ("mha_bf16_T1000_d64_rows_and_block_masked", (1, 2, 2, 1000, 1000, 64, "bf16", False),
     lambda B, Tq, Tk: structured_mask(Tq, Tk, 3)),
    ("gqa_fp32_T200_d64_causal", (1, 2, 1, 200, 200, 64, "fp32", True),
     lambda B, Tq, Tk: random_mask((Tq, Tk), 4, 0.5)),
    ("mha_fp32_Tq130_Tk700_d128", (1, 2, 2, 130, 700, 128, "fp32", False),
     lambda B, Tq, Tk: random_mask((B, Tq, Tk), 5, 0.5)),
    ("gqa_bf16_T600_d128_sparse", (1, 4, 2, 600, 600, 128, "bf16", False),
     lambda B, Tq, Tk: random_mask((Tq, Tk), 6, 0.02)),
    ("gqa_fp32_T300_d128_causal_per_entry", (2, 4, 2, 300, 300, 128, "fp32", True),
     lambda B, Tq, Tk: random_mask((B, Tq, Tk), 7, 0.6)),
]


def drafter_mask(B, Tq, Tk, prefixes):
    """Entry b's 32 positions see keys [0, prefix_b) and their own block [Tk - 32, Tk)."""
    m = np.zeros((B, Tq, Tk), dtype=bool)
    for b, p in enumerate(prefixes):
        m[b, :, :p] = True
        m[b, :, Tk - Tq:] = True
    return m


CASES.append(("gqa_bf16_B4_Tq32_Tk1056_d128_drafter_blocks", (4, 32, 8, 32, 1056, 128, "bf16", False),
              lambda B, Tq, Tk: drafter_mask(B, Tq, Tk, [1024, 700, 300, 0])))


@pytest.mark.parametrize("name,shape,maker", CASES, ids=[c[0] for c in CASES])
def test_mask_parity_full(fa, name, shape, maker):
    B, Hq, Hkv, Tq, Tk, d, dtype, causal = shape
    log(f"case {name}")
    w = wl.Workload(name, B, Hq, Hkv, Tq, Tk, d, dtype, causal, 31)
    inp = wl.make_inputs(w)
    mask = maker(B, Tq, Tk)
    got = run(fa, w, mask, inp, backward=True)
    ref = dict(zip(("O", "L", "dQ", "dK", "dV"),
                   oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, causal, w.scale, mask=mask)))
    check_all(name, dtype, got, ref)


def test_mask_without_keys(fa):
    import torch
    w = wl.Workload("gqa_bf16_T64_Tk0", 1, 4, 2, 64, 0, 128, "bf16", False, 3)
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    m = torch.zeros(64, 0, dtype=torch.bool, device="cuda")
    o, lse = fa.forward_masked(q, k, v, m)
    dq, dk, dv = fa.backward_masked(q, k, v, o, lse, torch.ones_like(q), m)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse)) and torch.all(dq == 0)


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("bf16", 64, False), ("fp32", 128, False)])
def test_all_true_mask_is_the_plain_call(fa, dtype, d, causal):
    import torch
    w = wl.Workload("all_true", 2, 4, 2, 333, 333, d, dtype, causal, 12)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    ones = torch.ones(333, 333, dtype=torch.bool, device="cuda")
    o1, l1 = fa.forward(q, k, v, causal, w.scale)
    o2, l2 = fa.forward_masked(q, k, v, ones, causal, w.scale)
    g1 = fa.backward(q, k, v, o1, l1, do, causal, w.scale)
    g2 = fa.backward_masked(q, k, v, o1, l1, do, ones, causal, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_mask_headline_shape_sampled(fa):
    w = wl.WORKLOADS["gqa_bf16_T4096_d128_causal"].with_(B=1)
    log(f"case {w.name} B=1 with a random mask: generating inputs")
    inp = wl.make_inputs(w)
    mask = random_mask((w.Tq, w.Tk), 8, 0.5)
    got = run(fa, w, mask, inp, backward=True)
    log("GPU done")
    O, L = got["O"], got["L"]
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095], rng.integers(0, w.Tq, 6)]))
    for h in (0, 13, 31):
        g = h // w.G
        Oref, Lref, _ = oa.head_forward(inp.q[0, h, rows], inp.k[0, g], inp.v[0, g], True, w.scale, rows=rows,
                                        Tq=w.Tq, mask=mask)
        check(f"{w.name}[h={h}, {len(rows)} rows]", w.dtype, O[0, h, rows], L[0, h, rows], Oref, Lref)
    g = 5
    ref = oa.group_forward_backward(inp.q, inp.k, inp.v, inp.do, 0, g, True, w.scale, mask=mask)
    sl = slice(g * w.G, (g + 1) * w.G)
    check_all(f"{w.name}[b=0, g={g}]", w.dtype,
              {"O": O[0, sl], "L": L[0, sl], "dQ": got["dQ"][0, sl], "dK": got["dK"][0, g], "dV": got["dV"][0, g]},
              ref)


def test_autograd_wrapper_with_mask(fa):
    """attention(..., mask=) runs fa_fwd_mask / fa_bwd_mask: the same values as the direct calls."""
    import torch
    w = wl.Workload("autograd_mask", 2, 4, 2, 200, 260, 64, "bf16", True, 41)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    m = torch.from_numpy(random_mask((2, 200, 260), 42, 0.4)).cuda()
    o_ref, l_ref = fa.forward_masked(q, k, v, m, True, w.scale)
    g_ref = fa.backward_masked(q, k, v, o_ref, l_ref, do, m, True, w.scale)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fa.attention(qa, ka, va, True, w.scale, mask=m)
    o.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    for a, b in zip((qa.grad, ka.grad, va.grad), g_ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("nsplit", [0, 3])
def test_mask_split_forward_drafter_blocks(fa, nsplit):
    """fa_fwd_mask_splitk on the drafter layout: 32 positions per entry against its own prefix."""
    import torch
    w = wl.Workload("gqa_bf16_B4_Tq32_Tk1056_d128_drafter_split", 4, 32, 8, 32, 1056, 128, "bf16", False, 43)
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    mask = drafter_mask(4, 32, 1056, [1024, 700, 300, 0])
    o, lse = fa.forward_masked(q, k, v, torch.from_numpy(mask).cuda(), False, w.scale, nsplit=nsplit)
    torch.cuda.synchronize()
    Oref, Lref = oa.attention_forward(inp.q, inp.k, inp.v, False, w.scale, mask=mask)
    check(f"{w.name}[nsplit={nsplit}]", w.dtype, o.float().cpu().numpy(), lse.cpu().numpy(), Oref, Lref)


def test_mask_split_forward_decode_shape(fa):
    """The 16-block decode shape (32 positions against 8032 keys) under per-entry prefix masks,
    automatic key split."""
    import torch
    w = wl.WORKLOADS["gqa_bf16_B16_Tq32_Tk8032_d128_causal"].with_(causal=False)
    inp = wl.make_inputs(w)
    q, k, v, _ = wl.to_device(inp, w.dtype)
    prefixes = list(np.random.default_rng(44).integers(0, 8001, size=16))
    mask = drafter_mask(16, 32, 8032, prefixes)
    o, lse = fa.forward_masked(q, k, v, torch.from_numpy(mask).cuda(), False, w.scale, nsplit=0)
    torch.cuda.synchronize()
    Oref, Lref = oa.attention_forward(inp.q, inp.k, inp.v, False, w.scale, mask=mask)
    check(f"{w.name} prefix masks, auto split", w.dtype, o.float().cpu().numpy(), lse.cpu().numpy(), Oref, Lref)


def test_mask_with_one_entry_is_shared(fa):
    """A [1, Tq, Tk] mask serves every batch entry, as a [Tq, Tk] one does."""
    import torch
    w = wl.Workload("shared_entry", 3, 4, 2, 150, 270, 64, "bf16", True, 45)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    m2 = torch.from_numpy(random_mask((150, 270), 46, 0.5)).cuda()
    o1, l1 = fa.forward_masked(q, k, v, m2, True, w.scale)
    o2, l2 = fa.forward_masked(q, k, v, m2[None], True, w.scale)
    g1 = fa.backward_masked(q, k, v, o1, l1, do, m2, True, w.scale)
    g2 = fa.backward_masked(q, k, v, o1, l1, do, m2[None], True, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
