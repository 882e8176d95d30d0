"""No entry point writes past the end of an output or of its workspace.

Every output and workspace here is the head of a larger buffer whose tail (4 KiB)
is filled with a sentinel byte; after each call the tail must be untouched.
Parity compares only a tensor's own elements, so an access that runs past the
end (a wide store on the last row, a split merge or a packer writing whole
words past the last row) would otherwise go unseen.  Shapes have ragged tails
in both lengths so that the last row of every output sits in a partial tile.
Covered: forward (plain, window, dv != d, fp32 d = 32), backward (same), the
key-split forward and its merge (bf16, fp32 d = 64 and d = 32), variable-length
forward and backward, paged forward (one pass and split) and backward, mask packing, masked
forward (one pass and split) and masked backward (whose workspace holds the
key-major mask copy), also with a window and dv != d, the masked varlen
forward and backward, and the key-split varlen forward (with and without a
mask) with its merge.
"""

import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 0xA5


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


class Guarded:
    """Tensors carved from the heads of sentinel-filled buffers."""

    def __init__(self):
        self.bufs = []

    def tensor(self, name, shape, dtype):
        import torch
        es = torch.empty((), dtype=dtype).element_size()
        nbytes = math.prod(shape) * es
        raw = torch.full((nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.bufs.append((name, raw, nbytes))
        return raw[:nbytes].view(dtype).view(shape)

    def workspace(self, name, nbytes):
        import torch
        raw = torch.full((nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")
        self.bufs.append((name, raw, nbytes))
        return raw[:nbytes]

    def check(self, case):
        import torch
        torch.cuda.synchronize()
        for name, raw, nbytes in self.bufs:
            tail = raw[nbytes:]
            bad = int((tail != SENTINEL).sum())
            assert bad == 0, f"{case}: {bad} bytes past the end of {name} were written"


def rnd(shape, dtype, seed):
    import torch
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g).to(dtype).cuda()


def dt(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float32


DENSE = [
    # name, dtype, B, Hq, Hkv, Tq, Tk, d, dv, causal, window
    ("bf16_d128_causal", "bf16", 2, 4, 2, 200, 333, 128, 128, True, 0),
    ("bf16_d64_window", "bf16", 1, 4, 1, 333, 200, 64, 64, True, 50),
    ("bf16_d128_dv64", "bf16", 1, 4, 2, 131, 257, 128, 64, False, 0),
    ("bf16_d64_dv128", "bf16", 1, 2, 1, 131, 257, 64, 128, True, 0),
    ("fp32_d64", "fp32", 1, 2, 2, 130, 77, 64, 64, False, 0),
    ("bf16_d32_causal", "bf16", 2, 4, 2, 200, 333, 32, 32, True, 0),
    ("fp32_d128_dv64", "fp32", 1, 2, 1, 131, 257, 128, 64, True, 0),
    ("fp32_d32_causal", "fp32", 2, 4, 2, 201, 201, 32, 32, True, 0),
    ("fp32_d128", "fp32", 1, 2, 1, 70, 150, 128, 128, True, 0),
]


@pytest.mark.parametrize("case", DENSE, ids=[c[0] for c in DENSE])
def test_forward_backward_stay_in_bounds(fa, case):
    name, dtn, B, Hq, Hkv, Tq, Tk, d, dv, causal, window = case
    print(f"case {name}", flush=True)
    import torch
    t = dt(dtn)
    q, k, v = rnd((B, Hq, Tq, d), t, 1), rnd((B, Hkv, Tk, d), t, 2), rnd((B, Hkv, Tk, dv), t, 3)
    do = rnd((B, Hq, Tq, dv), t, 4)
    g = Guarded()
    o, lse = g.tensor("O", (B, Hq, Tq, dv), t), g.tensor("L", (B, Hq, Tq), torch.float32)
    fa.forward(q, k, v, causal, out=o, lse=lse, window=window)
    code = fa.FA_DTYPE_BF16 if dtn == "bf16" else fa.FA_DTYPE_F32
    ws = g.workspace("workspace", fa.workspace_bytes(B, Hq, Hkv, Tq, Tk, d, code))
    dq, dk, dvv = g.tensor("dQ", q.shape, t), g.tensor("dK", k.shape, t), g.tensor("dV", v.shape, t)
    fa.backward(q, k, v, o, lse, do, causal, workspace=ws, dq=dq, dk=dk, dv=dvv, window=window)
    g.check(name)
    assert torch.isfinite(o.float()).all() and torch.isfinite(dq.float()).all()


SPLIT = [
    # name, dtype, B, Hq, Hkv, Tq, Tk, d, causal, nsplit
    ("bf16_d128_decode", "bf16", 3, 8, 2, 32, 1000, 128, True, 0),
    ("bf16_d64_rows5", "bf16", 1, 4, 1, 5, 777, 64, False, 3),
    ("fp32_d64_rows7", "fp32", 2, 2, 2, 7, 500, 64, True, 4),
    ("fp32_d32_rows1", "fp32", 1, 2, 1, 1, 300, 32, False, 3),
    ("fp32_d32_rows33", "fp32", 2, 4, 2, 33, 640, 32, True, 0),
]


@pytest.mark.parametrize("case", SPLIT, ids=[c[0] for c in SPLIT])
def test_split_forward_and_merge_stay_in_bounds(fa, case):
    name, dtn, B, Hq, Hkv, Tq, Tk, d, causal, nsplit = case
    print(f"case {name}", flush=True)
    import torch
    t = dt(dtn)
    q, k, v = rnd((B, Hq, Tq, d), t, 5), rnd((B, Hkv, Tk, d), t, 6), rnd((B, Hkv, Tk, d), t, 7)
    code = fa.FA_DTYPE_BF16 if dtn == "bf16" else fa.FA_DTYPE_F32
    g = Guarded()
    ws = g.workspace("split workspace", fa.splitk_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, code, nsplit))
    o, lse = g.tensor("O", (B, Hq, Tq, d), t), g.tensor("L", (B, Hq, Tq), torch.float32)
    fa.forward_splitk(q, k, v, causal, nsplit=nsplit, workspace=ws, out=o, lse=lse)
    g.check(name)
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("dtn,d", [("bf16", 128), ("fp32", 32)])
def test_varlen_stays_in_bounds(fa, dtn, d):
    import torch
    t = dt(dtn)
    lens = [(1, 1), (200, 333), (0, 40), (129, 7), (65, 65)]
    Hq, Hkv = 4, 2
    tq, tk = sum(a for a, _ in lens), sum(b for _, b in lens)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)).cuda()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)).cuda()
    mq, mk = max(a for a, _ in lens), max(b for _, b in lens)
    q, k, v = rnd((Hq, tq, d), t, 8), rnd((Hkv, tk, d), t, 9), rnd((Hkv, tk, d), t, 10)
    do = rnd((Hq, tq, d), t, 11)
    code = fa.FA_DTYPE_BF16 if dtn == "bf16" else fa.FA_DTYPE_F32
    g = Guarded()
    o, lse = g.tensor("O", q.shape, t), g.tensor("L", (Hq, tq), torch.float32)
    fa.forward_varlen(q, k, v, cu_q, cu_k, mq, mk, True, out=o, lse=lse)
    ws = g.workspace("workspace", fa.workspace_bytes(len(lens), Hq, Hkv, mq, mk, d, code))
    dq, dk, dvv = g.tensor("dQ", q.shape, t), g.tensor("dK", k.shape, t), g.tensor("dV", v.shape, t)
    fa.backward_varlen(q, k, v, o, lse, do, cu_q, cu_k, mq, mk, True, workspace=ws, dq=dq, dk=dk, dv=dvv)
    g.check(f"varlen {dtn} d={d}")


@pytest.mark.parametrize("nsplit", [1, 3])
def test_paged_stays_in_bounds(fa, nsplit):
    import torch
    B, Hq, Hkv, Tq, d, P = 3, 8, 2, 33, 128, 128
    lens = [1, 300, 513]
    pps = max((n + P - 1) // P for n in lens)
    num_pages = 3 * pps + 1
    q = rnd((B, Hq, Tq, d), torch.bfloat16, 12)
    kp, vp = rnd((num_pages, Hkv, P, d), torch.bfloat16, 13), rnd((num_pages, Hkv, P, d), torch.bfloat16, 14)
    table = torch.tensor(np.random.default_rng(3).permutation(num_pages)[:B * pps].reshape(B, pps)
                         .astype(np.int32)).cuda()
    seqlens = torch.tensor(np.array(lens, dtype=np.int32)).cuda()
    lib = fa.load_library()
    need = int(lib.fa_fwd_paged_workspace_bytes(B, Hq, Hkv, Tq, pps, P, d, fa.FA_DTYPE_BF16, nsplit))
    g = Guarded()
    ws = g.workspace("paged workspace", need)
    o, lse = g.tensor("O", q.shape, torch.bfloat16), g.tensor("L", (B, Hq, Tq), torch.float32)
    fa.forward_paged(q, kp, vp, table, seqlens, True, nsplit=nsplit, workspace=ws, out=o, lse=lse)
    g.check(f"paged nsplit={nsplit}")


@pytest.mark.parametrize("dtn,d", [("bf16", 128), ("fp32", 32)])
def test_paged_backward_stays_in_bounds(fa, dtn, d):
    import torch
    t = torch.bfloat16 if dtn == "bf16" else torch.float32
    code = fa.FA_DTYPE_BF16 if dtn == "bf16" else fa.FA_DTYPE_F32
    B, Hq, Hkv, Tq, P = 3, 4, 2, 33, 128
    lens = [0, 300, 513]
    pps = max((n + P - 1) // P for n in lens)
    num_pages = 3 * pps + 1
    q, do = rnd((B, Hq, Tq, d), t, 15), rnd((B, Hq, Tq, d), t, 16)
    kp, vp = rnd((num_pages, Hkv, P, d), t, 17), rnd((num_pages, Hkv, P, d), t, 18)
    table = torch.tensor(np.random.default_rng(4).permutation(num_pages)[:B * pps].reshape(B, pps)
                         .astype(np.int32)).cuda()
    seqlens = torch.tensor(np.array(lens, dtype=np.int32)).cuda()
    o, lse = fa.forward_paged(q, kp, vp, table, seqlens, True)
    need = int(fa.load_library().fa_bwd_paged_workspace_bytes(B, Hq, Hkv, Tq, pps, P, d, code))
    g = Guarded()
    ws = g.workspace("paged backward workspace", need)
    dq = g.tensor("dQ", q.shape, t)
    dkp, dvp = g.tensor("dK pages", kp.shape, t), g.tensor("dV pages", vp.shape, t)
    fa.backward_paged(q, kp, vp, o, lse, do, table, seqlens, True, workspace=ws, dq=dq, dk_pages=dkp,
                      dv_pages=dvp)
    g.check(f"paged backward {dtn} d={d}")


@pytest.mark.parametrize("Tq,Tk", [(1, 1), (77, 129), (200, 333), (64, 128)])
def test_mask_pack_stays_in_bounds(fa, Tq, Tk):
    import torch
    mask = torch.from_numpy(np.random.default_rng(Tq).random((2, Tq, Tk)) < 0.5).cuda()
    rw = fa.load_library().fa_mask_row_words(Tk)
    g = Guarded()
    bits = g.tensor("mask bits", (2, Tq, rw), torch.int32)
    fa.pack_mask(mask, out=bits)
    g.check(f"pack {Tq}x{Tk}")


@pytest.mark.parametrize("dtn,d,dvh,window", [("bf16", 128, 128, 0), ("fp32", 64, 64, 0), ("fp32", 32, 32, 0),
                                              ("bf16", 128, 64, 70), ("bf16", 64, 128, 0), ("fp32", 32, 32, 45)])
def test_masked_paths_stay_in_bounds(fa, dtn, d, dvh, window):
    import torch
    t = dt(dtn)
    B, Hq, Hkv, Tq, Tk = 2, 4, 2, 200, 333
    q, k, v = rnd((B, Hq, Tq, d), t, 15), rnd((B, Hkv, Tk, d), t, 16), rnd((B, Hkv, Tk, dvh), t, 17)
    do = rnd((B, Hq, Tq, dvh), t, 18)
    mask = torch.from_numpy(np.random.default_rng(9).random((B, Tq, Tk)) < 0.5).cuda()
    bits = fa.pack_mask(mask)
    lib = fa.load_library()
    code = fa.FA_DTYPE_BF16 if dtn == "bf16" else fa.FA_DTYPE_F32
    stride = Tq * lib.fa_mask_row_words(Tk)
    g = Guarded()
    o, lse = g.tensor("O", (B, Hq, Tq, dvh), t), g.tensor("L", (B, Hq, Tq), torch.float32)
    fa.forward_masked(q, k, v, bits, True, out=o, lse=lse, window=window)
    ws = g.workspace("mask split workspace", int(lib.fa_fwd_mask_splitk_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, dvh,
                                                                                        code, 3)))
    o2, lse2 = g.tensor("O (split)", (B, Hq, Tq, dvh), t), g.tensor("L (split)", (B, Hq, Tq), torch.float32)
    fa.forward_masked(q, k, v, bits, True, out=o2, lse=lse2, nsplit=3, workspace=ws, window=window)
    wsb = g.workspace("mask backward workspace", int(lib.fa_bwd_mask_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, code,
                                                                                      stride)))
    dq, dk, dvv = g.tensor("dQ", q.shape, t), g.tensor("dK", k.shape, t), g.tensor("dV", v.shape, t)
    fa.backward_masked(q, k, v, o, lse, do, bits, True, workspace=wsb, dq=dq, dk=dk, dv=dvv, window=window)
    g.check(f"masked {dtn} d={d} dv={dvh} window={window}")


def test_varlen_masked_paths_stay_in_bounds(fa):
    import torch
    lens = [(1, 1), (120, 333), (0, 40), (77, 0), (200, 150)]
    B, Hq, Hkv, d = len(lens), 4, 2, 128
    mq, mk = max(a for a, _ in lens), max(b for _, b in lens)
    tq, tk = sum(a for a, _ in lens), sum(b for _, b in lens)
    t = torch.bfloat16
    q, k, v, do = rnd((Hq, tq, d), t, 19), rnd((Hkv, tk, d), t, 20), rnd((Hkv, tk, d), t, 21), rnd((Hq, tq, d), t, 22)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)).cuda()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)).cuda()
    mask = torch.from_numpy(np.random.default_rng(10).random((B, mq, mk)) < 0.5).cuda()
    lib = fa.load_library()
    stride = mq * lib.fa_mask_row_words(mk)
    g = Guarded()
    o, lse = g.tensor("O", q.shape, t), g.tensor("L", (Hq, tq), torch.float32)
    fa.forward_varlen_masked(q, k, v, cu_q, cu_k, mq, mk, mask, True, window=60, out=o, lse=lse)
    ws = g.workspace("varlen mask workspace", int(lib.fa_bwd_mask_workspace_bytes(B, Hq, Hkv, mq, mk, d,
                                                                                   fa.FA_DTYPE_BF16, stride)))
    dq, dk, dvv = g.tensor("dQ", q.shape, t), g.tensor("dK", k.shape, t), g.tensor("dV", v.shape, t)
    fa.backward_varlen_masked(q, k, v, o, lse, do, cu_q, cu_k, mq, mk, mask, True, window=60, workspace=ws,
                              dq=dq, dk=dk, dv=dvv)
    g.check("varlen masked")


@pytest.mark.parametrize("dtn,d,masked", [("bf16", 128, False), ("bf16", 128, True), ("fp32", 32, False)])
def test_varlen_split_stays_in_bounds(fa, dtn, d, masked):
    import torch
    t = dt(dtn)
    lens = [(32, 900), (1, 1), (0, 40), (77, 0), (32, 333)]
    B, Hq, Hkv = len(lens), 8, 2
    mq, mk = max(a for a, _ in lens), max(b for _, b in lens)
    tq, tk = sum(a for a, _ in lens), sum(b for _, b in lens)
    q, k, v = rnd((Hq, tq, d), t, 23), rnd((Hkv, tk, d), t, 24), rnd((Hkv, tk, d), t, 25)
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum([a for a, _ in lens])]).astype(np.int32)).cuda()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum([b for _, b in lens])]).astype(np.int32)).cuda()
    mask = torch.from_numpy(np.random.default_rng(11).random((B, mq, mk)) < 0.5).cuda() if masked else None
    lib = fa.load_library()
    code = fa.FA_DTYPE_BF16 if dtn == "bf16" else fa.FA_DTYPE_F32
    g = Guarded()
    o, lse = g.tensor("O", q.shape, t), g.tensor("L", (Hq, tq), torch.float32)
    ws = g.workspace("varlen split workspace",
                     int(lib.fa_fwd_varlen_splitk_workspace_bytes(B, Hq, Hkv, tq, tk, mq, mk, d, code, 3,
                                                                  int(masked))))
    fa.forward_varlen_splitk(q, k, v, cu_q, cu_k, mq, mk, True, window=200, mask=mask, nsplit=3, workspace=ws,
                             out=o, lse=lse)
    g.check(f"varlen split {dtn} d={d} masked={masked}")
    assert torch.isfinite(o.float()).all()
