"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes the workspace, and rejects bad arguments before any
HIP call (all calls below fail validation, so nothing reaches the device)."""

import ctypes
import math
import os
import re

import pytest

import attention_fa_fwd_05_amd as fa
from attention_fa_fwd_05_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from attention_fa_fwd_05_amd import build
        build.build(verbose=False)
    return fa.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(_binding.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(13):
        s = fa.status_string(code)
        assert s and s != "unknown status"
    assert fa.status_string(99) == "unknown status"
    assert lib.fa_abi_version() >> 16 == 2


def test_head_dim_status_names_every_accepted_dim(lib):
    # the checks accept d = 32, 64, 128 and, in bf16, 256
    s = fa.status_string(4)
    for dim in ("32", "64", "128", "256"):
        assert dim in s, s


def test_workspace_bytes(lib):
    # D and L2 per query row, rows padded to a multiple of 64 per head, 256-byte aligned parts
    rows = 4 * 32 * 4096
    assert fa.workspace_bytes(4, 32, 8, 4096, 4096, 128, fa.FA_DTYPE_BF16) == 2 * rows * 4
    assert fa.workspace_bytes(1, 1, 1, 100, 100, 64, fa.FA_DTYPE_F32) == 512 + 512
    assert fa.workspace_bytes(3, 1, 1, 1, 100, 64, fa.FA_DTYPE_BF16) == 768 + 768
    assert fa.workspace_bytes(1, 1, 1, 0, 5, 64, fa.FA_DTYPE_BF16) == 0
    # invalid arguments -> 0
    assert fa.workspace_bytes(1, 3, 2, 10, 10, 64, fa.FA_DTYPE_BF16) == 0
    assert fa.workspace_bytes(1, 1, 1, 10, 10, 96, fa.FA_DTYPE_BF16) == 0


FAKE = 1 << 20   # aligned, never dereferenced: every call below fails validation first


def fwd(lib, Q=FAKE, K=FAKE, V=FAKE, O=FAKE, L=FAKE, B=1, Hq=2, Hkv=1, Tq=16, Tk=16, d=64,
        causal=0, scale=0.125, dtype=1):
    return lib.fa_fwd(Q, K, V, O, L, B, Hq, Hkv, Tq, Tk, d, causal, scale, dtype, None)


def bwd(lib, ws=FAKE, ws_bytes=1 << 30, Q=FAKE, dQ=FAKE, B=1, Hq=2, Hkv=1, Tq=16, Tk=16, d=64,
        scale=0.125, dtype=1):
    return lib.fa_bwd(Q, FAKE, FAKE, FAKE, FAKE, FAKE, dQ, FAKE, FAKE, ws, ws_bytes,
                      B, Hq, Hkv, Tq, Tk, d, 0, scale, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2), (dict(Tq=-1), 2), (dict(Tk=-5), 2),
    (dict(Hq=3, Hkv=2), 3), (dict(d=96), 4), (dict(d=256, dtype=0), 4), (dict(dtype=7), 5),
    (dict(scale=math.inf), 6), (dict(scale=math.nan), 6),
    (dict(Q=None), 1), (dict(L=None), 1), (dict(V=FAKE + 4), 8), (dict(Tq=1 << 25), 9),
])
def test_fwd_rejects_bad_arguments(lib, kw, status):
    assert fwd(lib, **kw) == status


def test_fwd_null_pointers_allowed_for_empty_tensors(lib):
    # Tq == 0: Q, O, L have no elements; a no-op that touches nothing
    assert fwd(lib, Q=None, O=None, L=None, Tq=0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), 7), (dict(ws_bytes=100), 7), (dict(ws=FAKE + 8), 8),
    (dict(Q=None), 1), (dict(dQ=None), 1), (dict(Hq=4, Hkv=3), 3), (dict(scale=-math.inf), 6),
])
def test_bwd_rejects_bad_arguments(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_bwd_stages_rejects_unknown_bits(lib):
    args = (FAKE,) * 10 + (1 << 30, 1, 2, 1, 16, 16, 64, 0, 0.125, 1)
    assert lib.fa_bwd_stages(*args, 8, None) == 11
    assert lib.fa_bwd_stages(*(args[:2] + (None,) + args[3:]), 2, None) == 1


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _binding.load_library(str(tmp_path / "nope.so"))


def fwd_varlen(lib, cu_q=FAKE, cu_k=FAKE, B=2, Hq=2, Hkv=1, total_q=32, total_k=32, max_q=16, max_k=16,
               d=64, Q=FAKE):
    return lib.fa_fwd_varlen(Q, FAKE, FAKE, FAKE, FAKE, cu_q, cu_k, B, Hq, Hkv, total_q, total_k, max_q,
                             max_k, d, 1, 0, 0.125, 1, None)


@pytest.mark.parametrize("kw,status", [
    (dict(cu_q=None), 1), (dict(cu_k=None), 1), (dict(cu_q=FAKE + 2), 8), (dict(total_q=-1), 2),
    (dict(max_q=40), 2), (dict(max_k=-1), 2), (dict(Hq=3, Hkv=2), 3), (dict(d=80), 4), (dict(Q=None), 1),
])
def test_fwd_varlen_rejects_bad_arguments(lib, kw, status):
    assert fwd_varlen(lib, **kw) == status


def test_bwd_varlen_rejects_missing_workspace(lib):
    args = (FAKE,) * 9 + (None, 0, FAKE, FAKE, 2, 2, 1, 32, 32, 16, 16, 64, 1, 0, 0.125, 1, None)
    assert lib.fa_bwd_varlen(*args) == 7


def test_splitk_rejects_too_many_slices(lib):
    assert lib.fa_fwd_splitk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, 1, 2, 1, 16, 16, 64, 1, 0, 0.125, 1,
                             5000, None) == 9
    assert lib.fa_fwd_splitk(FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, 1, 2, 1, 16, 16, 64, 1, 0, 0.125, 1,
                             4, None) == 7


@pytest.mark.parametrize("d,dv,dtype", [(128, 96, 1), (128, 256, 1), (32, 64, 0), (64, 32, 0), (96, 64, 1)])
def test_dv_rejects_unsupported_pairs(lib, d, dv, dtype):
    assert lib.fa_fwd_dv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 16, 16, d, dv, 1, 0, 0.125, dtype, None) == 4
    assert lib.fa_bwd_dv(*(FAKE,) * 10, 1 << 30, 1, 2, 1, 16, 16, d, dv, 1, 0, 0.125, dtype, 7, None) == 4


@pytest.mark.parametrize("kw,status", [
    (dict(P=100), 2), (dict(P=0), 2), (dict(pps=0), 2), (dict(npages=0), 2), (dict(table=None), 1),
    (dict(seqlens=None), 1), (dict(table=FAKE + 2), 8), (dict(d=80), 4),
])
def test_fwd_paged_rejects_bad_arguments(lib, kw, status):
    a = dict(table=FAKE, seqlens=FAKE, pps=4, P=128, npages=8, d=64)
    a.update(kw)
    assert lib.fa_fwd_paged(FAKE, FAKE, FAKE, FAKE, FAKE, a["table"], a["seqlens"], 2, 2, 1, 16, a["pps"], a["P"],
                            a["npages"], a["d"], 1, 0, 0.125, 1, None, 0, 1, None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(P=100), 2), (dict(P=0), 2), (dict(pps=0), 2), (dict(npages=0), 2), (dict(table=None), 1),
    (dict(seqlens=None), 1), (dict(table=FAKE + 2), 8), (dict(seqlens=FAKE + 1), 8), (dict(d=80), 4),
    (dict(d=96), 4), (dict(ws=None), 7), (dict(wsb=4096), 7), (dict(ws=FAKE + 8), 8), (dict(Hkv=3), 3),
])
def test_bwd_paged_rejects_bad_arguments(lib, kw, status):
    a = dict(table=FAKE, seqlens=FAKE, pps=4, P=128, npages=8, d=64, ws=FAKE, wsb=1 << 30, Hkv=1)
    a.update(kw)
    assert lib.fa_bwd_paged(*(FAKE,) * 9, a["table"], a["seqlens"], 2, 2, a["Hkv"], 16, a["pps"], a["P"],
                            a["npages"], a["d"], 1, 0, 0.125, 1, a["ws"], a["wsb"], None) == status


def test_bwd_paged_workspace_bytes(lib):
    # fa_bwd's workspace, then gathered K, V and per-sequence dK, dV ([B][Hkv][pps * P][d] each)
    B, Hq, Hkv, Tq, pps, P, d = 3, 8, 2, 33, 5, 128, 128
    for code, esize in ((fa.FA_DTYPE_BF16, 2), (fa.FA_DTYPE_F32, 4)):
        part = -(-B * Hkv * pps * P * d * esize // 256) * 256
        base = lib.fa_bwd_workspace_bytes(B, Hq, Hkv, Tq, pps * P, d, code)
        assert lib.fa_bwd_paged_workspace_bytes(B, Hq, Hkv, Tq, pps, P, d, code) == base + 4 * part
    assert lib.fa_bwd_paged_workspace_bytes(B, Hq, Hkv, Tq, pps, 100, d, 1) == 0
    assert lib.fa_bwd_paged_workspace_bytes(B, Hq, Hkv, Tq, 0, P, d, 1) == 0
    assert lib.fa_bwd_paged_workspace_bytes(B, Hq, Hkv, Tq, pps, P, 80, 1) == 0


def test_mask_row_words(lib):
    assert [lib.fa_mask_row_words(t) for t in (0, 1, 127, 128, 129, 1000)] == [0, 4, 4, 4, 8, 32]
    assert lib.fa_mask_row_words(-1) == -1


@pytest.mark.parametrize("kw,status", [
    (dict(mask=None), 1), (dict(mask=FAKE + 4), 8), (dict(stride=-1), 2), (dict(stride=5), 2), (dict(stride=16 * 12 + 2), 8),
    (dict(d=80, dv=80), 4), (dict(Hkv=3), 3), (dict(scale=math.nan), 6), (dict(dv=96), 4),
    (dict(d=32, dv=64, dtype=0), 4), (dict(d=128, dv=32, dtype=0), 4),
])
def test_fwd_mask_rejects_bad_arguments(lib, kw, status):
    a = dict(mask=FAKE, stride=0, d=64, dv=64, Hkv=2, scale=0.125, dtype=1)
    a.update(kw)
    assert lib.fa_fwd_mask(FAKE, FAKE, FAKE, FAKE, FAKE, a["mask"], a["stride"], 2, 4, a["Hkv"], 16, 300, a["d"],
                           a["dv"], 1, 50, a["scale"], a["dtype"], None) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, -1, 10), 2), ((FAKE, FAKE, 4, -1), 2), ((None, FAKE, 4, 10), 1), ((FAKE, None, 4, 10), 1),
    ((FAKE, FAKE + 4, 4, 10), 8),
])
def test_mask_pack_rejects_bad_arguments(lib, args, status):
    assert lib.fa_mask_pack(*args, None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(mask=None), 1), (dict(stride=-4), 2), (dict(stride=6), 2), (dict(ws=None), 7), (dict(wsb=64), 7),
    (dict(d=80, dv=80), 4), (dict(dv=96), 4), (dict(d=32, dv=64, dtype=0), 4),
])
def test_bwd_mask_rejects_bad_arguments(lib, kw, status):
    a = dict(mask=FAKE, stride=0, ws=FAKE, wsb=1 << 30, d=64, dv=64, dtype=1)
    a.update(kw)
    assert lib.fa_bwd_mask(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["ws"], a["wsb"], a["mask"],
                           a["stride"], 2, 4, 2, 16, 300, a["d"], a["dv"], 1, 50, 0.125, a["dtype"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(mask=None), 1), (dict(stride=-4), 2), (dict(stride=6), 2), (dict(cu_q=None), 1), (dict(cu_k=FAKE + 2), 8),
    (dict(max_q=40), 2), (dict(d=80), 4), (dict(scale=0.0), 6),
])
def test_varlen_mask_rejects_bad_arguments(lib, kw, status):
    a = dict(mask=FAKE, stride=0, cu_q=FAKE, cu_k=FAKE, max_q=16, d=64, scale=0.125)
    a.update(kw)
    # B = 2 sequences, Hq = 4, Hkv = 2, total_q = 32, total_k = 300, longest 16 and 200
    assert lib.fa_fwd_varlen_mask(*(FAKE,) * 5, a["mask"], a["stride"], a["cu_q"], a["cu_k"], 2, 4, 2, 32, 300,
                                  a["max_q"], 200, a["d"], 1, 0, a["scale"], 1, None) == status
    assert lib.fa_bwd_varlen_mask(*(FAKE,) * 9, FAKE, 1 << 30, a["mask"], a["stride"], a["cu_q"], a["cu_k"], 2, 4, 2,
                                  32, 300, a["max_q"], 200, a["d"], 1, 0, a["scale"], 1, None) == status
    assert lib.fa_bwd_varlen_mask(*(FAKE,) * 9, None, 0, FAKE, 0, FAKE, FAKE, 2, 4, 2, 32, 300, 16, 200, 64, 1, 0,
                                  0.125, 1, None) == 7


def test_bwd_mask_workspace_adds_the_key_major_copy(lib):
    base = lib.fa_bwd_workspace_bytes(2, 4, 2, 200, 300, 64, 1)
    shared = lib.fa_bwd_mask_workspace_bytes(2, 4, 2, 200, 300, 64, 1, 0)
    per = lib.fa_bwd_mask_workspace_bytes(2, 4, 2, 200, 300, 64, 1, 200 * 12)
    words = 300 * 4 * math.ceil(200 / 128)
    assert shared - base == math.ceil(words * 4 / 256) * 256
    assert per - base == math.ceil(2 * words * 4 / 256) * 256
    assert lib.fa_bwd_mask_workspace_bytes(2, 4, 2, 200, 300, 64, 1, -1) == 0


def test_mask_splitk_workspace_and_arguments(lib):
    assert lib.fa_fwd_mask_splitk_workspace_bytes(4, 32, 8, 32, 1056, 128, 128, 1, 1) == 0
    n3 = lib.fa_fwd_mask_splitk_workspace_bytes(4, 32, 8, 32, 1056, 128, 128, 1, 3)
    rows = 4 * 32 * 32
    assert n3 == math.ceil(3 * rows * 128 * 4 / 256) * 256 + math.ceil(3 * rows * 4 / 256) * 256
    # fp32 partials dv wide
    n3v = lib.fa_fwd_mask_splitk_workspace_bytes(4, 32, 8, 32, 1056, 128, 64, 1, 3)
    assert n3v == math.ceil(3 * rows * 64 * 4 / 256) * 256 + math.ceil(3 * rows * 4 / 256) * 256
    assert lib.fa_fwd_mask_splitk_workspace_bytes(4, 32, 8, 32, 1056, 128, 96, 1, 3) == 0
    # a split call without its workspace, then with too small a one
    assert lib.fa_fwd_mask_splitk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None, 0, 4, 32, 8, 32, 1056, 128, 128, 0,
                                  0, 0.125, 1, 3, None) == 7
    assert lib.fa_fwd_mask_splitk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 64, 4, 32, 8, 32, 1056, 128, 128, 0,
                                  0, 0.125, 1, 3, None) == 7
    assert lib.fa_fwd_mask_splitk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 30, 4, 32, 8, 32, 1056, 128, 128,
                                  0, 0, 0.125, 1, 5000, None) == 9


def test_varlen_splitk_workspace_and_arguments(lib):
    """fa_fwd_varlen_splitk: partials for Hq * total_q rows per slice; B = 2 sequences, Hq = 4,
    Hkv = 2, total_q = 32, total_k = 300, longest 16 and 200, d = 64, bf16."""
    size = lambda ns, masked=0, d=64, total_q=32, max_q=16, total_k=300: lib.fa_fwd_varlen_splitk_workspace_bytes(
        2, 4, 2, total_q, total_k, max_q, 200, d, 1, ns, masked)
    rows = 4 * 32
    assert size(3) == math.ceil(3 * rows * 64 * 4 / 256) * 256 + math.ceil(3 * rows * 4 / 256) * 256
    assert size(3, masked=1) == size(3)
    assert size(1) == 0 and size(1, masked=1) == 0
    assert size(3, d=96) == 0 and size(3, max_q=40) == 0 and size(3, total_k=100) == 0 and size(5000) == 0

    def call(mask=None, stride=0, cu_q=FAKE, ws=FAKE, wsb=1 << 30, ns=3, d=64, window=0):
        return lib.fa_fwd_varlen_splitk(*(FAKE,) * 5, mask, stride, cu_q, FAKE, ws, wsb, 2, 4, 2, 32, 300, 16, 200, d,
                                        1, window, 0.125, 1, ns, None)
    assert call(ws=None, wsb=0) == 7 and call(wsb=64) == 7 and call(mask=FAKE, ws=None, wsb=0) == 7
    assert call(ns=5000) == 9
    assert call(ws=FAKE + 4) == 8
    assert call(cu_q=None) == 1 and call(d=80) == 4
    assert call(mask=FAKE, stride=-4) == 2 and call(mask=FAKE, stride=6) == 2
    # one slice needs no workspace: validation passes and stops at the NULL output
    assert lib.fa_fwd_varlen_splitk(FAKE, FAKE, FAKE, None, FAKE, None, 0, FAKE, FAKE, None, 0, 2, 4, 2, 32, 300,
                                    16, 200, 64, 1, 0, 0.125, 1, 1, None) == 1


def test_varlen_split_automatic_count(lib):
    """The automatic slice count of fa_fwd_varlen_splitk, read back through the workspace size
    (which grows linearly with the count).  16 blocks of 32 queries, Hq = 32, Hkv = 8, d = 128,
    bf16: with key counts near the mean (longest 7759 of 64000 keys) it is the fixed layout's
    count for the longest lengths (2); with one 8032-key prefix among short ones (12344 keys in
    all, longest / mean = 10.4) the workgroup target grows by sqrt(10.4), to 7 slices."""
    size = lambda total_k, max_k, ns, masked=0: lib.fa_fwd_varlen_splitk_workspace_bytes(
        16, 32, 8, 512, total_k, 32, max_k, 128, 1, ns, masked)
    assert size(64000, 7759, 0) == size(64000, 7759, 2) > 0
    # the same rows as 16 fixed-layout entries of 32 queries: the same count and size
    assert size(64000, 7759, 0) == lib.fa_fwd_splitk_workspace_bytes(16, 32, 8, 32, 7759, 128, 1, 0)
    assert size(12344, 8032, 0) == size(12344, 8032, 7)
    assert size(12344, 8032, 0, masked=1) == size(12344, 8032, 7, masked=1)


@pytest.mark.parametrize("d,fp32,bf16", [(32, 1, 1), (64, 1, 1), (128, 1, 1), (16, 4, 4), (96, 4, 4), (256, 4, 1)])
def test_head_dims(lib, d, fp32, bf16):
    # supported head dims pass validation (then fail on the NULL output); 256 is bf16 only
    for dtype, status in ((0, fp32), (1, bf16)):
        assert lib.fa_fwd(FAKE, FAKE, FAKE, None, FAKE, 1, 2, 1, 16, 16, d, 0, 0.125, dtype, None) == status


def test_head_dim_256_is_bf16_only(lib):
    # workspace functions: sized for bf16, 0 (invalid) for fp32
    assert lib.fa_bwd_workspace_bytes(1, 2, 1, 16, 16, 256, 1) > 0
    assert lib.fa_bwd_workspace_bytes(1, 2, 1, 16, 16, 256, 0) == 0
    assert lib.fa_bwd_paged_workspace_bytes(2, 2, 1, 16, 4, 128, 256, 1) > 0
    # validation passes in bf16 and stops at the NULL output, before any launch
    assert lib.fa_fwd_mask(FAKE, FAKE, FAKE, None, FAKE, FAKE, 0, 2, 4, 2, 16, 300, 256, 256, 1, 0, 0.125, 1,
                           None) == 1
    assert lib.fa_bwd(*(FAKE,) * 6, None, FAKE, FAKE, FAKE, 1 << 30, 1, 2, 1, 16, 16, 256, 1, 0.125, 1, None) == 1
    assert lib.fa_bwd(*(FAKE,) * 10, 1 << 30, 1, 2, 1, 16, 16, 256, 1, 0.125, 0, None) == 4


# Every entry point that takes a scale, called with arguments that pass every
# other check (fake aligned pointers, room in the workspace), so that the scale
# is what fails: zero and negative scales are rejected like NaN, because the
# kernels mask scores with -inf before scaling and take the row maximum of the
# unscaled scores, which hold only for a positive scale.
def _scale_calls(lib, s):
    W = 1 << 30
    return {
        "fa_fwd": lambda: lib.fa_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 16, 16, 64, 1, s, 1, None),
        "fa_fwd_window": lambda: lib.fa_fwd_window(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 16, 16, 64, 1, 8, s, 1,
                                                   None),
        "fa_fwd_dv": lambda: lib.fa_fwd_dv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 1, 16, 16, 128, 64, 1, 0, s, 1, None),
        "fa_fwd_splitk": lambda: lib.fa_fwd_splitk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, W, 1, 2, 1, 16, 16, 64, 1, 0,
                                                   s, 1, 2, None),
        "fa_fwd_varlen": lambda: lib.fa_fwd_varlen(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 1, 32, 32, 16, 16,
                                                   64, 1, 0, s, 1, None),
        "fa_fwd_paged": lambda: lib.fa_fwd_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 2, 1, 16, 4, 128, 8,
                                                 64, 1, 0, s, 1, None, 0, 1, None),
        "fa_fwd_mask": lambda: lib.fa_fwd_mask(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 4, 2, 16, 300, 64, 64, 1, 0,
                                               s, 1, None),
        "fa_fwd_mask_splitk": lambda: lib.fa_fwd_mask_splitk(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, W, 2, 4, 2,
                                                             16, 300, 64, 64, 1, 0, s, 1, 2, None),
        "fa_fwd_varlen_mask": lambda: lib.fa_fwd_varlen_mask(*(FAKE,) * 6, 0, FAKE, FAKE, 2, 4, 2, 32, 300, 16, 200, 64,
                                                             1, 0, s, 1, None),
        "fa_bwd_varlen_mask": lambda: lib.fa_bwd_varlen_mask(*(FAKE,) * 10, W, FAKE, 0, FAKE, FAKE, 2, 4, 2, 32, 300,
                                                             16, 200, 64, 1, 0, s, 1, None),
        "fa_fwd_varlen_splitk": lambda: lib.fa_fwd_varlen_splitk(*(FAKE,) * 5, None, 0, FAKE, FAKE, FAKE, W, 2, 4, 2,
                                                                 32, 300, 16, 200, 64, 1, 0, s, 1, 2, None),
        "fa_bwd": lambda: lib.fa_bwd(*(FAKE,) * 10, W, 1, 2, 1, 16, 16, 64, 1, s, 1, None),
        "fa_bwd_stages": lambda: lib.fa_bwd_stages(*(FAKE,) * 10, W, 1, 2, 1, 16, 16, 64, 1, s, 1, 7, None),
        "fa_bwd_window": lambda: lib.fa_bwd_window(*(FAKE,) * 10, W, 1, 2, 1, 16, 16, 64, 1, 8, s, 1, 7, None),
        "fa_bwd_dv": lambda: lib.fa_bwd_dv(*(FAKE,) * 10, W, 1, 2, 1, 16, 16, 128, 64, 1, 0, s, 1, 7, None),
        "fa_bwd_varlen": lambda: lib.fa_bwd_varlen(*(FAKE,) * 10, W, FAKE, FAKE, 2, 2, 1, 32, 32, 16, 16, 64, 1, 0,
                                                   s, 1, None),
        "fa_bwd_mask": lambda: lib.fa_bwd_mask(*(FAKE,) * 10, W, FAKE, 0, 2, 4, 2, 16, 300, 64, 64, 1, 0, s, 1, None),
        "fa_bwd_noalloc": lambda: lib.fa_bwd_noalloc(*(FAKE,) * 9, 1, 2, 1, 16, 16, 64, 1, s, 1, None),
        "fa_bwd_paged": lambda: lib.fa_bwd_paged(*(FAKE,) * 11, 2, 2, 1, 16, 4, 128, 8, 64, 1, 0, s, 1, FAKE, W,
                                                 None),
    }


@pytest.mark.parametrize("scale", [0.0, -0.0, -0.1, -math.inf, math.inf, math.nan])
def test_every_entry_point_rejects_a_non_positive_or_non_finite_scale(lib, scale):
    calls = _scale_calls(lib, scale)
    got = {name: call() for name, call in calls.items()}
    assert got == {name: 6 for name in calls}


def test_scale_table_covers_every_entry_point_that_takes_a_scale():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    with_scale = {m.group(1) for m in re.finditer(r"\b(fa_[a-z_0-9]+)\s*\(([^;]*?)\);", text, flags=re.S)
                  if re.search(r"\bfloat\s+scale\b", m.group(2))}
    assert with_scale == set(_scale_calls(None, 0.125))


_NO_DEVICE_SCRIPT = r"""
import ctypes, sys
lib = ctypes.CDLL(sys.argv[1])
vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
lib.fa_fwd.argtypes = [vp] * 5 + [i] * 7 + [f, i, vp]
lib.fa_hip_error_string.restype = ctypes.c_char_p
F = 1 << 20
print(lib.fa_fwd(F, F, F, F, F, 1, 2, 1, 16, 16, 64, 0, 0.125, 1, None))
print(lib.fa_hip_error_string().decode())
"""


def test_a_launch_without_a_device_returns_the_hip_status():
    """With valid arguments and no HIP device the launch itself fails: the call returns
    FA_ERR_HIP and the HIP text names the missing device.  The arguments are fake device
    pointers, so this must never run where a GPU is visible (skipped there)."""
    import subprocess
    import sys
    from conftest import gpu_available
    if gpu_available() or os.path.exists("/dev/kfd"):
        pytest.skip("a GPU is visible: the fake pointers of this test must not reach it")
    r = subprocess.run([sys.executable, "-c", _NO_DEVICE_SCRIPT, fa.LIB_PATH], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    status, text = r.stdout.strip().splitlines()[-2:]
    assert int(status) == 10
    assert "device" in text.lower()


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """fa_bwd_noalloc needs 8 bytes per padded query row; beyond its fixed scratch it returns
    FA_ERR_SCRATCH before any HIP call (fake pointers: nothing is launched)."""
    cap = lib.fa_bwd_noalloc_scratch_bytes()
    assert cap == 16 << 20
    rows_max = cap // 8                                    # 2,097,152 padded rows
    ok_heads = rows_max // 4096
    # one more head than fits: rejected; the other checks still come first
    assert lib.fa_bwd_noalloc(*(FAKE,) * 9, 1, ok_heads + 1, 1, 4096, 64, 64, 1, 0.125, 1, None) == 12
    assert lib.fa_bwd_noalloc(*(FAKE,) * 9, 1, 3, 2, 4096, 64, 64, 1, 0.125, 1, None) == 3
    assert lib.fa_bwd_noalloc(*(FAKE,) * 8, None, 1, 2, 1, 16, 16, 64, 1, 0.125, 1, None) == 1
    # padding counts: Tq = 4033 pads to 4096 rows per head
    assert lib.fa_bwd_noalloc(*(FAKE,) * 9, 1, ok_heads + 1, 1, 4033, 64, 64, 1, 0.125, 1, None) == 12
