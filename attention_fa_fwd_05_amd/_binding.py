"""ctypes binding of libfa05.so (include/fa.h): argument marshalling only.

Torch provides device memory (outputs and the backward workspace are
allocated here, outside the library) and the current HIP stream; every step
of the computation runs in the library's kernels.  A missing library raises;
there is no fallback.
"""

from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa05.so")

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1

STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL_PTR", 2: "FA_ERR_BAD_SHAPE", 3: "FA_ERR_GQA_RATIO",
    4: "FA_ERR_HEAD_DIM", 5: "FA_ERR_DTYPE", 6: "FA_ERR_SCALE", 7: "FA_ERR_WORKSPACE",
    8: "FA_ERR_ALIGNMENT", 9: "FA_ERR_TOO_LARGE", 10: "FA_ERR_HIP", 11: "FA_ERR_STAGES",
    12: "FA_ERR_SCRATCH",
}
STAGE_PRE, STAGE_DKDV, STAGE_DQ, STAGE_ALL = 1, 2, 4, 7
EXPORTS = ["fa_fwd", "fa_bwd", "fa_bwd_stages", "fa_fwd_window", "fa_bwd_window", "fa_fwd_dv", "fa_bwd_dv",
           "fa_fwd_splitk",
           "fa_fwd_splitk_workspace_bytes", "fa_fwd_varlen", "fa_bwd_varlen", "fa_fwd_paged",
           "fa_fwd_paged_workspace_bytes", "fa_bwd_paged", "fa_bwd_paged_workspace_bytes", "fa_bwd_workspace_bytes",
           "fa_mask_row_words", "fa_mask_pack", "fa_fwd_mask", "fa_bwd_mask", "fa_bwd_mask_workspace_bytes",
           "fa_fwd_mask_splitk", "fa_fwd_mask_splitk_workspace_bytes", "fa_fwd_varlen_mask", "fa_bwd_varlen_mask",
           "fa_fwd_varlen_splitk", "fa_fwd_varlen_splitk_workspace_bytes",
           "fa_bwd_noalloc", "fa_bwd_noalloc_scratch_bytes",
           "fa_status_string", "fa_hip_error_string", "fa_abi_version"]

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = status_string(status)
        if status == 10:
            detail += ": " + load_library().fa_hip_error_string().decode()
        super().__init__(f"{where}: {STATUS.get(status, status)} ({detail})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfa05.so and declare the C signatures (cached)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m attention_fa_fwd_05_amd.build`")
    # The library shares torch's HIP runtime (same soname).  Its kernels must be
    # registered after that runtime has initialised the device, or launches
    # fail with "no ROCm-capable device", so bring torch's device up first.
    import torch
    if torch.cuda.is_available():
        torch.cuda.init()
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                           i, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_stages.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                  i, i, i, i, i, i, i, f, i, ctypes.c_uint, vp]
    lib.fa_bwd_stages.restype = i
    lib.fa_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_window.restype = i
    lib.fa_bwd_window.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                  i, i, i, i, i, i, i, i, f, i, ctypes.c_uint, vp]
    lib.fa_bwd_window.restype = i
    lib.fa_fwd_splitk.argtypes = [vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_splitk.restype = i
    lib.fa_fwd_splitk_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    lib.fa_fwd_splitk_workspace_bytes.restype = sz
    lib.fa_fwd_dv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_dv.restype = i
    lib.fa_bwd_dv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                              i, i, i, i, i, i, i, i, i, f, i, ctypes.c_uint, vp]
    lib.fa_bwd_dv.restype = i
    lib.fa_fwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f, i, vp, sz, i, vp]
    lib.fa_fwd_paged.restype = i
    lib.fa_fwd_paged_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.fa_fwd_paged_workspace_bytes.restype = sz
    lib.fa_bwd_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f, i,
                                 vp, sz, vp]
    lib.fa_bwd_paged.restype = i
    lib.fa_bwd_paged_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    lib.fa_bwd_paged_workspace_bytes.restype = sz
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp,
                                  i, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_varlen.restype = i
    ll = ctypes.c_longlong
    lib.fa_mask_row_words.argtypes = [i]
    lib.fa_mask_row_words.restype = i
    lib.fa_mask_pack.argtypes = [vp, vp, ll, i, vp]
    lib.fa_mask_pack.restype = i
    lib.fa_fwd_mask.argtypes = [vp, vp, vp, vp, vp, vp, ll, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_mask.restype = i
    lib.fa_fwd_mask_splitk.argtypes = [vp, vp, vp, vp, vp, vp, ll, vp, sz, i, i, i, i, i, i, i, i, i, f, i, i,
                                       vp]
    lib.fa_fwd_mask_splitk.restype = i
    lib.fa_fwd_mask_splitk_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.fa_fwd_mask_splitk_workspace_bytes.restype = sz
    lib.fa_bwd_mask.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, ll, i, i, i, i, i, i, i, i, i, f, i,
                                vp]
    lib.fa_bwd_mask.restype = i
    lib.fa_fwd_varlen_mask.argtypes = [vp, vp, vp, vp, vp, vp, ll, vp, vp, i, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_varlen_mask.restype = i
    lib.fa_bwd_varlen_mask.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, ll, vp, vp,
                                       i, i, i, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_varlen_mask.restype = i
    lib.fa_fwd_varlen_splitk.argtypes = [vp, vp, vp, vp, vp, vp, ll, vp, vp, vp, sz, i, i, i, i, i, i, i, i, i, i,
                                         f, i, i, vp]
    lib.fa_fwd_varlen_splitk.restype = i
    lib.fa_fwd_varlen_splitk_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i, i, i]
    lib.fa_fwd_varlen_splitk_workspace_bytes.restype = sz
    lib.fa_bwd_mask_workspace_bytes.argtypes = [i, i, i, i, i, i, i, ll]
    lib.fa_bwd_mask_workspace_bytes.restype = sz
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_scratch_bytes.argtypes = []
    lib.fa_bwd_noalloc_scratch_bytes.restype = sz
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_hip_error_string.argtypes = []
    lib.fa_hip_error_string.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    if path == LIB_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return FA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t) -> int | None:
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _on_gpu(t, name):
    """Every tensor handed to the library must live in device memory: a host pointer would be
    dereferenced by a kernel."""
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")


def _shapes(q, k, v, same_dv: bool = False):
    """(B, Hq, Hkv, Tq, Tk, d) of q [B, Hq, Tq, d], k [B, Hkv, Tk, d], v [B, Hkv, Tk, dv].

    ``same_dv``: the entry point has no dv argument (its kernels index V with stride d), so v's
    head dim must equal q's."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    if Bk != B or dk != d or tuple(v.shape[:3]) != (B, Hkv, Tk):
        raise ValueError(f"inconsistent shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if same_dv and v.shape[3] != d:
        raise ValueError(f"this entry point needs v's head dim ({v.shape[3]}) equal to q's ({d})")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share dtype and device")
    _on_gpu(q, "q")
    return B, Hq, Hkv, Tq, Tk, d


def _out(t, name, shape, like, dtype=None):
    """A caller-supplied output (or None, then allocated by the caller of this helper): it must
    have the exact shape, the dtype (``like``'s unless given), ``like``'s device and be
    contiguous, since the library writes every element of that extent."""
    if t is None:
        return None
    dtype = like.dtype if dtype is None else dtype
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != like.device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {like.device}, "
                         f"got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _ws(ws, need, like):
    """The caller's workspace (a device tensor of at least ``need`` bytes) or a new one."""
    import torch
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=like.device)
    if ws.device != like.device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, {need} needed")
    return ws


def workspace_bytes(B, Hq, Hkv, Tq, Tk, d, dtype_code) -> int:
    return int(load_library().fa_bwd_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, dtype_code))


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
            window: int = 0):
    """fa_fwd (fa_fwd_window when window > 0, fa_fwd_dv when v's head dim differs from q's):
    returns (o, lse), o [B, Hq, Tq, dv], lse float32 [B, Hq, Tq]."""
    import torch
    lib = load_library()
    B, Hq, Hkv, Tq, Tk, d = _shapes(q, k, v)
    dv = v.shape[3]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = _out(out, "out", (B, Hq, Tq, dv), q)
    o = q.new_empty((B, Hq, Tq, dv)) if o is None else o
    L = _out(lse, "lse", (B, Hq, Tq), q, torch.float32)
    L = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if L is None else L
    if dv != d:
        st = lib.fa_fwd_dv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), B, Hq, Hkv, Tq, Tk, d, dv,
                           int(bool(causal)), int(window), scale, _dtype_code(q), _stream(q))
        if st != 0:
            raise FaError(st, "fa_fwd_dv")
        return o, L
    if window > 0:
        st = lib.fa_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), B, Hq, Hkv, Tq, Tk, d,
                               int(bool(causal)), int(window), scale, _dtype_code(q), _stream(q))
    else:
        st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), B, Hq, Hkv, Tq, Tk, d,
                        int(bool(causal)), scale, _dtype_code(q), _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd_window" if window > 0 else "fa_fwd")
    return o, L


def splitk_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, dtype_code, nsplit=0) -> int:
    return int(load_library().fa_fwd_splitk_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, dtype_code, nsplit))


def forward_splitk(q, k, v, causal: bool = False, scale: float | None = None, window: int = 0,
                   nsplit: int = 0, workspace=None, out=None, lse=None):
    """fa_fwd_splitk: the forward split over key slices and merged; returns (o, lse)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, Tq, Tk, d = _shapes(q, k, v, same_dv=True)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = splitk_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, code, nsplit)
    ws = _ws(workspace, need, q)
    o = _out(out, "out", q.shape, q)
    o = torch.empty_like(q) if o is None else o
    L = _out(lse, "lse", (B, Hq, Tq), q, torch.float32)
    L = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if L is None else L
    st = lib.fa_fwd_splitk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), ws.data_ptr(), _nbytes(ws),
                           B, Hq, Hkv, Tq, Tk, d, int(bool(causal)), int(window), scale, code, int(nsplit),
                           _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd_splitk")
    return o, L


def _varlen_shapes(q, k, v, cu_q, cu_k):
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("varlen q, k, v must be [H, total, d]")
    Hq, total_q, d = q.shape
    Hkv, total_k, dk = k.shape
    if dk != d or tuple(v.shape) != (Hkv, total_k, d):
        raise ValueError(f"inconsistent shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous and share dtype and device")
    for c in (cu_q, cu_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous() or c.device != q.device:
            raise ValueError("cu_seqlens must be contiguous int32 [B + 1] on q's device")
    if cu_q.numel() != cu_k.numel() or cu_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 >= 2 offsets")
    _on_gpu(q, "q")
    return cu_q.numel() - 1, Hq, Hkv, total_q, total_k, d


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                   causal: bool = False, scale: float | None = None, window: int = 0, out=None, lse=None):
    """fa_fwd_varlen: q [Hq, total_q, d], k, v [Hkv, total_k, d] packed head-major; returns
    (o like q, lse float32 [Hq, total_q])."""
    import torch
    lib = load_library()
    B, Hq, Hkv, total_q, total_k, d = _varlen_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = _out(out, "out", q.shape, q)
    o = torch.empty_like(q) if o is None else o
    L = _out(lse, "lse", (Hq, total_q), q, torch.float32)
    L = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device) if L is None else L
    st = lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), cu_seqlens_q.data_ptr(),
                           cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q),
                           int(max_seqlen_k), d, int(bool(causal)), int(window), scale, _dtype_code(q), _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd_varlen")
    return o, L


def backward_varlen(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    causal: bool = False, scale: float | None = None, window: int = 0, workspace=None,
                    dq=None, dk=None, dv=None):
    """fa_bwd_varlen: returns (dq, dk, dv) like q, k, v (packed head-major)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, total_q, total_k, d = _varlen_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k)
    _out(o, "o", q.shape, q)
    _out(do, "do", q.shape, q)
    _out(lse, "lse", (Hq, total_q), q, torch.float32)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = workspace_bytes(B, Hq, Hkv, int(max_seqlen_q), int(max_seqlen_k), d, code)
    ws = _ws(workspace, need, q)
    dq = torch.empty_like(q) if _out(dq, "dq", q.shape, q) is None else dq
    dk = torch.empty_like(k) if _out(dk, "dk", k.shape, q) is None else dk
    dv = torch.empty_like(v) if _out(dv, "dv", v.shape, q) is None else dv
    st = lib.fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                           _ptr(dv), ws.data_ptr(), _nbytes(ws), cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                           B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), d,
                           int(bool(causal)), int(window), scale, code, _stream(q))
    if st != 0:
        raise FaError(st, "fa_bwd_varlen")
    return dq, dk, dv


def _varlen_mask_bits(lib, mask, q, B, max_q, max_k):
    """(packed int32 bits, per-sequence stride in words) of a varlen mask: bool/uint8 or packed
    int32, [max_q, max_k] (shared) or [B, max_q, max_k]."""
    return _mask_bits(lib, mask, q, B, max_q, max_k)


def forward_varlen_masked(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, mask,
                          causal: bool = False, scale: float | None = None, window: int = 0, out=None,
                          lse=None):
    """fa_fwd_varlen_mask: forward_varlen under a boolean mask per sequence (``mask`` [max_q, max_k]
    for every sequence or [B, max_q, max_k], indexed by each sequence's own positions)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, total_q, total_k, d = _varlen_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k)
    bits, stride = _varlen_mask_bits(lib, mask, q, B, int(max_seqlen_q), int(max_seqlen_k))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if _out(out, "out", q.shape, q) is None else out
    L = _out(lse, "lse", (Hq, total_q), q, torch.float32)
    L = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device) if L is None else L
    st = lib.fa_fwd_varlen_mask(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), _ptr(bits), stride,
                                cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k,
                                int(max_seqlen_q), int(max_seqlen_k), d, int(bool(causal)), int(window), scale,
                                _dtype_code(q), _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd_varlen_mask")
    return o, L


def backward_varlen_masked(q, k, v, o, lse, do, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                           mask, causal: bool = False, scale: float | None = None, window: int = 0,
                           workspace=None, dq=None, dk=None, dv=None):
    """fa_bwd_varlen_mask: the backward of forward_varlen_masked; returns (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, total_q, total_k, d = _varlen_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k)
    _out(o, "o", q.shape, q)
    _out(do, "do", q.shape, q)
    _out(lse, "lse", (Hq, total_q), q, torch.float32)
    bits, stride = _varlen_mask_bits(lib, mask, q, B, int(max_seqlen_q), int(max_seqlen_k))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = int(lib.fa_bwd_mask_workspace_bytes(B, Hq, Hkv, int(max_seqlen_q), int(max_seqlen_k), d, code, stride))
    ws = _ws(workspace, need, q)
    dq = torch.empty_like(q) if _out(dq, "dq", q.shape, q) is None else dq
    dk = torch.empty_like(k) if _out(dk, "dk", k.shape, q) is None else dk
    dv = torch.empty_like(v) if _out(dv, "dv", v.shape, q) is None else dv
    st = lib.fa_bwd_varlen_mask(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
                                _ptr(dv), ws.data_ptr(), _nbytes(ws), _ptr(bits), stride, cu_seqlens_q.data_ptr(),
                                cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q),
                                int(max_seqlen_k), d, int(bool(causal)), int(window), scale, code, _stream(q))
    if st != 0:
        raise FaError(st, "fa_bwd_varlen_mask")
    return dq, dk, dv


def _paged_shapes(q, k_pages, v_pages, page_table, seqlens_k):
    import torch
    if q.dim() != 4 or k_pages.dim() != 4 or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("q [B, Hq, Tq, d], k_pages = v_pages shape [num_pages, Hkv, page_size, d]")
    B, Hq, Tq, d = q.shape
    num_pages, Hkv, page_size, dk = k_pages.shape
    if dk != d or page_table.dim() != 2 or page_table.shape[0] != B or tuple(seqlens_k.shape) != (B,):
        raise ValueError("inconsistent paged shapes")
    for t in (q, k_pages, v_pages, page_table, seqlens_k):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("tensors must be contiguous on q's device")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise ValueError("q, k_pages, v_pages must share a dtype")
    _on_gpu(q, "q")
    if page_table.dtype != torch.int32 or seqlens_k.dtype != torch.int32:
        raise ValueError("page_table and seqlens_k must be int32")
    return B, Hq, Tq, d, num_pages, Hkv, page_size, page_table.shape[1]


def forward_paged(q, k_pages, v_pages, page_table, seqlens_k, causal: bool = False, scale: float | None = None,
                  window: int = 0, nsplit: int = 0, workspace=None, out=None, lse=None):
    """fa_fwd_paged: q [B, Hq, Tq, d]; k_pages, v_pages [num_pages, Hkv, page_size, d]; page_table
    int32 [B, pages_per_seq]; seqlens_k int32 [B].  Returns (o like q, lse float32 [B, Hq, Tq])."""
    import torch
    lib = load_library()
    B, Hq, Tq, d, num_pages, Hkv, page_size, pps = _paged_shapes(q, k_pages, v_pages, page_table, seqlens_k)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = int(lib.fa_fwd_paged_workspace_bytes(B, Hq, Hkv, Tq, pps, page_size, d, code, int(nsplit)))
    ws = _ws(workspace, need, q)
    o = _out(out, "out", q.shape, q)
    o = torch.empty_like(q) if o is None else o
    L = _out(lse, "lse", (B, Hq, Tq), q, torch.float32)
    L = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if L is None else L
    st = lib.fa_fwd_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o), _ptr(L), page_table.data_ptr(),
                          seqlens_k.data_ptr(), B, Hq, Hkv, Tq, pps, page_size, num_pages, d, int(bool(causal)),
                          int(window), scale, code, ws.data_ptr(), _nbytes(ws), int(nsplit), _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd_paged")
    return o, L


def backward_paged(q, k_pages, v_pages, o, lse, do, page_table, seqlens_k, causal: bool = False,
                   scale: float | None = None, window: int = 0, workspace=None, dq=None, dk_pages=None,
                   dv_pages=None):
    """fa_bwd_paged: the backward of forward_paged.  Returns (dq like q, dk_pages like k_pages,
    dv_pages like v_pages); a page no table entry references gets zeros."""
    import torch
    lib = load_library()
    B, Hq, Tq, d, num_pages, Hkv, page_size, pps = _paged_shapes(q, k_pages, v_pages, page_table, seqlens_k)
    _out(o, "o", q.shape, q)
    _out(do, "do", q.shape, q)
    _out(lse, "lse", (B, Hq, Tq), q, torch.float32)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = int(lib.fa_bwd_paged_workspace_bytes(B, Hq, Hkv, Tq, pps, page_size, d, code))
    if need == 0:
        raise ValueError("unsupported paged backward sizes")
    ws = _ws(workspace, need, q)
    dq = torch.empty_like(q) if _out(dq, "dq", q.shape, q) is None else dq
    dk_pages = torch.empty_like(k_pages) if _out(dk_pages, "dk_pages", k_pages.shape, q) is None else dk_pages
    dv_pages = torch.empty_like(v_pages) if _out(dv_pages, "dv_pages", v_pages.shape, q) is None else dv_pages
    st = lib.fa_bwd_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq),
                          _ptr(dk_pages), _ptr(dv_pages), page_table.data_ptr(), seqlens_k.data_ptr(), B, Hq, Hkv,
                          Tq, pps, page_size, num_pages, d, int(bool(causal)), int(window), scale, code,
                          ws.data_ptr(), _nbytes(ws), _stream(q))
    if st != 0:
        raise FaError(st, "fa_bwd_paged")
    return dq, dk_pages, dv_pages


def pack_mask(mask, Tk: int | None = None, out=None):
    """fa_mask_pack: a boolean (or uint8, nonzero = visible) mask [..., Tq, Tk] on the GPU to the
    library's bit layout, int32 [..., Tq, fa_mask_row_words(Tk)] (the same leading dims)."""
    import torch
    lib = load_library()
    if mask.dtype not in (torch.bool, torch.uint8) or not mask.is_contiguous() or mask.dim() < 2:
        raise ValueError("mask must be a contiguous bool or uint8 tensor [..., Tq, Tk]")
    _on_gpu(mask, "mask")
    Tk = mask.shape[-1] if Tk is None else Tk
    if Tk != mask.shape[-1]:
        raise ValueError("Tk does not match the mask")
    rw = lib.fa_mask_row_words(Tk)
    if rw < 0:
        raise ValueError(f"Tk {Tk} out of range")
    rows = mask.numel() // Tk if Tk > 0 else math.prod(mask.shape[:-1])
    shape = tuple(mask.shape[:-1]) + (rw,)
    bits = _out(out, "out", shape, mask, torch.int32)
    bits = torch.empty(shape, dtype=torch.int32, device=mask.device) if bits is None else bits
    st = lib.fa_mask_pack(_ptr(mask), _ptr(bits), rows, Tk, _stream(mask))
    if st != 0:
        raise FaError(st, "fa_mask_pack")
    return bits


def forward_varlen_splitk(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                          causal: bool = False, scale: float | None = None, window: int = 0, mask=None,
                          nsplit: int = 0, workspace=None, out=None, lse=None):
    """fa_fwd_varlen_splitk: forward_varlen (forward_varlen_masked when ``mask`` is given) with
    each sequence's keys split over ``nsplit`` slices (0: automatic) and merged; returns
    (o like q, lse float32 [Hq, total_q])."""
    import torch
    lib = load_library()
    B, Hq, Hkv, total_q, total_k, d = _varlen_shapes(q, k, v, cu_seqlens_q, cu_seqlens_k)
    mq, mk = int(max_seqlen_q), int(max_seqlen_k)
    bits, stride = (None, 0) if mask is None else _varlen_mask_bits(lib, mask, q, B, mq, mk)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = int(lib.fa_fwd_varlen_splitk_workspace_bytes(B, Hq, Hkv, total_q, total_k, mq, mk, d, code, int(nsplit),
                                                        int(mask is not None)))
    ws = _ws(workspace, need, q)
    o = torch.empty_like(q) if _out(out, "out", q.shape, q) is None else out
    L = _out(lse, "lse", (Hq, total_q), q, torch.float32)
    L = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device) if L is None else L
    st = lib.fa_fwd_varlen_splitk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), None if bits is None else _ptr(bits),
                                  stride, cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), ws.data_ptr(),
                                  _nbytes(ws), B, Hq, Hkv, total_q, total_k, mq, mk, d, int(bool(causal)),
                                  int(window), scale, code, int(nsplit), _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd_varlen_splitk")
    return o, L


def _mask_bits(lib, mask, q, B, Tq, Tk):
    """(packed int32 bits, batch stride in words) of a bool/uint8 or already packed mask."""
    import torch
    if mask.device != q.device:
        raise ValueError("mask must be on q's device")
    if mask.dim() == 4 and mask.shape[1] == 1:
        mask = mask[:, 0]
    bits = mask if mask.dtype == torch.int32 else pack_mask(mask.contiguous(), Tk)
    rw = lib.fa_mask_row_words(Tk)
    if not bits.is_contiguous() or tuple(bits.shape[-2:]) != (Tq, rw) or bits.dim() not in (2, 3):
        raise ValueError(f"packed mask must be int32 [Tq, {rw}] or [B, Tq, {rw}]")
    if bits.dim() == 3 and bits.shape[0] not in (1, B):
        raise ValueError("a per-entry mask needs B entries (or one, shared by the batch)")
    return bits, (Tq * rw if bits.dim() == 3 and bits.shape[0] > 1 else 0)


def backward_masked(q, k, v, o, lse, do, mask, causal: bool = False, scale: float | None = None,
                    workspace=None, dq=None, dk=None, dv=None, window: int = 0):
    """fa_bwd_mask: gradients under the boolean mask (and window) of forward_masked; returns
    (dq, dk, dv)."""
    import torch
    lib = load_library()
    B, Hq, Hkv, Tq, Tk, d = _shapes(q, k, v)
    dvh = v.shape[3]
    _out(o, "o", (B, Hq, Tq, dvh), q)
    _out(do, "do", (B, Hq, Tq, dvh), q)
    _out(lse, "lse", (B, Hq, Tq), q, torch.float32)
    bits, stride = _mask_bits(lib, mask, q, B, Tq, Tk)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = int(lib.fa_bwd_mask_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, code, stride))
    ws = _ws(workspace, need, q)
    dq = torch.empty_like(q) if _out(dq, "dq", q.shape, q) is None else dq
    dk = torch.empty_like(k) if _out(dk, "dk", k.shape, q) is None else dk
    dv = torch.empty_like(v) if _out(dv, "dv", v.shape, q) is None else dv
    st = lib.fa_bwd_mask(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                         ws.data_ptr(), _nbytes(ws), _ptr(bits), stride, B, Hq, Hkv, Tq, Tk, d, dvh,
                         int(bool(causal)), int(window), scale, code, _stream(q))
    if st != 0:
        raise FaError(st, "fa_bwd_mask")
    return dq, dk, dv


def forward_masked(q, k, v, mask, causal: bool = False, scale: float | None = None, out=None, lse=None,
                   nsplit: int = 1, workspace=None, window: int = 0):
    """fa_fwd_mask (nsplit == 1) or fa_fwd_mask_splitk: attention under a boolean mask shared by
    all heads of a batch entry (with the causal bound and a sliding window if given).

    ``mask``: bool/uint8 [Tq, Tk] (whole batch) or [B, Tq, Tk] (or [B, 1, Tq, Tk]), packed here
    with fa_mask_pack; or an already packed int32 [..., Tq, fa_mask_row_words(Tk)].
    Returns (o [B, Hq, Tq, dv], lse float32 [B, Hq, Tq])."""
    import torch
    lib = load_library()
    B, Hq, Hkv, Tq, Tk, d = _shapes(q, k, v)
    dvh = v.shape[3]
    bits, stride = _mask_bits(lib, mask, q, B, Tq, Tk)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    o = _out(out, "out", (B, Hq, Tq, dvh), q)
    o = torch.empty((B, Hq, Tq, dvh), dtype=q.dtype, device=q.device) if o is None else o
    L = _out(lse, "lse", (B, Hq, Tq), q, torch.float32)
    L = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if L is None else L
    if nsplit == 1:
        st = lib.fa_fwd_mask(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), _ptr(bits), stride, B, Hq, Hkv, Tq, Tk,
                             d, dvh, int(bool(causal)), int(window), scale, code, _stream(q))
        if st != 0:
            raise FaError(st, "fa_fwd_mask")
        return o, L
    need = int(lib.fa_fwd_mask_splitk_workspace_bytes(B, Hq, Hkv, Tq, Tk, d, dvh, code, int(nsplit)))
    ws = _ws(workspace, need, q)
    st = lib.fa_fwd_mask_splitk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(L), _ptr(bits), stride, ws.data_ptr(),
                                _nbytes(ws), B, Hq, Hkv, Tq, Tk, d, dvh, int(bool(causal)), int(window), scale,
                                code, int(nsplit), _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd_mask_splitk")
    return o, L


def backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None,
             workspace=None, dq=None, dk=None, dv=None, stages: int = STAGE_ALL, window: int = 0):
    """fa_bwd (fa_bwd_stages for a partial stage mask, fa_bwd_window when window > 0):
    returns (dq, dk, dv) like q, k, v."""
    import torch
    lib = load_library()
    B, Hq, Hkv, Tq, Tk, d = _shapes(q, k, v)
    oshape = tuple(q.shape[:3]) + (v.shape[3],)
    _out(o, "o", oshape, q)
    _out(do, "do", oshape, q)
    _out(lse, "lse", (B, Hq, Tq), q, torch.float32)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    code = _dtype_code(q)
    need = workspace_bytes(B, Hq, Hkv, Tq, Tk, d, code)
    ws = _ws(workspace, need, q)
    dq = torch.empty_like(q) if _out(dq, "dq", q.shape, q) is None else dq
    dk = torch.empty_like(k) if _out(dk, "dk", k.shape, q) is None else dk
    dv = torch.empty_like(v) if _out(dv, "dv", v.shape, q) is None else dv
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk),
            _ptr(dv), ws.data_ptr(), _nbytes(ws), B, Hq, Hkv, Tq, Tk, d, int(bool(causal)))
    if v.shape[3] != d:
        st = lib.fa_bwd_dv(*args[:-1], v.shape[3], int(bool(causal)), int(window), scale, code, stages,
                           _stream(q))
        if st != 0:
            raise FaError(st, "fa_bwd_dv")
        return dq, dk, dv
    if window > 0:
        st = lib.fa_bwd_window(*args, int(window), scale, code, stages, _stream(q))
        if st != 0:
            raise FaError(st, "fa_bwd_window")
        return dq, dk, dv
    args = args + (scale, code)
    if stages == STAGE_ALL:
        st = lib.fa_bwd(*args, _stream(q))
    else:
        st = lib.fa_bwd_stages(*args, stages, _stream(q))
    if st != 0:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def backward_noalloc(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None,
                     dq=None, dk=None, dv=None):
    """fa_bwd_noalloc: fa_bwd's gradients with the library's fixed per-device scratch instead of
    a workspace (nothing is allocated by the library; dq, dk, dv may be passed in so that nothing
    is allocated here either).  Returns (dq, dk, dv) like q, k, v."""
    import torch
    lib = load_library()
    B, Hq, Hkv, Tq, Tk, d = _shapes(q, k, v, same_dv=True)
    _out(o, "o", q.shape, q)
    _out(do, "do", q.shape, q)
    _out(lse, "lse", (B, Hq, Tq), q, torch.float32)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q) if _out(dq, "dq", q.shape, q) is None else dq
    dk = torch.empty_like(k) if _out(dk, "dk", k.shape, q) is None else dk
    dv = torch.empty_like(v) if _out(dv, "dv", v.shape, q) is None else dv
    st = lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                            B, Hq, Hkv, Tq, Tk, d, int(bool(causal)), scale, _dtype_code(q), _stream(q))
    if st != 0:
        raise FaError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def _autograd_function():
    import torch

    class FlashAttention(torch.autograd.Function):
        """Autograd wrapper that saves exactly q, k, v, o and lse for the backward."""

        @staticmethod
        def forward(ctx, q, k, v, causal, scale, window, mask):
            if mask is None:
                o, lse = forward(q, k, v, causal, scale, window=window)
            else:
                if mask.dtype != torch.int32:
                    mask = pack_mask(mask.contiguous(), k.shape[2])
                o, lse = forward_masked(q, k, v, mask, causal, scale, window=window)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale, ctx.window, ctx.mask = causal, scale, window, mask
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            if ctx.mask is None:
                dq, dk, dv = backward(q, k, v, o, lse, do.contiguous(), ctx.causal, ctx.scale,
                                      window=ctx.window)
            else:
                dq, dk, dv = backward_masked(q, k, v, o, lse, do.contiguous(), ctx.mask, ctx.causal, ctx.scale,
                                             window=ctx.window)
            return dq, dk, dv, None, None, None, None

    return FlashAttention


_FN = None


def attention(q, k, v, causal: bool = False, scale: float | None = None, window: int = 0, mask=None):
    """Differentiable attention through the library (retains q, k, v, o, lse only, plus the
    packed mask bits when a boolean ``mask`` [Tq, Tk] / [B, Tq, Tk] is given)."""
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    return _FN.apply(q, k, v, causal, scale, window, mask)
