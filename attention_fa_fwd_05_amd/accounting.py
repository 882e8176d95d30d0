"""Work and memory accounting for the attention path (host-side arithmetic only).

Counted FLOPs: per (batch, query head) the forward counts 4*Tq*Tk*d (two
matrix products of 2*Tq*Tk*d) and the backward 10*Tq*Tk*d (five products:
the score recompute, dP, dV, dK, dQ), both halved when causal.  This is the
conventional count; the exact causal visible fraction is slightly above one
half and is not what is reported.

Retained-for-backward bytes: the recompute backward keeps Q, K, V, O (storage
dtype) and the fp32 row statistic L, all linear in T.  The dense baseline
keeps Q, K, V and the Tq x Tk probability matrix; for one head in fp32 this
is (3*T*d + T*T) * 4 bytes, which reproduces the dense column of the
measurement table on "What Ordinary Autograd Saves" (section "The
measurement") exactly, and 3*T*d*4 bytes is the recomputed payload of the
section "The way out is recomputation".
"""

from __future__ import annotations

DTYPE_BYTES = {"fp32": 4, "bf16": 2}


def flops(B, Hq, Tq, Tk, d, causal):
    """(forward, backward) counted FLOPs."""
    f = 4.0 * B * Hq * Tq * Tk * d
    b = 10.0 * B * Hq * Tq * Tk * d
    if causal:
        f, b = f / 2, b / 2
    return f, b


def kernel_flops(B, Hq, Tq, Tk, d, causal, window=0):
    """Matrix FLOPs each kernel performs (halved when causal; exactly counted
    visible pairs under a sliding window).

    Per visible (query, key) pair: forward 4d (S and PV); dK/dV pass 8d (S, dP,
    dV, dK); dQ pass 6d (S, dP, dQ).  The two backward passes together do 14d,
    4d more than the 10d the backward is credited with, because each rebuilds
    S and dP for itself.
    """
    if window > 0:
        pairs = float(B * Hq * visible_pairs(Tq, Tk, causal, window))
    else:
        pairs = B * Hq * Tq * Tk * (0.5 if causal else 1.0)
    return {"fwd_kernel": 4.0 * d * pairs, "dkdv_kernel": 8.0 * d * pairs, "dq_kernel": 6.0 * d * pairs}


def visible_pairs(Tq, Tk, causal, window=0):
    """Exact number of visible (query, key) pairs of one head.

    Query i sees keys lo(i) .. hi(i) with hi = min(Tk - 1, i + Tk - Tq) when
    causal (else Tk - 1) and lo = max(0, i + Tk - Tq - window + 1) for a
    sliding window (else 0).
    """
    import numpy as np
    i = np.arange(Tq, dtype=np.int64)
    off = Tk - Tq
    hi = np.minimum(Tk - 1, i + off) if causal else np.full(Tq, Tk - 1, dtype=np.int64)
    lo = np.maximum(0, i + off - window + 1) if window > 0 else np.zeros(Tq, dtype=np.int64)
    return int(np.maximum(0, hi - lo + 1).sum())


def window_flops(B, Hq, Tq, Tk, d, causal, window):
    """(forward, backward) FLOPs of a sliding-window workload: 4d and 10d per
    exactly visible pair (the causal-halving convention has no analogue for a
    window, so the pairs are counted)."""
    p = float(B * Hq * visible_pairs(Tq, Tk, causal, window))
    return 4.0 * d * p, 10.0 * d * p


def retained_bytes_recompute(B, Hq, Hkv, Tq, Tk, d, dtype):
    """Q, K, V, O in the storage dtype plus fp32 L: what the backward keeps."""
    e = DTYPE_BYTES[dtype]
    return e * (2 * B * Hq * Tq * d + 2 * B * Hkv * Tk * d) + 4 * B * Hq * Tq


def retained_bytes_dense(B, Hq, Hkv, Tq, Tk, d, dtype):
    """Q, K, V plus the Tq x Tk probability matrix per query head, storage dtype."""
    e = DTYPE_BYTES[dtype]
    return e * (B * Hq * Tq * d + 2 * B * Hkv * Tk * d + B * Hq * Tq * Tk)


def checkpoint_payload_bytes(T, d, dv, elem=4):
    """Inputs only (Q, K, V of one head): the payload left when everything is recomputed."""
    return elem * (2 * T * d + T * dv)


def kv_block_bytes(heads, max_kv, d, elem=2):
    """K and V for one block of `heads` expanded heads of max_kv keys (chunked-attention article)."""
    return 2 * heads * max_kv * d * elem


def min_hbm_bytes(B, Hq, Hkv, Tq, Tk, d, dtype):
    """(forward, backward) compulsory HBM traffic.

    Forward reads Q, K, V and writes O, L.  Backward reads Q, K, V, O, dO, L
    and writes dQ, dK, dV.
    """
    e = DTYPE_BYTES[dtype]
    q = B * Hq * Tq * d * e
    kv = B * Hkv * Tk * d * e
    lse = B * Hq * Tq * 4
    fwd = q + 2 * kv + q + lse
    bwd = 3 * q + 2 * kv + lse + q + 2 * kv
    return fwd, bwd
