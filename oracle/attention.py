"""Plain fp64 CPU oracle for exact attention: forward (O, L) and gradients (dQ, dK, dV).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the HIP
library and its Python binding) never calls it, and this module imports nothing
from the product path.

What it computes, and where each step comes from (web pages, cited by title and
section):

* "What Ordinary Autograd Saves: Tiling the Forward Pass Is Only Half the
  Algorithm", section "The implementation under test": the dense baseline
  softmax(Q K^T / sqrt(d)) V, and the tiled forward with three running
  statistics per row (max m, exponential sum l, unnormalised output), one
  rescale whenever the maximum moves, normalisation once at the end and the
  saved row statistic L = m + ln l (natural logarithm).
* Same page, section "Why this is FlashAttention's second idea": the backward
  keeps O and L and rebuilds the score and probability tiles from them.
* "Backward Pass Implementation", section "Limitations of PyTorch Autograd":
  S = Q K^T / sqrt(d), P = softmax(S), O = P V; and the gradients of a scalar
  loss with respect to Q, K and V are what the backward produces.
* "The Autograd Memory Trap: Diagnosing a Backward-Pass OOM in Chunked
  Attention", sections "Tracing the Autograd Graph" and "The GQA Expansion
  Question": query heads share key/value heads in groups (8 key/value heads
  serve 32 query heads); expanding K and V with repeat_interleave has a
  backward that sums over the repeated heads, so dK and dV are group sums.

Readings where the pages are silent (each is listed in the design notes):

* causal masking is stripped from the printed code; key j is visible to query i
  iff j <= i + (Tk - Tq) (end-aligned; equal to j <= i when Tq == Tk);
* a row with no visible key (Tk == 0, or causal with Tq > Tk) has O = 0,
  L = -inf and contributes nothing to any gradient;
* the backward is the vector-Jacobian product of <O, dO> with respect to Q, K
  and V (L receives no cotangent), written out as the textbook softmax/matmul
  derivative: dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
  dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO;
* the scale is an argument whose default is 1/sqrt(d);
* a sliding window of ``window`` keys (the chunked-attention article's
  sliding-window layers, section "The Reasoning: A Deep Dive into Autograd
  Memory" and its list of subtle mistakes: such layers see a much smaller key
  span than the full-attention layer) lets query i see only keys
  j > i + (Tk - Tq) - window, i.e. at most ``window`` keys ending at its
  end-aligned diagonal position; it combines with the causal bound, and
  window <= 0 means no window;
* a caller's boolean mask (the chunked-attention article, section "The GQA
  Expansion Question": a boolean attention mask together with grouped-query
  heads) is a [Tq, Tk] array, True where key j may be seen by query i, shared
  by every head of a batch entry ([B, Tq, Tk] for one per entry, or [Tq, Tk]
  for the whole batch); it narrows visibility further, after the causal
  bound and the window.

Layouts: Q, dO are [B, Hq, Tq, d]; K is [B, Hkv, Tk, d]; V is [B, Hkv, Tk, dv];
O is [B, Hq, Tq, dv]; L is [B, Hq, Tq].  Query head h reads key/value head
h // (Hq // Hkv).

Pins: every function here is checked against something other than itself in
tests/test_oracle.py (finite differences, brute-force loops with math.fsum,
torch autograd and torch's CPU scaled_dot_product_attention in float64, closed
forms and exact invariants).  Parity pinned for every output.
"""

from __future__ import annotations

import math

import numpy as np


def default_scale(d: int) -> float:
    """1/sqrt(d), the scale of the printed forward and of standard attention."""
    return 1.0 / math.sqrt(d)


def visible(Tq: int, Tk: int, causal: bool, window: int = 0, mask=None) -> np.ndarray:
    """Boolean [Tq, Tk] visibility of key j to query i.

    All True, narrowed by the end-aligned causal bound j <= i + Tk - Tq when
    causal, by the sliding window j > i + Tk - Tq - window when window > 0,
    and by a boolean [Tq, Tk] mask when one is given.
    """
    i = np.arange(Tq)[:, None]
    j = np.arange(Tk)[None, :]
    vis = np.ones((Tq, Tk), dtype=bool)
    if causal:
        vis &= j <= i + (Tk - Tq)
    if window > 0:
        vis &= j > i + (Tk - Tq) - window
    if mask is not None:
        mask = np.asarray(mask, dtype=bool)
        if mask.shape != (Tq, Tk):
            raise ValueError(f"mask must be [{Tq}, {Tk}], got {mask.shape}")
        vis &= mask
    return vis


def _check_shapes(Q, K, V):
    if Q.ndim != 4 or K.ndim != 4 or V.ndim != 4:
        raise ValueError("Q, K, V must be [B, H, T, d]")
    B, Hq, Tq, d = Q.shape
    Bk, Hkv, Tk, dk = K.shape
    if Bk != B or dk != d or V.shape[:3] != (B, Hkv, Tk):
        raise ValueError("inconsistent Q/K/V shapes")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Tq, Tk, d, V.shape[3]


def head_forward(q, k, v, causal, scale, rows=None, Tq=None, window=0, mask=None):
    """One query head against its key/value head, dense, fp64.

    Returns (O [Tq, dv], L [Tq], P [Tq, Tk]).  Steps as in standard attention:
    S = scale q k^T; masked scores do not exist (probability 0); per row
    m = max visible S, l = sum exp(S - m), L = m + ln l, P = exp(S - m) / l;
    O = P v.  With ``rows`` given, q holds only those query rows of a head
    with ``Tq`` rows (the causal mask needs their positions); ``mask`` is the
    head's whole [Tq, Tk] boolean mask in either case.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tk = k.shape[0]
    if rows is None:
        Tq = q.shape[0]
        vis = visible(Tq, Tk, causal, window, mask)
    else:
        vis = visible(Tq, Tk, causal, window, mask)[np.asarray(rows)]
    S = (q @ k.T) * scale
    Sm = np.where(vis, S, -np.inf)
    m = Sm.max(axis=1) if Tk > 0 else np.full(q.shape[0], -np.inf)
    has_key = np.isfinite(m)
    m_safe = np.where(has_key, m, 0.0)
    E = np.where(vis, np.exp(np.where(vis, S, 0.0) - m_safe[:, None]), 0.0)
    l = E.sum(axis=1)
    with np.errstate(divide="ignore"):
        L = np.where(has_key, m_safe + np.log(np.where(has_key, l, 1.0)), -np.inf)
    P = np.where(has_key[:, None], E / np.where(has_key, l, 1.0)[:, None], 0.0)
    O = P @ v
    return O, L, P


def head_backward(q, k, v, dO, O, P, scale):
    """Gradients of sum(O * dO) for one query head: (dq, dk_part, dv_part).

    dP = dO v^T; D = rowsum(dO * O); dS = P * (dP - D); dq = scale dS k;
    dk = scale dS^T q; dv = P^T dO.  Masked entries have P = 0, hence dS = 0.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    dP = dO @ v.T
    D = (dO * O).sum(axis=1)
    dS = P * (dP - D[:, None])
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    dv = P.T @ dO
    return dq, dk, dv


def attention_forward(Q, K, V, causal=False, scale=None, window=0, mask=None):
    """Dense exact attention with GQA: returns O [B,Hq,Tq,dv] and L [B,Hq,Tq] (fp64).

    ``mask``: optional boolean [Tq, Tk] (every batch entry) or [B, Tq, Tk],
    shared by all heads of an entry.
    """
    B, Hq, Hkv, Tq, Tk, d, dv = _check_shapes(Q, K, V)
    if scale is None:
        scale = default_scale(d)
    mask = _batch_masks(mask, B, Tq, Tk)
    G = Hq // Hkv
    O = np.zeros((B, Hq, Tq, dv))
    L = np.zeros((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            O[b, h], L[b, h], _ = head_forward(Q[b, h], K[b, g], V[b, g], causal, scale, window=window,
                                               mask=None if mask is None else mask[b])
    return O, L


def _batch_masks(mask, B, Tq, Tk):
    """A [Tq, Tk] or [B, Tq, Tk] boolean mask as [B, Tq, Tk] (None stays None)."""
    if mask is None:
        return None
    mask = np.asarray(mask, dtype=bool)
    if mask.ndim == 2:
        mask = np.broadcast_to(mask, (B,) + mask.shape)
    if mask.shape != (B, Tq, Tk):
        raise ValueError(f"mask must be [{Tq}, {Tk}] or [{B}, {Tq}, {Tk}], got {mask.shape}")
    return mask


def group_forward_backward(Q, K, V, dO, b, g, causal=False, scale=None, window=0, mask=None):
    """Everything for one (batch b, key/value head g): the G query heads of the group.

    Returns dict with O [G,Tq,dv], L [G,Tq], dQ [G,Tq,d], dK [Tk,d], dV [Tk,dv]
    (fp64).  dK and dV are summed over the group's query heads.  This is the
    unit the full functions loop over and the unit sampled at large sizes.
    ``mask``: optional boolean [Tq, Tk] of batch entry b (or [B, Tq, Tk]).
    """
    B, Hq, Hkv, Tq, Tk, d, dv = _check_shapes(Q, K, V)
    if scale is None:
        scale = default_scale(d)
    G = Hq // Hkv
    if mask is not None and np.ndim(mask) == 3:
        mask = np.asarray(mask, dtype=bool)[b]
    kg = np.asarray(K[b, g], dtype=np.float64)
    vg = np.asarray(V[b, g], dtype=np.float64)
    out = {
        "O": np.zeros((G, Tq, dv)),
        "L": np.zeros((G, Tq)),
        "dQ": np.zeros((G, Tq, d)),
        "dK": np.zeros((Tk, d)),
        "dV": np.zeros((Tk, dv)),
    }
    for r in range(G):
        h = g * G + r
        q = np.asarray(Q[b, h], dtype=np.float64)
        o, lse, p = head_forward(q, kg, vg, causal, scale, window=window, mask=mask)
        dq, dk, dvv = head_backward(q, kg, vg, dO[b, h], o, p, scale)
        out["O"][r], out["L"][r], out["dQ"][r] = o, lse, dq
        out["dK"] += dk
        out["dV"] += dvv
    return out


def attention_forward_backward(Q, K, V, dO, causal=False, scale=None, window=0, mask=None):
    """Full dense forward and backward: (O, L, dQ, dK, dV), all fp64.

    ``mask``: optional boolean [Tq, Tk] (every batch entry) or [B, Tq, Tk].
    """
    B, Hq, Hkv, Tq, Tk, d, dv = _check_shapes(Q, K, V)
    if scale is None:
        scale = default_scale(d)
    mask = _batch_masks(mask, B, Tq, Tk)
    G = Hq // Hkv
    O = np.zeros((B, Hq, Tq, dv))
    L = np.zeros((B, Hq, Tq))
    dQ = np.zeros((B, Hq, Tq, d))
    dK = np.zeros((B, Hkv, Tk, d))
    dV = np.zeros((B, Hkv, Tk, dv))
    for b in range(B):
        for g in range(Hkv):
            r = group_forward_backward(Q, K, V, dO, b, g, causal, scale, window,
                                       None if mask is None else mask[b])
            O[b, g * G:(g + 1) * G] = r["O"]
            L[b, g * G:(g + 1) * G] = r["L"]
            dQ[b, g * G:(g + 1) * G] = r["dQ"]
            dK[b, g] = r["dK"]
            dV[b, g] = r["dV"]
    return O, L, dQ, dK, dV


def tiled_head_forward(q, k, v, block_q, block_k, causal, scale, window=0):
    """The online-softmax recurrence of the printed tiled forward, in fp64.

    Outer loop over query blocks, inner loop over key blocks (the last ones may
    be ragged).  Per row: running max m (starts at -inf), running sum l and
    unnormalised output acc.  For each key block: S = scale q_i k_j^T with
    invisible keys at -inf; m_new = max(m, rowmax S); alpha = exp(m - m_new),
    taken as 0 while m is still -inf; P = exp(S - m_new) (0 where invisible);
    l = alpha l + rowsum P; acc = alpha acc + P v_j.  After the last block,
    O = acc / l and L = m + ln l.  Rows that never see a key keep m = -inf and
    end with O = 0, L = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Tq, Tk, dv = q.shape[0], k.shape[0], v.shape[1]
    O = np.zeros((Tq, dv))
    L = np.full(Tq, -np.inf)
    for i in range(0, Tq, block_q):
        qi = q[i:i + block_q]
        nq = qi.shape[0]
        m = np.full(nq, -np.inf)
        l = np.zeros(nq)
        acc = np.zeros((nq, dv))
        rows = np.arange(i, i + nq)[:, None]
        for j in range(0, Tk, block_k):
            kj, vj = k[j:j + block_k], v[j:j + block_k]
            cols = np.arange(j, j + kj.shape[0])[None, :]
            vis = np.ones((nq, kj.shape[0]), dtype=bool)
            if causal:
                vis &= cols <= rows + (Tk - Tq)
            if window > 0:
                vis &= cols > rows + (Tk - Tq) - window
            S = np.where(vis, (qi @ kj.T) * scale, -np.inf)
            m_new = np.maximum(m, S.max(axis=1))
            alpha = np.zeros(nq)
            had = np.isfinite(m)
            alpha[had] = np.exp(m[had] - m_new[had])
            base = np.where(np.isfinite(m_new), m_new, 0.0)
            P = np.where(vis, np.exp(np.where(vis, S, 0.0) - base[:, None]), 0.0)
            l = l * alpha + P.sum(axis=1)
            acc = acc * alpha[:, None] + P @ vj
            m = m_new
        seen = l > 0
        O[i:i + nq] = np.where(seen[:, None], acc / np.where(seen, l, 1.0)[:, None], 0.0)
        with np.errstate(divide="ignore"):
            L[i:i + nq] = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return O, L


def tiled_forward(Q, K, V, block_q=32, block_k=32, causal=False, scale=None, window=0):
    """tiled_head_forward over every (b, h) with GQA head mapping; fp64 O and L."""
    B, Hq, Hkv, Tq, Tk, d, dv = _check_shapes(Q, K, V)
    if scale is None:
        scale = default_scale(d)
    G = Hq // Hkv
    O = np.zeros((B, Hq, Tq, dv))
    L = np.zeros((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            O[b, h], L[b, h] = tiled_head_forward(Q[b, h], K[b, h // G], V[b, h // G],
                                                  block_q, block_k, causal, scale, window)
    return O, L


def relative_frobenius(x, ref, finite_only=False):
    """||x - ref||_F / ||ref||_F over the whole tensor, in fp64.

    With finite_only, entries where ref is -inf must be -inf in x as well
    (otherwise the result is +inf) and are left out of both norms.
    """
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if finite_only:
        neg = np.isneginf(ref)
        if not np.array_equal(np.isneginf(x), neg):
            return math.inf
        x = x[~neg]
        ref = ref[~neg]
    if not np.all(np.isfinite(x)):
        return math.inf
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return float(num / den)
