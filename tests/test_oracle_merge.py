"""The (O, L) merge identity behind the key-split forward, on the CPU.

Attention over a key set that is the disjoint union of slices equals the
merge of the per-slice results: with L_s the slice's row logsumexp and O_s its
normalised output, L = ln sum_s exp(L_s) and O = sum_s exp(L_s - L) O_s
(slices where a row sees no key contribute exp(-inf) = 0).  Checked against
the oracle's direct result, with the slices cut out by masking keys.
"""

import numpy as np
import pytest

import oracle.attention as oa


def slice_result(Q, K, V, causal, scale, window, lo, hi):
    """Oracle attention restricted to keys lo .. hi - 1 (others invisible)."""
    Tq, Tk = Q.shape[2], K.shape[2]
    O = np.zeros(Q.shape[:3] + (V.shape[3],))
    L = np.zeros(Q.shape[:3])
    G = Q.shape[1] // K.shape[1]
    keep = np.zeros(Tk, dtype=bool)
    keep[lo:hi] = True
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            vis = oa.visible(Tq, Tk, causal, window) & keep[None, :]
            S = np.where(vis, scale * Q[b, h] @ K[b, h // G].T, -np.inf)
            m = S.max(axis=1)
            ok = np.isfinite(m)
            E = np.where(vis, np.exp(np.where(vis, S, 0) - np.where(ok, m, 0)[:, None]), 0)
            l = E.sum(axis=1)
            with np.errstate(divide="ignore", invalid="ignore"):
                L[b, h] = np.where(ok, np.where(ok, m, 0) + np.log(np.where(ok, l, 1)), -np.inf)
                O[b, h] = np.where(ok[:, None], (E / np.where(ok, l, 1)[:, None]) @ V[b, h // G], 0)
    return O, L


@pytest.mark.parametrize("cuts", [(0, 13, 40), (0, 1, 2, 40), (0, 20, 21, 40)])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 9)])
def test_merge_of_key_slices_equals_full(cuts, causal, window):
    rng = np.random.default_rng(3)
    Q, K, V = rng.standard_normal((1, 4, 6, 5)), rng.standard_normal((1, 2, 40, 5)), rng.standard_normal((1, 2, 40, 5))
    parts = [slice_result(Q, K, V, causal, 0.5, window, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    Ls = np.stack([p[1] for p in parts])
    m = Ls.max(axis=0)
    ok = np.isfinite(m)
    wts = np.where(np.isfinite(Ls), np.exp(Ls - np.where(ok, m, 0)), 0.0)
    wsum = wts.sum(axis=0)
    with np.errstate(divide="ignore"):
        L = np.where(ok, np.where(ok, m, 0) + np.log(np.where(ok, wsum, 1)), -np.inf)
    O = sum(wt[..., None] * p[0] for wt, p in zip(wts, parts)) / np.where(ok, wsum, 1)[..., None]
    Oref, Lref = oa.attention_forward(Q, K, V, causal, 0.5, window=window)
    assert oa.relative_frobenius(O, Oref) < 1e-14
    assert oa.relative_frobenius(L, Lref, finite_only=True) < 1e-14
