"""Pins for the oracle's sliding-window mask (CPU only).

Reading (the chunked-attention article's sliding-window layers, which see a
much smaller key span than full attention): with window W > 0, query i sees
key j only if j > i + (Tk - Tq) - W, on top of the end-aligned causal bound
j <= i + (Tk - Tq) when causal.  Pins, each independent of the oracle's own
code path:
  * a pure-Python brute-force forward whose visibility test is written out
    per (i, j) pair, summed with math.fsum;
  * torch's CPU float64 scaled_dot_product_attention with a boolean mask built
    here, and torch autograd through it for the gradients;
  * central finite differences of sum(O * dO);
  * closed forms: causal W = 1 leaves each query exactly its diagonal key
    (O_i = V_(i+Tk-Tq), L_i = its score, dQ = dK = 0, dV_j = sum of the dO
    rows that see j); W >= Tq + Tk equals no window;
  * the tiled online-softmax recurrence with the window against the dense
    result, for blocks that split the window;
  * a planted off-by-one in the window bound fails the brute-force pin.
"""

import math

import numpy as np
import pytest

import oracle.attention as oa


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def case(B=1, Hq=2, Hkv=1, Tq=7, Tk=9, d=3, seed=0):
    return (rnd((B, Hq, Tq, d), seed), rnd((B, Hkv, Tk, d), seed + 1),
            rnd((B, Hkv, Tk, d), seed + 2), rnd((B, Hq, Tq, d), seed + 3))


def brute(q, k, v, causal, window, scale):
    Tq, Tk = len(q), len(k)
    O, L = [], []
    for i in range(Tq):
        diag = i + Tk - Tq
        sc = []
        for j in range(Tk):
            if causal and j > diag:
                continue
            if window > 0 and diag - j >= window:
                continue
            sc.append((j, scale * math.fsum(a * b for a, b in zip(q[i], k[j]))))
        if not sc:
            O.append([0.0] * len(v[0]))
            L.append(-math.inf)
            continue
        mx = max(s for _, s in sc)
        w = [(j, math.exp(s - mx)) for j, s in sc]
        z = math.fsum(e for _, e in w)
        L.append(mx + math.log(z))
        O.append([math.fsum(e * v[j][c] for j, e in w) / z for c in range(len(v[0]))])
    return np.array(O), np.array(L)


WINDOWS = [1, 2, 3, 5]
SHAPES = [dict(Tq=7, Tk=9), dict(Tq=9, Tk=6), dict(Tq=8, Tk=8)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("causal", [False, True])
def test_window_forward_matches_bruteforce(shape, window, causal):
    Q, K, V, _ = case(**shape)
    O, L = oa.attention_forward(Q, K, V, causal, 0.6, window=window)
    for h in range(Q.shape[1]):
        Ob, Lb = brute(Q[0, h].tolist(), K[0, 0].tolist(), V[0, 0].tolist(), causal, window, 0.6)
        assert np.array_equal(np.isneginf(Lb), np.isneginf(L[0, h]))
        fin = np.isfinite(Lb)
        assert np.abs(L[0, h][fin] - Lb[fin]).max(initial=0.0) < 1e-12
        assert np.abs(O[0, h] - Ob).max() < 1e-12


@pytest.mark.parametrize("window", [1, 3, 6])
@pytest.mark.parametrize("causal", [False, True])
def test_window_matches_torch_sdpa_with_explicit_mask(window, causal):
    import torch
    import torch.nn.functional as F
    Q, K, V, dO = case(B=2, Hq=4, Hkv=2, Tq=13, Tk=17, d=5, seed=4)
    Tq, Tk = 13, 17
    mask = torch.zeros(Tq, Tk, dtype=torch.bool)
    for i in range(Tq):
        for j in range(Tk):
            ok = (not causal or j <= i + Tk - Tq) and i + Tk - Tq - j < window
            mask[i, j] = ok
    rows = mask.any(dim=1)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=0.5, enable_gqa=True)
    # rows without keys: SDPA gives NaN there; the reading is O = 0 and no gradient
    out = torch.where(rows[None, None, :, None], out, torch.zeros_like(out))
    (out * torch.tensor(dO)).sum().backward()
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, causal, 0.5, window=window)
    assert oa.relative_frobenius(O, out.detach().numpy()) < 1e-12
    assert oa.relative_frobenius(dQ, np.nan_to_num(q.grad.numpy())) < 1e-12
    assert oa.relative_frobenius(dK, np.nan_to_num(k.grad.numpy())) < 1e-12
    assert oa.relative_frobenius(dV, np.nan_to_num(v.grad.numpy())) < 1e-12
    S = torch.matmul(torch.tensor(Q), torch.tensor(K).repeat_interleave(2, dim=1).transpose(-1, -2)) * 0.5
    lse = torch.logsumexp(S.masked_fill(~mask, -math.inf), dim=-1)
    assert oa.relative_frobenius(L, lse.numpy(), finite_only=True) < 1e-12


@pytest.mark.parametrize("window", [2, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_window_gradients_match_finite_differences(window, causal):
    Q, K, V, dO = case(Tq=6, Tk=8, d=3, seed=7)
    scale, hstep = 0.7, 1e-6

    def f(q, k, v):
        O, _ = oa.attention_forward(q, k, v, causal, scale, window=window)
        return float((O * dO).sum())

    _, _, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, causal, scale, window=window)
    for which, analytic in ((0, dQ), (1, dK), (2, dV)):
        args = [Q.copy(), K.copy(), V.copy()]
        fd = np.zeros_like(args[which])
        for idx in np.ndindex(fd.shape):
            base = args[which][idx]
            args[which][idx] = base + hstep
            fp = f(*args)
            args[which][idx] = base - hstep
            fm = f(*args)
            args[which][idx] = base
            fd[idx] = (fp - fm) / (2 * hstep)
        assert np.abs(analytic - fd).max() / np.abs(fd).max() < 1e-7


def test_causal_window_one_is_the_diagonal_key():
    Q, K, V, dO = case(B=1, Hq=2, Hkv=1, Tq=5, Tk=8, d=4, seed=11)
    Tq, Tk = 5, 8
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, True, 0.3, window=1)
    diag = np.arange(Tq) + Tk - Tq
    for h in range(2):
        assert np.allclose(O[0, h], V[0, 0][diag], atol=0, rtol=1e-15)
        assert np.allclose(L[0, h], 0.3 * (Q[0, h] * K[0, 0][diag]).sum(axis=1), atol=1e-15)
    assert np.abs(dQ).max() < 1e-15 and np.abs(dK).max() < 1e-15
    expect = np.zeros_like(dV[0, 0])
    for h in range(2):
        expect[diag] += dO[0, h]
    assert np.allclose(dV[0, 0], expect, atol=1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_wide_window_equals_no_window(causal):
    Q, K, V, dO = case(B=1, Hq=2, Hkv=1, Tq=9, Tk=11, d=4, seed=3)
    a = oa.attention_forward_backward(Q, K, V, dO, causal, 0.4, window=20)
    b = oa.attention_forward_backward(Q, K, V, dO, causal, 0.4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("window", [3, 10, 33])
@pytest.mark.parametrize("blocks", [(1, 1), (4, 5), (16, 7)])
def test_window_tiled_recurrence_matches_dense(window, blocks):
    Q, K, V, _ = case(B=1, Hq=1, Hkv=1, Tq=37, Tk=45, d=6, seed=5)
    O, L = oa.attention_forward(Q, K, V, True, 0.5, window=window)
    Ot, Lt = oa.tiled_forward(Q, K, V, blocks[0], blocks[1], True, 0.5, window=window)
    assert oa.relative_frobenius(Ot, O) < 1e-13
    assert oa.relative_frobenius(Lt, L, finite_only=True) < 1e-13


def test_planted_window_off_by_one_is_caught(monkeypatch):
    def wrong(Tq, Tk, causal, window=0, mask=None):
        i = np.arange(Tq)[:, None]
        j = np.arange(Tk)[None, :]
        vis = np.ones((Tq, Tk), dtype=bool)
        if causal:
            vis &= j <= i + (Tk - Tq)
        if window > 0:
            vis &= j >= i + (Tk - Tq) - window      # one key too many
        return vis
    monkeypatch.setattr(oa, "visible", wrong)
    with pytest.raises(AssertionError):
        test_window_forward_matches_bruteforce(dict(Tq=7, Tk=9), 2, True)
