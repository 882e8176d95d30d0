"""Pins for the oracle's boolean attention mask (CPU only).

Reading (the chunked-attention article, section "The GQA Expansion Question":
a caller's boolean attention mask used together with grouped-query heads): a
[Tq, Tk] boolean array, True where query i may see key j, shared by every head
of a batch entry, narrowing the causal bound when both are given; a row left
with no key has O = 0 and L = -inf.  Pins, each independent of the oracle's own
code path:
  * torch's CPU float64 scaled_dot_product_attention with the same boolean
    attn_mask and enable_gqa (O), and torch.logsumexp over the masked scores
    (L), for a shared and a per-entry mask, with and without the causal bound;
  * a pure-Python brute-force forward that tests the mask per (i, j) pair and
    sums with math.fsum;
  * exact invariants: an all-True mask is the unmasked call, the causal
    pattern as a mask is the causal call, a row with no True entry gives
    O = 0, L = -inf;
  * a planted mistake (the mask read transposed) fails the SDPA pin;
  * gradients under the mask: torch autograd through the same float64 SDPA
    call (a row without keys has no gradient), and central finite differences
    of sum(O * dO).
"""

import math

import numpy as np
import pytest

import oracle.attention as oa


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def inputs(B=2, Hq=4, Hkv=2, Tq=11, Tk=11, d=5, seed=0):
    return rnd((B, Hq, Tq, d), seed), rnd((B, Hkv, Tk, d), seed + 1), rnd((B, Hkv, Tk, d), seed + 2)


def random_mask(shape, seed, density=0.5):
    return np.random.default_rng(seed).random(shape) < density


def sdpa(Q, K, V, mask, causal, scale):
    """torch's SDPA in float64 with an explicit boolean mask (True = may attend)."""
    import torch
    import torch.nn.functional as F
    B, Hq, Tq, _ = Q.shape
    Tk = K.shape[2]
    m = torch.tensor(np.broadcast_to(mask, (B, Tq, Tk)).copy())
    if causal:
        i = torch.arange(Tq)[:, None]
        j = torch.arange(Tk)[None, :]
        m = m & (j <= i + Tk - Tq)[None]
    rows = m.any(dim=-1)                                   # [B, Tq]
    q, k, v = (torch.tensor(x) for x in (Q, K, V))
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=m[:, None], scale=scale, enable_gqa=True)
    out = torch.where(rows[:, None, :, None], out, torch.zeros_like(out))
    G = Hq // K.shape[1]
    S = torch.matmul(q, k.repeat_interleave(G, dim=1).transpose(-1, -2).contiguous()) * scale
    lse = torch.logsumexp(S.masked_fill(~m[:, None], -math.inf), dim=-1)
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("per_entry", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Tq,Tk", [(11, 11), (7, 13), (13, 6)])
def test_mask_matches_torch_sdpa(per_entry, causal, Tq, Tk):
    Q, K, V = inputs(Tq=Tq, Tk=Tk, seed=3)
    mask = random_mask((2, Tq, Tk) if per_entry else (Tq, Tk), seed=5, density=0.6)
    O, L = oa.attention_forward(Q, K, V, causal, 0.45, mask=mask)
    Ot, Lt = sdpa(Q, K, V, mask, causal, 0.45)
    assert oa.relative_frobenius(O, Ot) < 1e-12
    assert oa.relative_frobenius(L, Lt, finite_only=True) < 1e-12


def brute(q, k, v, mask, scale):
    Tq, Tk = len(q), len(k)
    O, L = np.zeros((Tq, v.shape[1])), np.full(Tq, -math.inf)
    for i in range(Tq):
        keys = [j for j in range(Tk) if mask[i][j]]
        if not keys:
            continue
        s = {j: scale * math.fsum(float(q[i][c]) * float(k[j][c]) for c in range(len(q[i]))) for j in keys}
        m = max(s.values())
        w = {j: math.exp(s[j] - m) for j in keys}
        tot = math.fsum(w.values())
        L[i] = m + math.log(tot)
        for c in range(v.shape[1]):
            O[i, c] = math.fsum(w[j] * float(v[j][c]) for j in keys) / tot
    return O, L


def test_mask_matches_brute_force():
    Q, K, V = inputs(B=1, Hq=2, Hkv=1, Tq=6, Tk=9, d=3, seed=8)
    mask = random_mask((6, 9), seed=9, density=0.4)
    mask[2] = False                                          # one row with no key
    O, L = oa.attention_forward(Q, K, V, False, 0.8, mask=mask)
    for h in range(2):
        Ob, Lb = brute(Q[0, h], K[0, 0], V[0, 0], mask, 0.8)
        fin = np.isfinite(Lb)
        assert np.array_equal(np.isneginf(L[0, h]), ~fin)
        assert np.abs(L[0, h][fin] - Lb[fin]).max() < 1e-12
        assert np.abs(O[0, h] - Ob).max() < 1e-12


def test_mask_invariants():
    Q, K, V = inputs(Tq=9, Tk=12, seed=11)
    O0, L0 = oa.attention_forward(Q, K, V, False, 0.5)
    O1, L1 = oa.attention_forward(Q, K, V, False, 0.5, mask=np.ones((9, 12), dtype=bool))
    assert np.array_equal(O0, O1) and np.array_equal(L0, L1)
    i, j = np.arange(9)[:, None], np.arange(12)[None, :]
    Oc, Lc = oa.attention_forward(Q, K, V, True, 0.5)
    Om, Lm = oa.attention_forward(Q, K, V, False, 0.5, mask=j <= i + 3)
    assert np.array_equal(Oc, Om) and np.array_equal(Lc, Lm)
    empty = np.ones((9, 12), dtype=bool)
    empty[4] = False
    Oe, Le = oa.attention_forward(Q, K, V, False, 0.5, mask=empty)
    assert np.all(Oe[:, :, 4] == 0.0) and np.all(np.isneginf(Le[:, :, 4]))
    assert np.all(np.isfinite(np.delete(Le, 4, axis=2)))


def test_mask_per_entry_equals_separate_calls():
    Q, K, V = inputs(Tq=8, Tk=10, seed=13)
    mask = random_mask((2, 8, 10), seed=14)
    O, L = oa.attention_forward(Q, K, V, True, 0.5, mask=mask)
    for b in range(2):
        Ob, Lb = oa.attention_forward(Q[b:b + 1], K[b:b + 1], V[b:b + 1], True, 0.5, mask=mask[b])
        assert np.array_equal(O[b:b + 1], Ob) and np.array_equal(L[b:b + 1], Lb)


def test_planted_transposed_mask_fails_sdpa_pin():
    Q, K, V = inputs(Tq=10, Tk=10, seed=17)
    mask = random_mask((10, 10), seed=18, density=0.5)
    assert not np.array_equal(mask, mask.T)
    Ot, _ = sdpa(Q, K, V, mask, False, 0.5)
    O_bad, _ = oa.attention_forward(Q, K, V, False, 0.5, mask=mask.T)
    assert oa.relative_frobenius(O_bad, Ot) > 1e-3


def test_mask_shape_is_checked():
    Q, K, V = inputs(Tq=5, Tk=6, seed=1)
    with pytest.raises(ValueError):
        oa.attention_forward(Q, K, V, False, 0.5, mask=np.ones((6, 5), dtype=bool))


@pytest.mark.parametrize("per_entry", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_mask_gradients_match_torch_autograd(per_entry, causal):
    """dQ, dK, dV under the mask: torch autograd through float64 SDPA with the same mask."""
    import torch
    import torch.nn.functional as F
    Tq, Tk = 9, 12
    Q, K, V = inputs(Tq=Tq, Tk=Tk, seed=21)
    dO = rnd(Q.shape, 22)
    mask = random_mask((2, Tq, Tk) if per_entry else (Tq, Tk), seed=23, density=0.5)
    mask[..., 3, :] = False                                  # a row without keys: no gradient
    m = torch.tensor(np.broadcast_to(mask, (2, Tq, Tk)).copy())
    if causal:
        m = m & (torch.arange(Tk)[None, :] <= torch.arange(Tq)[:, None] + Tk - Tq)[None]
    rows = m.any(dim=-1)
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=m[:, None], scale=0.6, enable_gqa=True)
    out = torch.where(rows[:, None, :, None], out, torch.zeros_like(out))
    (out * torch.tensor(dO)).sum().backward()
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, causal, 0.6, mask=mask)
    assert oa.relative_frobenius(O, out.detach().numpy()) < 1e-12
    assert oa.relative_frobenius(dQ, np.nan_to_num(q.grad.numpy())) < 1e-12
    assert oa.relative_frobenius(dK, np.nan_to_num(k.grad.numpy())) < 1e-12
    assert oa.relative_frobenius(dV, np.nan_to_num(v.grad.numpy())) < 1e-12


def test_mask_gradients_match_finite_differences():
    Q, K, V = inputs(B=1, Hq=2, Hkv=1, Tq=5, Tk=7, d=3, seed=25)
    dO = rnd(Q.shape, 26)
    mask = random_mask((5, 7), seed=27, density=0.6)
    scale, hstep = 0.7, 1e-6

    def f(q, k, v):
        O, _ = oa.attention_forward(q, k, v, False, scale, mask=mask)
        return float((O * dO).sum())

    _, _, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, False, scale, mask=mask)
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


def test_group_unit_takes_the_entry_mask():
    Q, K, V = inputs(Tq=8, Tk=10, seed=29)
    dO = rnd(Q.shape, 30)
    mask = random_mask((2, 8, 10), seed=31)
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, True, 0.5, mask=mask)
    r = oa.group_forward_backward(Q, K, V, dO, 1, 1, True, 0.5, mask=mask)
    assert np.array_equal(r["O"], O[1, 2:4]) and np.array_equal(r["dK"], dK[1, 1])
    r2 = oa.group_forward_backward(Q, K, V, dO, 1, 1, True, 0.5, mask=mask[1])
    assert np.array_equal(r2["dV"], dV[1, 1])
