"""Pins for the page-pool oracle (oracle/paged.py), CPU only.

  * central finite differences of f = sum(O * dO), O from the paged forward,
    with respect to every pool entry, including pages shared by several
    sequences, the rows of a page past a key count and pages no table entry
    reaches (where the difference is exactly zero);
  * torch autograd in float64 through index_select gathers from the pools;
  * the identity table (each sequence owns its pages, in order, all full)
    reduces to the plain backward of oracle.attention;
  * planted mistakes in the scatter (overwrite instead of add, a dropped
    key-count bound, a wrong row index) each fail a pin.
"""

import math

import numpy as np
import pytest

import oracle.attention as oa
import oracle.paged as op


def pooled_case(lens, P, Hq=2, Hkv=1, Tq=3, d=3, extra=2, share=True, seed=0):
    """A shuffled pool; when ``share`` the first page of sequence 0 is also the
    first page of every other sequence (a common prefix), and ``extra`` pages
    are referenced by no entry."""
    rng = np.random.default_rng(seed)
    B = len(lens)
    pps = max(1, max((n + P - 1) // P for n in lens))
    own = [max(1, (n + P - 1) // P) for n in lens]
    num_pages = sum(own) + extra
    order = rng.permutation(num_pages)
    table = np.full((B, pps), order[-1], dtype=np.int32)     # unused slots point at a spare page
    nxt = 0
    for b in range(B):
        for s in range(own[b]):
            table[b, s] = order[nxt]
            nxt += 1
    if share:
        table[1:, 0] = table[0, 0]
    Kp = rng.standard_normal((num_pages, Hkv, P, d))
    Vp = rng.standard_normal((num_pages, Hkv, P, d))
    Q = rng.standard_normal((B, Hq, Tq, d))
    dO = rng.standard_normal((B, Hq, Tq, d))
    return Q, Kp, Vp, table, np.array(lens, dtype=np.int32), dO


def read_rows(table, lens, shape):
    """Boolean pool mask: True on the rows some sequence gathers."""
    read = np.zeros(shape, dtype=bool)
    P = shape[2]
    for b, n in enumerate(lens):
        for j in range(int(n)):
            read[int(table[b, j // P]), :, j % P] = True
    return read


def fd_error(Q, Kp, Vp, table, lens, dO, causal, window=0, h=1e-6):
    scale = 0.8
    _, _, dQ, dKp, dVp = op.paged_forward_backward(Q, Kp, Vp, table, lens, dO, causal, scale, window)

    def f(q, k, v):
        O, _ = op.paged_forward(q, k, v, table, lens, causal, scale, window)
        return float((O * dO).sum())

    worst = 0.0
    for which, analytic in ((0, dQ), (1, dKp), (2, dVp)):
        args = [Q.copy(), Kp.copy(), Vp.copy()]
        fd = np.zeros_like(args[which])
        it = np.nditer(fd, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            base = args[which][idx]
            args[which][idx] = base + h
            fp = f(*args)
            args[which][idx] = base - h
            fm = f(*args)
            args[which][idx] = base
            fd[idx] = (fp - fm) / (2 * h)
        # pool rows that no sequence reads: exactly zero on both sides
        if which > 0:
            unread = ~read_rows(table, lens, Kp.shape)
            if analytic[unread].any() or fd[unread].any():
                return math.inf
        den = max(np.abs(fd).max(), 1e-300)
        worst = max(worst, float(np.abs(analytic - fd).max() / den))
    return worst


def torch_error(Q, Kp, Vp, table, lens, dO, causal, window=0, scale=0.5):
    """Oracle vs torch float64 autograd through index_select gathers from the pools."""
    import torch
    P = Kp.shape[2]
    kp, vp, q = (torch.tensor(x, requires_grad=True) for x in (Kp, Vp, Q))
    total = 0.0
    for b in range(Q.shape[0]):
        n = int(lens[b])
        j = torch.arange(n)
        page = torch.tensor(table[b])[j // P]
        flat = page * P + j % P                                   # row index into [num_pages * P]
        k = kp.permute(1, 0, 2, 3).reshape(Kp.shape[1], -1, Kp.shape[3]).index_select(1, flat)
        v = vp.permute(1, 0, 2, 3).reshape(Vp.shape[1], -1, Vp.shape[3]).index_select(1, flat)
        G = Q.shape[1] // Kp.shape[1]
        k, v = k.repeat_interleave(G, dim=0), v.repeat_interleave(G, dim=0)
        S = torch.matmul(q[b], k.transpose(-1, -2)) * scale
        Tq = Q.shape[2]
        i = torch.arange(Tq)[:, None]
        jj = torch.arange(n)[None, :]
        vis = torch.ones(Tq, n, dtype=torch.bool)
        if causal:
            vis &= jj <= i + (n - Tq)
        if window > 0:
            vis &= jj > i + (n - Tq) - window
        S = S.masked_fill(~vis, -math.inf)
        Pm = torch.softmax(S, dim=-1).nan_to_num(0.0)
        total = total + (torch.matmul(Pm, v) * torch.tensor(dO[b])).sum()
    total.backward()
    _, _, dQ, dKp, dVp = op.paged_forward_backward(Q, Kp, Vp, table, lens, dO, causal, scale, window)
    return max(oa.relative_frobenius(dQ, q.grad.numpy()), oa.relative_frobenius(dKp, kp.grad.numpy()),
               oa.relative_frobenius(dVp, vp.grad.numpy()))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens,P,window", [
    ([5, 3], 2, 0),          # shared first page, tails inside a page
    ([1, 4, 6], 4, 0),       # one-key sequence, Tq > key count under causal
    ([6, 6], 3, 2),          # window
])
def test_pool_gradients_match_finite_differences(lens, P, window, causal):
    assert fd_error(*pooled_case(lens, P, seed=len(lens) + P), causal, window) < 1e-7


@pytest.mark.parametrize("causal", [False, True])
def test_pool_gradients_match_torch_autograd(causal):
    case = pooled_case([40, 17, 64, 1], 16, Hq=4, Hkv=2, Tq=9, d=8, seed=5)
    assert torch_error(*case, causal) < 1e-12
    assert torch_error(*case, causal, window=7) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_identity_table_is_the_plain_backward(causal):
    rng = np.random.default_rng(9)
    B, Hq, Hkv, Tq, Tk, d, P = 2, 4, 2, 6, 12, 5, 4
    Q, K, V, dO = (rng.standard_normal(s) for s in ((B, Hq, Tq, d), (B, Hkv, Tk, d), (B, Hkv, Tk, d),
                                                    (B, Hq, Tq, d)))
    pps = Tk // P
    # page b * pps + s holds rows s*P .. s*P+P-1 of sequence b
    Kp = K.reshape(B, Hkv, pps, P, d).transpose(0, 2, 1, 3, 4).reshape(B * pps, Hkv, P, d)
    Vp = V.reshape(B, Hkv, pps, P, d).transpose(0, 2, 1, 3, 4).reshape(B * pps, Hkv, P, d)
    table = np.arange(B * pps, dtype=np.int32).reshape(B, pps)
    O, L, dQ, dKp, dVp = op.paged_forward_backward(Q, Kp, Vp, table, np.full(B, Tk), dO, causal)
    O2, L2, dQ2, dK2, dV2 = oa.attention_forward_backward(Q, K, V, dO, causal)
    back = lambda x: x.reshape(B, pps, Hkv, P, d).transpose(0, 2, 1, 3, 4).reshape(B, Hkv, Tk, d)
    for a, b in ((O, O2), (L, L2), (dQ, dQ2), (back(dKp), dK2), (back(dVp), dV2)):
        np.testing.assert_array_equal(a, b)


def test_unreferenced_pages_and_rows_past_the_key_count_are_zero():
    Q, Kp, Vp, table, lens, dO = pooled_case([5, 3], 4, extra=3, seed=2)
    _, _, _, dKp, dVp = op.paged_forward_backward(Q, Kp, Vp, table, lens, dO, True)
    used = set(table[0, :2].tolist()) | {int(table[1, 0])}
    for pg in range(Kp.shape[0]):
        if pg not in used:
            assert not dKp[pg].any() and not dVp[pg].any()
    # page table[0, 1] holds keys 4 .. 7 of sequence 0, which has 5: rows 1 .. 3 get nothing
    assert not dKp[table[0, 1], :, 1:].any() and dKp[table[0, 1], :, 0].any()


# ---------------------------------------------------------------- planted mistakes

def _mutant_overwrite(grad_pool, grad_rows, table, seqlens, b):
    P = grad_pool.shape[2]
    for j in range(int(seqlens[b])):
        grad_pool[int(table[b, j // P]), :, j % P] = grad_rows[:, j]


def _mutant_whole_page(grad_pool, grad_rows, table, seqlens, b):
    # rows past the key count receive the last valid row's gradient
    P = grad_pool.shape[2]
    n = int(seqlens[b])
    for j in range(((n + P - 1) // P) * P):
        grad_pool[int(table[b, j // P]), :, j % P] += grad_rows[:, min(j, n - 1)]


def _mutant_row_index(grad_pool, grad_rows, table, seqlens, b):
    P = grad_pool.shape[2]
    for j in range(int(seqlens[b])):
        grad_pool[int(table[b, j // P]), :, (P - 1 - j % P)] += grad_rows[:, j]


@pytest.mark.parametrize("mutant", [_mutant_overwrite, _mutant_whole_page, _mutant_row_index])
def test_planted_scatter_mistakes_are_caught(monkeypatch, mutant):
    case = pooled_case([5, 3], 2, seed=4)
    assert fd_error(*case, True) < 1e-7
    monkeypatch.setattr(op, "scatter_add", mutant)
    assert not fd_error(*case, True) < 1e-7
