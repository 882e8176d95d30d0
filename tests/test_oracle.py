"""Pins for the fp64 oracle: each output checked against something other than itself.

CPU only.  Pins used:
  * central finite differences of f = sum(O * dO) for dQ, dK, dV;
  * a brute-force pure-Python forward (math.exp, math.fsum) for O and L;
  * torch's CPU float64 scaled_dot_product_attention (with enable_gqa) for O,
    torch.logsumexp for L, and torch autograd through it for dQ, dK, dV;
  * the printed tiled recurrence (fp64 port of the recurrence, any block
    sizes, ragged tails) against the dense result;
  * closed forms (one key; all-zero keys) and exact invariants (rows of P sum
    to one, dK sums to zero over keys, dV sums to the summed cotangent, shift
    and permutation invariance, causal prefix independence);
  * GQA equals MHA on repeat_interleave'd K/V with group-summed dK/dV;
  * planted mistakes (in the oracle, on the CPU) each fail at least one pin.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle.attention as oa
from attention_fa_fwd_05_amd import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def small_case(B=1, Hq=2, Hkv=1, Tq=5, Tk=7, d=3, dv=None, seed=0, sigma=1.0):
    dv = d if dv is None else dv
    return (rnd((B, Hq, Tq, d), seed, sigma), rnd((B, Hkv, Tk, d), seed + 1, sigma),
            rnd((B, Hkv, Tk, dv), seed + 2), rnd((B, Hq, Tq, dv), seed + 3))


# ---------------------------------------------------------------- pin helpers

def fd_error(Q, K, V, dO, causal, h=1e-6):
    """Max |oracle grad - central FD| / max |FD| over Q, K and V."""
    scale = 0.7

    def f(q, k, v):
        O, _ = oa.attention_forward(q, k, v, causal, scale)
        return float((O * dO).sum())

    _, _, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, causal, scale)
    worst = 0.0
    for which, analytic in ((0, dQ), (1, dK), (2, dV)):
        args = [Q.copy(), K.copy(), V.copy()]
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
        den = max(np.abs(fd).max(), 1e-300)
        worst = max(worst, float(np.abs(analytic - fd).max() / den))
    return worst


def brute_forward(q, k, v, causal, scale):
    """Pure-Python dense attention for one head: lists in, lists out."""
    Tq, Tk, d, dv = len(q), len(k), len(q[0]) if q else 0, len(v[0]) if v else 0
    O, L = [], []
    for i in range(Tq):
        scores = []
        for j in range(Tk):
            if causal and j > i + Tk - Tq:
                continue
            scores.append((j, scale * math.fsum(q[i][c] * k[j][c] for c in range(d))))
        if not scores:
            O.append([0.0] * dv)
            L.append(-math.inf)
            continue
        mx = max(s for _, s in scores)
        w = [(j, math.exp(s - mx)) for j, s in scores]
        z = math.fsum(e for _, e in w)
        L.append(mx + math.log(z))
        O.append([math.fsum(e * v[j][c] for j, e in w) / z for c in range(dv)])
    return O, L


def brute_error(Q, K, V, causal, scale=0.6):
    O, L = oa.attention_forward(Q, K, V, causal, scale)
    G = Q.shape[1] // K.shape[1]
    worst = 0.0
    for b in range(Q.shape[0]):
        for h in range(Q.shape[1]):
            Ob, Lb = brute_forward(Q[b, h].tolist(), K[b, h // G].tolist(), V[b, h // G].tolist(),
                                   causal, scale)
            Ob, Lb = np.array(Ob).reshape(O[b, h].shape), np.array(Lb)
            if not np.array_equal(np.isneginf(Lb), np.isneginf(L[b, h])):
                return math.inf
            fin = np.isfinite(Lb)
            worst = max(worst, float(np.abs(O[b, h] - Ob).max(initial=0.0)),
                        float(np.abs(L[b, h][fin] - Lb[fin]).max(initial=0.0)))
    return worst


def torch_error(Q, K, V, dO, causal, scale=0.45):
    """Max relative error of oracle (O, L, dQ, dK, dV) vs torch CPU float64 SDPA + autograd."""
    import torch
    import torch.nn.functional as F
    G = Q.shape[1] // K.shape[1]
    Tq, Tk = Q.shape[2], K.shape[2]
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    mask = None
    if causal:
        i = torch.arange(Tq)[:, None]
        j = torch.arange(Tk)[None, :]
        mask = j <= i + (Tk - Tq)
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale, enable_gqa=True)
    (out * torch.tensor(dO)).sum().backward()
    S = torch.matmul(q.detach(), k.detach().repeat_interleave(G, dim=1).transpose(-1, -2)) * scale
    if mask is not None:
        S = S.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(S, dim=-1)
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, causal, scale)
    errs = [oa.relative_frobenius(O, out.detach().numpy()),
            oa.relative_frobenius(L, lse.numpy(), finite_only=True),
            oa.relative_frobenius(dQ, q.grad.numpy()),
            oa.relative_frobenius(dK, k.grad.numpy()),
            oa.relative_frobenius(dV, v.grad.numpy())]
    return max(errs)


def gqa_error(Q, K, V, dO, causal):
    G = Q.shape[1] // K.shape[1]
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, causal)
    Ke, Ve = np.repeat(K, G, axis=1), np.repeat(V, G, axis=1)
    O2, L2, dQ2, dKe, dVe = oa.attention_forward_backward(Q, Ke, Ve, dO, causal)
    B, Hkv, Tk, d = K.shape
    dK2 = dKe.reshape(B, Hkv, G, Tk, d).sum(axis=2)
    dV2 = dVe.reshape(B, Hkv, G, Tk, V.shape[3]).sum(axis=2)
    return max(float(np.abs(a - b).max()) for a, b in
               ((O, O2), (np.nan_to_num(L), np.nan_to_num(L2)), (dQ, dQ2), (dK, dK2), (dV, dV2)))


def tiled_error(Q, K, V, causal, bq, bk):
    O, L = oa.attention_forward(Q, K, V, causal)
    Ot, Lt = oa.tiled_forward(Q, K, V, bq, bk, causal)
    return max(oa.relative_frobenius(Ot, O), oa.relative_frobenius(Lt, L, finite_only=True))


# ---------------------------------------------------------------- the pins

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    dict(B=1, Hq=2, Hkv=1, Tq=5, Tk=7, d=3),          # GQA, Tk > Tq
    dict(B=2, Hq=1, Hkv=1, Tq=6, Tk=4, d=2, dv=3),    # Tq > Tk: causal rows with no key
    dict(B=1, Hq=3, Hkv=3, Tq=4, Tk=4, d=4),          # square MHA
])
def test_gradients_match_finite_differences(shape, causal):
    assert fd_error(*small_case(**shape), causal) < 1e-7


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    dict(B=1, Hq=2, Hkv=1, Tq=5, Tk=7, d=3),
    dict(B=1, Hq=1, Hkv=1, Tq=9, Tk=4, d=5, dv=2),
    dict(B=2, Hq=4, Hkv=2, Tq=6, Tk=6, d=4, sigma=3.0),
])
def test_forward_matches_bruteforce_fsum(shape, causal):
    Q, K, V, _ = small_case(**shape)
    assert brute_error(Q, K, V, causal) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [
    dict(B=2, Hq=4, Hkv=2, Tq=33, Tk=47, d=8),
    dict(B=1, Hq=4, Hkv=1, Tq=40, Tk=40, d=16, sigma=3.0),
])
def test_matches_torch_sdpa_float64(shape, causal):
    assert torch_error(*small_case(**shape), causal) < 1e-12


def test_rows_of_p_sum_to_one_and_l_is_logsumexp():
    q, k, v = rnd((37, 8), 1), rnd((53, 8), 2), rnd((53, 8), 3)
    for causal in (False, True):
        O, L, P = oa.head_forward(q, k, v, causal, 0.35)
        assert np.abs(P.sum(axis=1) - 1.0).max() < 1e-13
        vis = oa.visible(37, 53, causal)
        for i in range(37):
            s = [0.35 * float(q[i] @ k[j]) for j in range(53) if vis[i, j]]
            assert abs(L[i] - math.log(math.fsum(math.exp(x) for x in s))) < 1e-12
        assert np.all(P[~vis] == 0.0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blocks", [(1, 1), (7, 7), (32, 32), (7, 32), (64, 5), (10**6, 10**6)])
def test_tiled_recurrence_matches_dense(blocks, causal):
    Q, K, V, _ = small_case(B=1, Hq=2, Hkv=1, Tq=45, Tk=71, d=8, seed=5, sigma=3.0)
    assert tiled_error(Q, K, V, causal, *blocks) < 1e-12


def test_tiled_recurrence_rows_without_keys():
    Q, K, V, _ = small_case(B=1, Hq=1, Hkv=1, Tq=20, Tk=6, d=4, seed=9)
    O, L = oa.tiled_forward(Q, K, V, 4, 3, causal=True)
    assert np.all(np.isneginf(L[0, 0, :14])) and np.all(O[0, 0, :14] == 0.0)
    assert tiled_error(Q, K, V, True, 4, 3) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeat_interleave_with_group_sums(causal):
    assert gqa_error(*small_case(B=2, Hq=8, Hkv=2, Tq=9, Tk=11, d=4, seed=3), causal) < 1e-13


def test_closed_form_single_key():
    Q, K, V, dO = small_case(B=1, Hq=2, Hkv=1, Tq=6, Tk=1, d=4, seed=11)
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, False, 0.5)
    assert np.allclose(O, np.broadcast_to(V[:, :1], O.shape), atol=1e-15, rtol=0)
    assert np.allclose(L, 0.5 * np.einsum("bhtd,bd->bht", Q, K[:, 0, 0]), atol=1e-14, rtol=0)
    assert np.abs(dQ).max() < 1e-14 and np.abs(dK).max() < 1e-14
    assert np.allclose(dV[0, 0, 0], dO[0].sum(axis=(0, 1)), atol=1e-13, rtol=0)


def test_closed_form_zero_keys_uniform_weights():
    Q, _, V, _ = small_case(B=1, Hq=1, Hkv=1, Tq=9, Tk=9, d=4, seed=12)
    K = np.zeros((1, 1, 9, 4))
    O, L = oa.attention_forward(Q, K, V, False)
    assert np.allclose(O[0, 0], np.broadcast_to(V[0, 0].mean(axis=0), (9, 4)), atol=1e-14, rtol=0)
    assert np.allclose(L, math.log(9), atol=1e-14, rtol=0)
    O, L = oa.attention_forward(Q, K, V, True)
    prefix = np.cumsum(V[0, 0], axis=0) / np.arange(1, 10)[:, None]
    assert np.allclose(O[0, 0], prefix, atol=1e-14, rtol=0)
    assert np.allclose(L[0, 0], np.log(np.arange(1, 10)), atol=1e-14, rtol=0)


def test_empty_key_set():
    Q = rnd((1, 2, 5, 4), 0)
    K = np.zeros((1, 1, 0, 4))
    V = np.zeros((1, 1, 0, 4))
    dO = rnd((1, 2, 5, 4), 1)
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, False)
    assert np.all(O == 0) and np.all(np.isneginf(L)) and np.all(dQ == 0)
    assert dK.shape == (1, 1, 0, 4) and dV.shape == (1, 1, 0, 4)


@pytest.mark.parametrize("causal", [False, True])
def test_exact_invariants(causal):
    Q, K, V, dO = small_case(B=2, Hq=4, Hkv=2, Tq=12, Tk=12, d=5, seed=21)
    scale = 0.4
    O, L, dQ, dK, dV = oa.attention_forward_backward(Q, K, V, dO, causal, scale)
    # rows of dS sum to zero, so summing dK over keys gives zero
    assert np.abs(dK.sum(axis=2)).max() < 1e-12
    # rows of P sum to one, so summing dV over keys gives the group's summed cotangent
    G = 2
    expect = dO.reshape(2, 2, G, 12, 5).sum(axis=(2, 3))
    assert np.abs(dV.sum(axis=2) - expect).max() < 1e-12
    # shifting every key by the same vector c leaves O and adds scale*q.c to L
    c = rnd((5,), 99)
    O2, L2 = oa.attention_forward(Q, K + c, V, causal, scale)
    assert np.abs(O2 - O).max() < 1e-12
    assert np.abs(L2 - (L + scale * (Q @ c))).max() < 1e-12
    if not causal:
        perm = np.random.default_rng(5).permutation(12)
        O3, L3, dQ3, dK3, dV3 = oa.attention_forward_backward(Q, K[:, :, perm], V[:, :, perm], dO,
                                                               causal, scale)
        assert np.abs(O3 - O).max() < 1e-12 and np.abs(L3 - L).max() < 1e-12
        assert np.abs(dQ3 - dQ).max() < 1e-12
        assert np.abs(dK3 - dK[:, :, perm]).max() < 1e-12
        assert np.abs(dV3 - dV[:, :, perm]).max() < 1e-12
    else:
        # query i cannot see keys beyond i (Tq == Tk): changing them leaves row i alone
        K4, V4 = K.copy(), V.copy()
        K4[:, :, 7:] += 5.0
        V4[:, :, 7:] -= 3.0
        O4, L4 = oa.attention_forward(Q, K4, V4, causal, scale)
        assert np.abs(O4[:, :, :7] - O[:, :, :7]).max() < 1e-14
        assert np.abs(L4[:, :, :7] - L[:, :, :7]).max() < 1e-14


def test_relative_frobenius():
    a = np.array([3.0, 4.0])
    assert oa.relative_frobenius(a, a) == 0.0
    assert abs(oa.relative_frobenius(a + np.array([0.3, 0.4]), a) - 0.1) < 1e-15
    assert oa.relative_frobenius(np.array([-np.inf, 1.0]), np.array([-np.inf, 1.0]), True) == 0.0
    assert oa.relative_frobenius(np.array([0.0, 1.0]), np.array([-np.inf, 1.0]), True) == math.inf
    assert oa.relative_frobenius(np.array([np.nan, 1.0]), np.array([0.0, 1.0])) == math.inf


# ---------------------------------------------------------------- planted mistakes

def _mutant_backward_no_D(q, k, v, dO, O, P, scale):
    dP = np.asarray(dO) @ np.asarray(v).T
    dS = P * dP                                   # dropped "- D"
    return scale * (dS @ k), scale * (dS.T @ q), P.T @ dO


def _mutant_backward_unscaled_dk(q, k, v, dO, O, P, scale):
    dP = np.asarray(dO) @ np.asarray(v).T
    D = (dO * O).sum(axis=1)
    dS = P * (dP - D[:, None])
    return scale * (dS @ k), dS.T @ q, P.T @ dO   # dK without the scale


def _mutant_backward_sign(q, k, v, dO, O, P, scale):
    dP = np.asarray(dO) @ np.asarray(v).T
    D = (dO * O).sum(axis=1)
    dS = P * (D[:, None] - dP)                    # wrong sign
    return scale * (dS @ k), scale * (dS.T @ q), P.T @ dO


def _mutant_forward_log2(q, k, v, causal, scale, rows=None, Tq=None, window=0, mask=None):
    O, L, P = _ORIG_HEAD_FORWARD(q, k, v, causal, scale, rows, Tq, window=window, mask=mask)
    return O, L / math.log(2.0), P                # L in log2


def _mutant_visible_start_aligned(Tq, Tk, causal, window=0, mask=None):
    if not causal:
        return np.ones((Tq, Tk), dtype=bool)
    return np.arange(Tk)[None, :] <= np.arange(Tq)[:, None]


_ORIG_HEAD_FORWARD = oa.head_forward


def _mutant_gqa_modulo(Q, K, V, causal=False, scale=None, window=0, mask=None):
    B, Hq, Hkv, Tq, Tk, d, dv = oa._check_shapes(Q, K, V)
    scale = oa.default_scale(d) if scale is None else scale
    O = np.zeros((B, Hq, Tq, dv))
    L = np.zeros((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            O[b, h], L[b, h], _ = oa.head_forward(Q[b, h], K[b, h % Hkv], V[b, h % Hkv], causal, scale,
                                                  window=window)
    return O, L


def _all_pins_pass():
    """Run a compact version of every pin; True iff all pass."""
    c1 = small_case(B=1, Hq=2, Hkv=1, Tq=4, Tk=6, d=3, seed=31)
    c2 = small_case(B=1, Hq=4, Hkv=2, Tq=7, Tk=5, d=3, seed=32)
    c3 = small_case(B=1, Hq=4, Hkv=2, Tq=16, Tk=20, d=4, seed=33)
    return (fd_error(*c1, True) < 1e-7 and fd_error(*c1, False) < 1e-7
            and brute_error(*c2[:3], True) < 1e-12 and brute_error(*c2[:3], False) < 1e-12
            and torch_error(*c3, True) < 1e-12 and gqa_error(*c3, False) < 1e-13
            and tiled_error(*c3[:3], True, 5, 3) < 1e-12)


def test_unmutated_oracle_passes_compact_pins():
    assert _all_pins_pass()


@pytest.mark.parametrize("target,mutant", [
    ("head_backward", _mutant_backward_no_D),
    ("head_backward", _mutant_backward_unscaled_dk),
    ("head_backward", _mutant_backward_sign),
    ("head_forward", _mutant_forward_log2),
    ("visible", _mutant_visible_start_aligned),
    ("attention_forward", _mutant_gqa_modulo),
])
def test_planted_mistakes_are_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(oa, target, mutant)
    assert not _all_pins_pass()


# ---------------------------------------------------------------- printed numbers

def test_dense_retained_bytes_reproduce_printed_table():
    tab = json.load(open(os.path.join(GOLDEN, "retained_payload_table.json")))
    d = tab["setup"]["d"]
    for row in tab["rows"]:
        T = row["T"]
        dense = accounting.retained_bytes_dense(1, 1, 1, T, T, d, "fp32")
        assert dense == row["dense_kib"] * 1024
        assert abs(row["tiled_kib"] / row["dense_kib"] - row["ratio"]) < 0.006
    t0, t1 = tab["rows"][0], tab["rows"][-1]
    red0 = t0["tiled_kib"] * 1024 / accounting.checkpoint_payload_bytes(t0["T"], d, d)
    red1 = t1["tiled_kib"] * 1024 / accounting.checkpoint_payload_bytes(t1["T"], d, d)
    assert round(red0) == tab["recompute"]["reduction_T128_approx"]
    assert round(red1) == tab["recompute"]["reduction_T1024_approx"]


def test_chunk_arithmetic_reproduces_article():
    g = json.load(open(os.path.join(GOLDEN, "chunk_arithmetic.json")))
    assert g["max_prefix"] + g["block_len"] == g["max_kv"]
    per_block = accounting.kv_block_bytes(g["heads_expanded"], g["max_kv"], g["head_dim"], g["elem_bytes"])
    assert round(per_block / 1e6, 1) == g["bytes_per_block_mb"]
    blocks = int(g["budget_bytes"] // per_block)
    assert blocks == g["blocks_per_chunk_approx"]
    assert math.ceil(g["anchors"] / blocks) == g["chunks_approx"]
    assert g["heads_expanded"] // g["kv_heads"] == g["gqa_expansion"]


def test_flop_count_convention():
    f, b = accounting.flops(4, 32, 4096, 4096, 128, True)
    assert f == 2 * 4096 * 4096 * 128 * 128 and b == 5 * 4096 * 4096 * 128 * 128
    assert abs((f + b) / 1e9 - 1924.145) < 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_row_subset_matches_bruteforce(causal):
    q, k, v = rnd((30, 6), 41), rnd((23, 6), 42), rnd((23, 5), 43)
    rows = np.array([0, 3, 7, 8, 29])
    O, L, _ = oa.head_forward(q[rows], k, v, causal, 0.5, rows=rows, Tq=30)
    Ob, Lb = brute_forward(q.tolist(), k.tolist(), v.tolist(), causal, 0.5)
    Ob, Lb = np.array(Ob)[rows], np.array(Lb)[rows]
    assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
    fin = np.isfinite(Lb)
    assert np.abs(O - Ob).max() < 1e-12 and np.abs(L[fin] - Lb[fin]).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_row_subset_dq_matches_full_backward(causal):
    """dQ of a query row depends only on that row's P, dP and D, so the backward
    applied to a row subset (as the long-sequence GPU check does) gives exactly
    those rows of the full head's dQ (itself pinned by finite differences and
    torch autograd above).  Rows 0..3 of a causal Tq > Tk head see no key."""
    Tq, Tk = 40, 31
    q, k, v, dO = rnd((Tq, 6), 51), rnd((Tk, 6), 52), rnd((Tk, 6), 53), rnd((Tq, 6), 54)
    O, L, P = oa.head_forward(q, k, v, causal, 0.7)
    dq_full, _, _ = oa.head_backward(q, k, v, dO, O, P, 0.7)
    rows = np.array([0, 2, 9, 10, 27, 39])
    Or, Lr, Pr = oa.head_forward(q[rows], k, v, causal, 0.7, rows=rows, Tq=Tq)
    dq_rows, _, _ = oa.head_backward(q[rows], k, v, dO[rows], Or, Pr, 0.7)
    assert np.abs(dq_rows - dq_full[rows]).max() < 1e-12
    if causal:
        assert np.all(dq_rows[0] == 0.0)
