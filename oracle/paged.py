"""Plain fp64 CPU oracle for attention over a page pool: forward and gradients.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it, and this module imports nothing from the product path.

Source: "The Autograd Memory Trap: Diagnosing a Backward-Pass OOM in Chunked
Attention", section "The Scene" (each block of new positions gathers its keys
and values from a prefix cache) and section "The OOM: When Inference Lies"
(the same computation run with gradients enabled: training differentiates
through that gather).

Readings where the page is silent (each is listed in the design notes):

* the prefix cache is a pool of fixed-size pages, K_pages and V_pages
  [num_pages, Hkv, page_size, d]; sequence b has seqlens[b] keys, key j being
  row j % page_size of page table[b, j // page_size];
* the forward of sequence b is ordinary attention (oracle.attention) of its
  queries against its gathered keys, with the causal bound and the window
  end-aligned on its own key count;
* the gradient of the pools is the adjoint of the gather: every gathered row's
  gradient is added into the pool row it was read from, so a page referenced
  by several table entries receives the sum of all of them, rows of a page
  past the sequence's key count receive nothing, and pages that no table entry
  reaches have a zero gradient.

Pins (tests/test_oracle_paged.py): central finite differences of
f = sum(O * dO) with respect to pool entries on shared pages; torch autograd
in float64 through index_select gathers; the identity table reducing to the
plain backward; zeros on unreferenced pages and rows past the key counts.
Parity pinned for every output.
"""

from __future__ import annotations

import numpy as np

from . import attention as oa


def gather(pool, table, seqlens, b):
    """Keys (or values) of sequence b in order: [Hkv, seqlens[b], d] (fp64)."""
    P = pool.shape[2]
    n = int(seqlens[b])
    rows = [np.asarray(pool[int(table[b, j // P]), :, j % P], dtype=np.float64) for j in range(n)]
    if not rows:
        return np.zeros((pool.shape[1], 0, pool.shape[3]))
    return np.stack(rows, axis=1)


def paged_forward(Q, K_pages, V_pages, table, seqlens, causal=False, scale=None, window=0):
    """(O, L) of every sequence against its gathered keys: O [B, Hq, Tq, d], L [B, Hq, Tq]."""
    B, Hq, Tq, d = Q.shape
    O = np.zeros((B, Hq, Tq, V_pages.shape[3]))
    L = np.zeros((B, Hq, Tq))
    for b in range(B):
        k = gather(K_pages, table, seqlens, b)[None]
        v = gather(V_pages, table, seqlens, b)[None]
        Ob, Lb = oa.attention_forward(Q[b:b + 1], k, v, causal, scale, window=window)
        O[b], L[b] = Ob[0], Lb[0]
    return O, L


def scatter_add(grad_pool, grad_rows, table, seqlens, b):
    """Adjoint of gather: add sequence b's row gradients [Hkv, seqlens[b], d] into the pool."""
    P = grad_pool.shape[2]
    for j in range(int(seqlens[b])):
        grad_pool[int(table[b, j // P]), :, j % P] += grad_rows[:, j]


def paged_forward_backward(Q, K_pages, V_pages, table, seqlens, dO, causal=False, scale=None, window=0):
    """(O, L, dQ, dK_pages, dV_pages), fp64: the vector-Jacobian product of
    <O, dO> with respect to Q and the two pools, through the gather."""
    B, Hq, Tq, d = Q.shape
    O = np.zeros((B, Hq, Tq, V_pages.shape[3]))
    L = np.zeros((B, Hq, Tq))
    dQ = np.zeros(Q.shape)
    dKp = np.zeros(K_pages.shape)
    dVp = np.zeros(V_pages.shape)
    for b in range(B):
        k = gather(K_pages, table, seqlens, b)[None]
        v = gather(V_pages, table, seqlens, b)[None]
        Ob, Lb, dQb, dKb, dVb = oa.attention_forward_backward(Q[b:b + 1], k, v, dO[b:b + 1], causal, scale,
                                                              window=window)
        O[b], L[b], dQ[b] = Ob[0], Lb[0], dQb[0]
        scatter_add(dKp, dKb[0], table, seqlens, b)
        scatter_add(dVp, dVb[0], table, seqlens, b)
    return O, L, dQ, dKp, dVp
