"""Seeded synthetic workloads: shapes, seeds and input tensors.

This module holds no attention arithmetic.  It draws Q, K, V and the output
cotangent dO from a seeded generator, and rounds them to bfloat16 where the
workload computes in bfloat16, so that the HIP path and the CPU checker receive
bit-identical inputs.

Recipe (for every workload): ``numpy.random.default_rng(seed)``, four
``standard_normal(..., dtype=float32)`` draws in the order Q [B,Hq,Tq,d],
K [B,Hkv,Tk,d], V [B,Hkv,Tk,dv], dO [B,Hq,Tq,dv] (dv = d unless stated); Q and K are then multiplied
by ``sigma_qk`` in float32 (1 unless stated); for bfloat16 workloads each
value is rounded to bfloat16 with round-to-nearest-even on the float32 bits.
"""

from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    d: int
    dtype: str          # "fp32" or "bf16": storage type of Q, K, V, O, dO, dQ, dK, dV
    causal: bool
    seed: int
    sigma_qk: float = 1.0
    window: int = 0      # > 0: sliding window of that many keys (query i sees j > i + Tk - Tq - window)
    dv: int = 0          # head dim of V and O (and dO) when it differs from d; 0 means d

    @property
    def dvv(self) -> int:
        return self.dv or self.d

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads the parity tests and the benchmark run.  Names state what each
# one is.  The first is the small single-head case at the printed experiment's
# tile size (32x32 blocks, d = 64); the second has a ragged last tile; the last
# has the long-sequence shape of the chunked-attention article (32 query heads
# over 8 key/value heads, 8000 queries against 8000 + 32 keys, d = 128).
WORKLOADS = {
    w.name: w for w in [
        Workload("mha_fp32_T128_d64", 1, 1, 1, 128, 128, 64, "fp32", False, 0),
        Workload("mha_fp32_T1000_d64", 4, 8, 8, 1000, 1000, 64, "fp32", False, 2),
        Workload("mha_fp32_T1000_d64_causal", 4, 8, 8, 1000, 1000, 64, "fp32", True, 2),
        Workload("mha_fp32_T1000_d64_sigma3", 4, 8, 8, 1000, 1000, 64, "fp32", False, 23, 3.0),
        Workload("mha_fp32_T1000_d64_sigma3_causal", 4, 8, 8, 1000, 1000, 64, "fp32", True, 23, 3.0),
        Workload("mha_bf16_T2048_d128_causal", 8, 16, 16, 2048, 2048, 128, "bf16", True, 3),
        Workload("gqa_bf16_T4096_d128_causal", 4, 32, 8, 4096, 4096, 128, "bf16", True, 4),
        Workload("gqa_bf16_T8000x8032_d128", 1, 32, 8, 8000, 8032, 128, "bf16", False, 5),
        # 16 blocks of 32 new positions, each against its own 8000 + 32 key prefix
        # (the article's drafter block shape), forward only
        Workload("gqa_bf16_B16_Tq32_Tk8032_d128_causal", 16, 32, 8, 32, 8032, 128, "bf16", True, 7),
        # the same shape under the article's sliding-window layers: 2080 keys per query
        Workload("gqa_bf16_T8000x8032_d128_causal_window2080", 1, 32, 8, 8000, 8032, 128, "bf16", True, 6,
                 window=2080),
    ]
}

# The benchmark's headline workload: d = 128, T = 4096, GQA 32/8, causal, bf16.
HEADLINE = "gqa_bf16_T4096_d128_causal"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); uint16 bits.

    Inputs are finite normal draws, so no NaN/inf handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Host copies of one workload's inputs.

    ``q, k, v, do`` are float32 arrays holding exactly the values the device
    receives (already bfloat16-representable for bf16 workloads); ``bits``
    holds the uint16 bfloat16 patterns for bf16 workloads (None for fp32).
    """
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: np.ndarray
    bits: dict | None


def make_inputs(w: Workload, seed: int | None = None) -> Inputs:
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = rng.standard_normal((w.B, w.Hq, w.Tq, w.d), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.Tk, w.d), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.Tk, w.dvv), dtype=np.float32)
    do = rng.standard_normal((w.B, w.Hq, w.Tq, w.dvv), dtype=np.float32)
    if w.sigma_qk != 1.0:
        q *= np.float32(w.sigma_qk)
        k *= np.float32(w.sigma_qk)
    if w.dtype == "fp32":
        return Inputs(q, k, v, do, None)
    if w.dtype != "bf16":
        raise ValueError(f"unknown dtype {w.dtype}")
    bits = {n: f32_to_bf16_bits(a) for n, a in (("q", q), ("k", k), ("v", v), ("do", do))}
    return Inputs(*(bf16_bits_to_f32(bits[n]) for n in ("q", "k", "v", "do")), bits)


def to_device(inp: Inputs, dtype: str, device="cuda"):
    """Torch device tensors (q, k, v, do) holding exactly ``inp``'s values."""
    import torch
    if dtype == "fp32":
        return tuple(torch.from_numpy(a).to(device) for a in (inp.q, inp.k, inp.v, inp.do))
    return tuple(torch.from_numpy(inp.bits[n].view(np.int16)).view(torch.bfloat16).to(device)
                 for n in ("q", "k", "v", "do"))
