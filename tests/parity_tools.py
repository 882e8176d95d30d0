"""Comparison helpers shared by the GPU parity tests (not collected by pytest).

Two measures per output tensor X against the oracle X*:

* the whole-tensor relative Frobenius error ||X - X*|| / ||X*|| (the stated
  tolerance: 1e-4 for fp32 storage, 2e-2 for bf16 storage with fp32
  accumulation); L rows that are -inf in the oracle must be -inf exactly and
  are left out of the norm;
* a per-row bound, so that one wrong row cannot hide inside a large tensor
  (over a 131072-row group a completely wrong row moves the whole-tensor error
  by only about 0.004): for every row i (the last axis is the row's feature
  axis; L is one value per row) ||x_i - x*_i|| <= ROW_TOL * max(||x*_i||, f),
  with the floor f = RMS_i ||x*_i||, so that rows whose exact value nearly
  cancels are measured against the tensor's typical row size: a causal row
  that sees one key has dQ = 0 exactly, while the bf16 path leaves a residue of
  the order of the rounding of O (D is formed from the stored O).  A wrong row
  of typical size still shows an error near 1.  For L the row error is
  |L_i - L*_i| against max(1, |L*_i|).
"""

import numpy as np

import oracle.attention as oa

TOL = {"fp32": 1e-4, "bf16": 2e-2}
# A row may be off by 10% of the larger of its own size and the typical row size in bf16
# (the worst bf16 rows are the early causal rows, whose exact dQ nearly cancels: about 0.06 at
# T = 4096), 0.1% in fp32; a wrong row shows an error near 1.
ROW_TOL = {"fp32": 1e-3, "bf16": 1e-1}


def log(msg):
    print(msg, flush=True)


def row_error(x, ref, is_L=False):
    """Largest per-row error of x against ref (see module note)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if is_L:
        ninf = np.isneginf(ref)
        if not np.array_equal(np.isneginf(x), ninf):
            return float("inf")
        if (~ninf).sum() == 0:
            return 0.0
        return float((np.abs(x[~ninf] - ref[~ninf]) / np.maximum(1.0, np.abs(ref[~ninf]))).max())
    if ref.size == 0:
        return 0.0
    xr = x.reshape(-1, x.shape[-1])
    rr = ref.reshape(-1, ref.shape[-1])
    rn = np.linalg.norm(rr, axis=1)
    floor = np.sqrt(np.mean(rn * rn))
    if floor == 0.0:
        return float(np.abs(xr).max()) if xr.size else 0.0
    return float((np.linalg.norm(xr - rr, axis=1) / np.maximum(rn, floor)).max())


def errors(got: dict, ref: dict) -> dict:
    """{name: (whole-tensor relative Frobenius, worst row)} for every output in ref."""
    out = {}
    for n, r in ref.items():
        isL = n == "L"
        out[n] = (oa.relative_frobenius(got[n], r, finite_only=isL), row_error(got[n], r, is_L=isL))
    return out


def check(name, dtype, errs):
    log(f"{name}: " + " ".join(f"{k}={v[0]:.2e}/row {v[1]:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not (v[0] <= TOL[dtype] and v[1] <= ROW_TOL[dtype])}
    assert not bad, f"{name}: over tolerance (Frobenius {TOL[dtype]}, row {ROW_TOL[dtype]}): {bad}"


class Accum:
    """Whole-tensor relative Frobenius error and worst row accumulated over parts (groups) of a
    tensor that is compared piece by piece."""

    def __init__(self):
        self.num, self.den, self.row = {}, {}, {}

    def add(self, name, x, ref):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        isL = name == "L"
        if isL:
            ninf = np.isneginf(ref)
            assert np.array_equal(np.isneginf(x), ninf), f"{name}: -inf rows differ"
            x, ref = x[~ninf], ref[~ninf]
        self.num[name] = self.num.get(name, 0.0) + float(np.sum((x - ref) ** 2))
        self.den[name] = self.den.get(name, 0.0) + float(np.sum(ref * ref))

    def add_rows(self, name, x, ref):
        self.row[name] = max(self.row.get(name, 0.0), row_error(x, ref, is_L=(name == "L")))

    def result(self) -> dict:
        return {n: (float(np.sqrt(self.num[n] / self.den[n])) if self.den[n] > 0 else 0.0, self.row.get(n, 0.0))
                for n in self.num}
