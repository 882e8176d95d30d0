"""GPU parity on seeded random configurations against the fp64 oracle.

Forty configurations drawn from a fixed seed across the option space the
other parity tests cover one by one: dtype, head dims (32, 64, 128; bf16 256;
dv != d as (128, 64) and (64, 128)), group sizes 1, 2, 4 and 8, batch 1 to 3,
lengths 1 to 400 with Tq != Tk both ways, causal or not, a sliding window or
none, and a boolean mask (shared or per entry) on some of them.  Small sizes
keep the oracle fast; the random lengths land anywhere relative to the tiles,
so ragged tails, single rows and rows without keys all occur.  O, L, dQ, dK,
dV: whole-tensor relative Frobenius error 1e-4 (fp32) / 2e-2 (bf16) and the
per-row bound of parity_tools.
"""

import numpy as np
import pytest

import oracle.attention as oa
from attention_fa_fwd_05_amd import workloads as wl
from parity_tools import check, errors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa(require_gpu):
    import attention_fa_fwd_05_amd as fa_mod
    fa_mod.load_library()
    return fa_mod


def draw(i):
    rng = np.random.default_rng(9000 + i)
    dtype = "bf16" if rng.random() < 0.7 else "fp32"
    heads = [(32, 32), (64, 64), (128, 128), (128, 64), (64, 128)] + ([(256, 256)] if dtype == "bf16" else [])
    d, dv = heads[rng.integers(len(heads))]
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 3))
    B = int(rng.integers(1, 4))
    Tq, Tk = int(rng.integers(1, 401)), int(rng.integers(1, 401))
    causal = bool(rng.random() < 0.6)
    window = int(rng.integers(1, 300)) if rng.random() < 0.3 else 0
    masked = bool(rng.random() < 0.3)
    per_entry = bool(rng.random() < 0.5)
    return dict(dtype=dtype, d=d, dv=dv, Hq=G * Hkv, Hkv=Hkv, B=B, Tq=Tq, Tk=Tk, causal=causal, window=window,
                masked=masked, per_entry=per_entry, seed=9000 + i)


CASES = [draw(i) for i in range(40)]


def name(c):
    return (f"{c['dtype']}_B{c['B']}_H{c['Hq']}x{c['Hkv']}_Tq{c['Tq']}_Tk{c['Tk']}_d{c['d']}"
            f"{'_dv' + str(c['dv']) if c['dv'] != c['d'] else ''}{'_causal' if c['causal'] else ''}"
            f"{'_w' + str(c['window']) if c['window'] else ''}{'_mask' if c['masked'] else ''}")


@pytest.mark.parametrize("c", CASES, ids=[name(c) for c in CASES])
def test_random_configuration(fa, c):
    import torch
    print(f"case {name(c)}", flush=True)
    w = wl.Workload(name(c), c["B"], c["Hq"], c["Hkv"], c["Tq"], c["Tk"], c["d"], c["dtype"], c["causal"],
                    c["seed"], window=c["window"], dv=c["dv"] if c["dv"] != c["d"] else 0)
    inp = wl.make_inputs(w)
    q, k, v, do = wl.to_device(inp, w.dtype)
    mask = None
    if c["masked"]:
        shape = (w.B, w.Tq, w.Tk) if c["per_entry"] else (w.Tq, w.Tk)
        mask = np.random.default_rng(c["seed"] + 1).random(shape) < 0.6
        m = torch.from_numpy(mask).cuda()
        o, lse = fa.forward_masked(q, k, v, m, w.causal, w.scale, window=w.window)
        dq, dk, dv = fa.backward_masked(q, k, v, o, lse, do, m, w.causal, w.scale, window=w.window)
    else:
        o, lse = fa.forward(q, k, v, w.causal, w.scale, window=w.window)
        dq, dk, dv = fa.backward(q, k, v, o, lse, do, w.causal, w.scale, window=w.window)
    torch.cuda.synchronize()
    got = {n: t.float().cpu().numpy() for n, t in (("O", o), ("L", lse), ("dQ", dq), ("dK", dk), ("dV", dv))}
    ref = dict(zip(("O", "L", "dQ", "dK", "dV"),
                   oa.attention_forward_backward(inp.q, inp.k, inp.v, inp.do, w.causal, w.scale, window=w.window,
                                                 mask=mask)))
    empty = np.isneginf(ref["L"])
    assert np.isneginf(got["L"][empty]).all() and not got["O"][empty].any() and not got["dQ"][empty].any()
    check(name(c), w.dtype, errors(got, ref))
