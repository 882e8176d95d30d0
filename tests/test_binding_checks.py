"""Argument checks of the Python binding that need no GPU: every one raises before the
library is called, so these run on host tensors.

The key-split forward has no dv argument (its kernels index V with stride d), so a v whose
head dim differs from q's must be refused by the binding, or the forward would read past V's
end."""

import math

import pytest
import torch

import attention_fa_fwd_05_amd as fa
from attention_fa_fwd_05_amd import _binding


def qkv(d=128, dv=64, B=1, Hq=2, Hkv=1, Tq=8, Tk=8, dtype=torch.bfloat16):
    q = torch.zeros(B, Hq, Tq, d, dtype=dtype)
    k = torch.zeros(B, Hkv, Tk, d, dtype=dtype)
    v = torch.zeros(B, Hkv, Tk, dv, dtype=dtype)
    return q, k, v


def test_forward_splitk_refuses_dv_not_d():
    q, k, v = qkv()
    with pytest.raises(ValueError, match="head dim"):
        _binding.forward_splitk(q, k, v)


def test_host_tensors_are_refused():
    q, k, v = qkv(dv=128)
    with pytest.raises(ValueError, match="GPU tensor"):
        _binding.forward(q, k, v)
    with pytest.raises(ValueError, match="GPU tensor"):
        _binding.pack_mask(torch.ones(8, 8, dtype=torch.bool))


@pytest.mark.parametrize("bad", [
    torch.zeros(1, 2, 8, 64),                                  # wrong dtype
    torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16),            # wrong shape
    torch.zeros(1, 2, 64, 8, dtype=torch.bfloat16).transpose(2, 3),   # not contiguous
    torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)[:, :1],     # too small
])
def test_caller_outputs_must_match_exactly(bad):
    like = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        _binding._out(bad, "out", (1, 2, 8, 64), like)
    assert _binding._out(None, "out", (1, 2, 8, 64), like) is None
    good = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    assert _binding._out(good, "out", (1, 2, 8, 64), like) is good


def test_caller_workspace_must_be_large_enough():
    like = torch.zeros(4)
    with pytest.raises(ValueError, match="needed"):
        _binding._ws(torch.zeros(10, dtype=torch.uint8), 11, like)
    ws = torch.zeros(3, dtype=torch.float32)      # 12 bytes
    assert _binding._ws(ws, 12, like) is ws
    assert _binding._nbytes(ws) == 12
