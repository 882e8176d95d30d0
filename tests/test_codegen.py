"""Checks on the gfx950 code the compiler generates for the kernels (CPU only).

The direct global->LDS loads take their LDS base from M0, written by inline
assembly right before each load (csrc/fa_common.h, dma16 / dma16s / dma4).
That is safe only if nothing else writes M0 between the two and the compiler
never keeps a value of its own in M0 across them.  This compiles every kernel
source to assembly with the library's flags and checks that every M0 write
is one of those helper sequences, that no other instruction that reads M0
appears, and that register-indexing brackets (s_set_gpr_idx_on .. _off, which
keep their index in M0; the compiler emits them only in the fp32 d = 128
test-path kernel) contain no direct load.  It also checks that the bf16 kernels keep everything in registers
(no scratch), which the schedules assume (head dim 256's backward excepted),
and that no kernel calls a function (everything is inlined).
"""

import os
import re
import shutil
import subprocess

import pytest

from attention_fa_fwd_05_amd import build

SOURCES = [s for s in build.SOURCES if s != "fa_api.hip"]   # every kernel source
# Instructions that read M0 implicitly on gfx9 (besides the direct loads).
M0_READERS = re.compile(r"^\s*(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_append|ds_consume|v_interp)")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in SOURCES:
        dst = d / (src + ".s")
        cmd = [hipcc, *build.HIPCC_FLAGS, "-I", os.path.join(build.ROOT, "include"), "--cuda-device-only",
               "-S", os.path.join(build.CSRC, src), "-o", str(dst)]
        subprocess.run(cmd, check=True, capture_output=True)
        out[src] = dst.read_text()
    return out


def kernels(text):
    """(name, body) of every kernel function in an assembly listing."""
    parts = re.split(r"^(_ZN2fa\w+):.*$", text, flags=re.M)
    return [(parts[i], parts[i + 1].split(".Lfunc_end")[0]) for i in range(1, len(parts) - 1, 2)]


def test_m0_only_written_by_the_load_helpers(asm):
    for src, text in asm.items():
        for name, body in kernels(text):
            lines = [l.strip() for l in body.splitlines()
                     if l.strip() and not l.strip().startswith((";", ".", "//"))]
            in_idx = False
            for i, l in enumerate(lines):
                assert not M0_READERS.match(l), f"{src}:{name}: {l}"
                if l.startswith("s_set_gpr_idx_on"):
                    in_idx = True
                    continue
                if l.startswith("s_set_gpr_idx_off"):
                    in_idx = False
                    continue
                assert not (in_idx and l.startswith("global_load_lds")), f"{src}:{name}: load inside an index bracket"
                if re.search(r"\bm0\b", l):
                    assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", l), f"{src}:{name}: unexpected M0 use: {l}"
                    nxt = lines[i + 1]
                    assert nxt.startswith("global_load_lds_dword"), f"{src}:{name}: M0 write not followed by a load: {nxt}"
                if l.startswith("global_load_lds_dword"):
                    assert re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", lines[i - 1]), f"{src}:{name}: load without M0 set: {l}"


def test_bf16_kernels_use_no_scratch(asm):
    for src, text in asm.items():
        for m in re.finditer(r"\.amdhsa_kernel (_ZN2fa\w+)(.*?)\.end_amdhsa_kernel", text, flags=re.S):
            name, desc = m.group(1), m.group(2)
            if "DF16b" not in name and "dkdv_pair_kernel" not in name:
                continue
            # head dim 256's backward (a 256-wide dQ accumulator, or half of dK and dV beside the
            # whole of K and V) fills the register file of one wave per SIMD; it may spill.
            if ("dkdv_kernel" in name or "dq_kernel" in name) and "Li256E" in name:
                continue
            size = int(re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", desc).group(1))
            assert size == 0, f"{src}:{name} uses {size} bytes of scratch per lane"


def test_kernels_make_no_calls(asm):
    # Every helper and lambda is inlined into its kernel: a call would pass the
    # kernel's register arrays through scratch and break the hand-ordered
    # schedules (a lambda called from two places once stayed out of line and
    # ran twenty times slower).
    for src, text in asm.items():
        for name, body in kernels(text):
            # (s_setpc_b64 alone is the compiler's long branch inside a large kernel, not a call)
            assert not re.search(r"^\s*s_swappc_b64", body, flags=re.M), f"{src}:{name} calls a function"
