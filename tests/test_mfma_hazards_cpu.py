"""The attention kernels' gfx950 assembly leaves every MFMA result alone for at
least 8 wait states on every control-flow path (the requirement of the 4-pass
MFMAs these kernels use: 16x16x32 bf16/f16, 16x16x16 bf16/f16, 16x16x32 fp8).

The compiler enforces this inside a basic block but was seen to drop it for a
read reached through a branch (a maximum taken right after the S^T MFMAs): the
read then picked up stale accumulator values and repeated calls differed.  The
kernels are written so that the first use of an MFMA result sits in the MFMA's
own block; this test holds them to it."""

import os
import shutil

import pytest

from _mfma_hazards import find_hazards, functions

from segmented_attention_paged_amd import build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs hipcc")


def test_checker_flags_a_read_through_a_branch():
    body = """
	v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0
	s_cbranch_scc1 .LBB0_2
; %bb.1:
	s_nop 7
	v_mul_f32_e32 v12, v0, v0
.LBB0_2:
	v_max_f32_e32 v13, v1, v2
	s_endpgm
""".splitlines()
    hz = find_hazards(body)
    assert [(u, w) for _, u, w in hz] == [("v_max_f32_e32 v13, v1, v2", 1)]


def test_checker_accepts_waits_and_chained_accumulation():
    body = """
	v_mfma_f32_16x16x32_bf16 v[0:3], v[4:7], v[8:11], 0
	v_mfma_f32_16x16x32_bf16 v[0:3], v[14:17], v[18:21], v[0:3]
	s_nop 7
	v_mul_f32_e32 v12, v0, v0
	s_endpgm
""".splitlines()
    assert find_hazards(body) == []


def test_attention_kernels_have_no_mfma_hazards(tmp_path):
    src = os.path.join(build.CSRC, "pa_attention.hip")
    asm = open(build.device_asm(src, str(tmp_path / "pa_attention.s"))).read()
    funcs = functions(asm)
    assert sum("attn_kernel" in f for f in funcs) > 10
    bad = {name: hz for name, body in funcs.items() if (hz := find_hazards(body))}
    assert not bad, "\n".join(f"{n}: {hz[:3]}" for n, hz in bad.items())
