"""The gfx950 assembly of the HIP kernels has no short MFMA-to-read path.

Compiles each kernel source to device assembly with hipcc (CPU only) and checks
that every read of an MFMA result, along every branch path, comes at least 10
wait states after the MFMA (see tests/isa_hazards.py).
"""
import os
import shutil
import subprocess

import pytest

import isa_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "causal_self_attention_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

BAD = """
_Z3badv:
	v_mfma_f32_16x16x4_f32 a[0:3], v1, v2, a[0:3]
	s_cbranch_scc0 .LBB0_2
	s_nop 7
	s_nop 7
.LBB0_2:
	v_accvgpr_read_b32 v0, a0
	s_endpgm
.Lfunc_end0:
"""
GOOD = BAD.replace("s_cbranch_scc0 .LBB0_2", "s_nop 9")


def test_checker_flags_a_branch_into_the_read():
    assert isa_hazards.short_paths(BAD)           # taken branch: 1 wait state
    assert not isa_hazards.short_paths(GOOD)      # straight line: enough


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["attn_fwd.hip", "attn_bwd.hip", "attn_decode.hip", "attn_kv.hip", "attn_materialized.hip",
                                 "attn_prefill.hip"])
def test_kernel_assembly_has_no_short_mfma_read_paths(src, tmp_path):
    out = tmp_path / (src + ".s")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", "-x", "hip", "--cuda-device-only", "-S", "-o", str(out),
                    os.path.join(CSRC, src)], check=True, capture_output=True)
    text = out.read_text()
    assert isa_hazards.functions(text), "no kernels found in the assembly"
    bad = isa_hazards.short_paths(text)
    assert not bad, bad[:5]
