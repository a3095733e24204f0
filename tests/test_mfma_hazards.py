"""Wait states around the inline-assembly MFMAs of the pipelined backward kernels.

The dK/dV and dQ kernels issue their MFMAs from inline assembly (explicit
register classes), which the compiler's hazard recognizer does not see.
These tests compile both sources for gfx950 and check every instance with
tests/mfma_hazards.py, and that no instruction other than the copies'
set_m0 writes M0; planted listings show that the checker catches each kind
of hazard.
"""

import os
import tempfile

import pytest

from tests.mfma_hazards import check, compile_to_asm, functions, m0_writers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_attn_amd", "csrc")


def test_checker_catches_planted_hazards():
    raw_in = [
        "v_accvgpr_read_b32 v15, a3",
        "v_mfma_f32_32x32x16_bf16 v[32:47], v[4:7], a[8:11], v[0:15]",
    ]
    assert any("accumulator input" in p for p in check(raw_in))
    in_place = [
        "v_mov_b64_e32 v[14:15], 0",
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
    ]
    assert any("accumulator input" in p for p in check(in_place))
    agpr_back = [
        "v_accvgpr_write_b32 a15, v3",
        "s_waitcnt lgkmcnt(4)",
        "v_mfma_f32_32x32x16_bf16 a[0:15], v[16:19], v[20:23], a[0:15]",
    ]
    assert any("accumulator input" in p for p in check(agpr_back))
    guarded = ["v_accvgpr_write_b32 a15, v3", "s_nop 4", "v_mfma_f32_32x32x16_bf16 a[0:15], v[16:19], v[20:23], a[0:15]"]
    assert check(guarded) == []
    war_c = [
        "v_mfma_f32_32x32x16_bf16 v[32:47], v[4:7], a[8:11], v[0:15]",
        "s_nop 7",
        "v_mov_b32_e32 v3, 0",
    ]
    assert any("accumulator input overwritten" in p for p in check(war_c))
    early_read = [
        "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]",
        "s_nop 7",
        "v_accvgpr_read_b32 v1, a3",
    ]
    assert any("result read" in p for p in check(early_read))
    spaced = [
        "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]",
        "s_nop 7",
        "s_nop 7",
        "s_nop 3",
        "v_accvgpr_read_b32 v1, a3",
    ]
    assert check(spaced) == []
    chain = [
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[0:3], v[0:15]",
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], a[4:7], v[0:15]",
    ]
    assert check(chain) == []


@pytest.mark.parametrize("src", ["attn_bwd_kv2.hip"])
def test_kernel_m0_writes(src):
    """A kernel whose MFMAs are compiler builtins (the compiler spaces them)
    but whose grouped direct copies keep M0 between set_m0 statements:
    nothing else may write M0."""
    with tempfile.TemporaryDirectory() as d:
        asm = open(compile_to_asm(os.path.join(CSRC, src), os.path.join(d, "k.s"))).read()
    kernels = {k: v for k, v in functions(asm).items() if "kernel" in k}
    assert kernels, "no kernels in the listing"
    other = {k: m0_writers(v)[:3] for k, v in kernels.items() if m0_writers(v)}
    assert not other, other


@pytest.mark.parametrize("src", ["attn_bwd_kv.hip", "attn_bwd_dq_pipe.hip"])
def test_kernel_wait_states(src):
    with tempfile.TemporaryDirectory() as d:
        asm = open(compile_to_asm(os.path.join(CSRC, src), os.path.join(d, "k.s"))).read()
    kernels = {k: v for k, v in functions(asm).items() if "kernel" in k}
    assert kernels, "no kernels in the listing"
    found = {k: check(v) for k, v in kernels.items()}
    bad = {k: v[:3] for k, v in found.items() if v}
    assert not bad, bad
    # The grouped direct copies keep M0 between set_m0 statements: nothing
    # else may write it.
    other = {k: m0_writers(v)[:3] for k, v in kernels.items() if m0_writers(v)}
    assert not other, other
