"""The build's static wait-state checks (exact_attention_12_amd/hazards.py) on
small hand-written gfx950 listings: a VALU write one or two instructions
before an MFMA operand read, and a VALU access to an AGPR accumulator too
soon after the product that writes it, must be flagged; the same code with
enough wait states in between must pass."""

import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hazards():
    spec = importlib.util.spec_from_file_location(
        "hazards", os.path.join(ROOT, "exact_attention_12_amd", "hazards.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _func(body: str) -> str:
    return "_Z1kv:\n" + body + "\n.Lfunc_end0:\n"


MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[4:7], v[8:11], a[0:15]"


@pytest.mark.parametrize("body,n", [
    # B operand written by the instruction right before
    ("v_cvt_pk_bf16_f32 v9, v1, v2\n" + MFMA, 1),
    # one instruction in between is only one wait state
    ("v_cvt_pk_bf16_f32 v9, v1, v2\ns_waitcnt lgkmcnt(0)\n" + MFMA, 1),
    # A operand
    ("v_mov_b32 v5, v1\n" + MFMA, 1),
    # accumulator written by v_accvgpr_write
    ("v_accvgpr_write_b32 a3, v1\n" + MFMA, 1),
    # a label inside the window: another path may reach the MFMA
    ("v_mov_b32 v40, v1\n.LBB0_1:\n" + MFMA, 1),
    # two wait states: a nop of 1, or two other instructions
    ("v_cvt_pk_bf16_f32 v9, v1, v2\ns_nop 1\n" + MFMA, 0),
    ("v_cvt_pk_bf16_f32 v9, v1, v2\ns_waitcnt lgkmcnt(0)\ns_nop 0\n" + MFMA, 0),
    # writes of registers the MFMA does not read
    ("v_cvt_pk_bf16_f32 v12, v1, v2\n" + MFMA, 0),
    ("v_accvgpr_write_b32 a16, v1\n" + MFMA, 0),
    # a VGPR pair range overlapping the operand
    ("v_lshlrev_b64 v[10:11], 1, v[2:3]\n" + MFMA, 1),
    # an AGPR accumulator copied while the product is still being written
    (MFMA + "\ns_nop 7\nv_accvgpr_mov_b32 a40, a15", 1),
    (MFMA + "\nv_accvgpr_read_b32 v1, a3", 1),
    (MFMA + "\ns_nop 7\ns_nop 7\ns_nop 1\nv_accvgpr_mov_b32 a40, a15", 0),
    # other registers, or past an unconditional branch
    (MFMA + "\nv_accvgpr_mov_b32 a40, a16", 0),
    (MFMA + "\ns_branch .LBB0_2\nv_accvgpr_read_b32 v1, a3", 0),
    # compiler-managed products (VGPR results) are not the check's business
    ("v_mfma_f32_32x32x16_bf16 v[16:31], v[4:7], v[8:11], v[16:31]\nv_mov_b32 v40, v16", 0),
])
def test_hazard_rule(body, n):
    assert len(_hazards().check(_func(body))) == n


def test_built_bwd_assembly_is_clean():
    """The assembly the last build checked (if a build has run here)."""
    path = os.path.join(ROOT, "exact_attention_12_amd", "_build", "attn_bwd.hip.gfx950.s")
    if not os.path.exists(path):
        pytest.skip("no build output here")
    with open(path) as f:
        assert _hazards().check(f.read()) == []
