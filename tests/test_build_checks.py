"""The build's gates (host logic, no GPU): register-spill remarks, the M0
discipline of the DMA asm, and the packed-fp32 pattern."""
from lm_head_reverse_amd import build as B

REMARKS = """\
x.hip:1:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs: 12 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark: Function Name: _Z3barPf [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs: 256 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]
x.hip:9:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]
"""


def test_spill_remarks_are_parsed_and_gated():
    res = B.kernel_resources(REMARKS)
    assert set(res) == {"_Z3fooPf", "_Z3barPf"}
    assert res["_Z3barPf"]["VGPRs Spill"] == "3"
    bad = B.check_spills(res)
    assert len(bad) == 1 and bad[0].startswith("_Z3barPf")


def test_m0_discipline():
    ok = ["s_mov_b32 m0, s12", "global_load_lds_dwordx4 v3, s[4:5]", "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"]
    assert B.m0_violations(ok) == []
    # M0 written for anything else, a DMA without its own write, a write not
    # followed by its DMA, or another implicit reader of M0
    assert B.m0_violations(["s_mov_b32 m0, -1", "ds_read_b32 v0, v1"])
    assert B.m0_violations(["s_add_i32 m0, s9, 0x2000", "global_load_lds_dwordx4 v[4:5], off"])
    assert B.m0_violations(["global_load_lds_dwordx4 v3, s[4:5]"])
    assert B.m0_violations(["s_mov_b32 m0, s12", "s_nop 0", "global_load_lds_dwordx4 v3, s[4:5]"])
    assert B.m0_violations(["s_sendmsg sendmsg(MSG_DEALLOC_VGPRS)"])


def test_packed_fp32_pattern():
    assert B.PACKED_FP32.search("v_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]")
    assert B.PACKED_FP32.search("v_pk_mul_f32 v[0:1], v[2:3], v[4:5]")
    assert not B.PACKED_FP32.search("v_pk_add_f16 v0, v1, v2")
    assert not B.PACKED_FP32.search("v_cvt_pk_f16_f32 v0, v1, v2")
