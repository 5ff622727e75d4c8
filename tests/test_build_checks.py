"""CPU tests of the build-time checks: the kernel-resource-usage gate (no
scratch, no spills) and the static check that every inline-asm LDS read of
the attention kernels is waited for before its registers are touched. Each
check is run on small hand-written inputs, with and without a planted
mistake, and on the compiled library's own assembly and resource report when they are there."""

import os

import pytest

from shared_prefix_attention_amd import build as B
from shared_prefix_attention_amd import lds_wait_check as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _remarks(scratch="0", vspill="0", sspill="0", name="kern_a", occupancy="2", lds="67584"):
    return "\n".join([
        f"x.hpp:1:1: remark: Function Name: {name} [-Rpass-analysis=kernel-resource-usage]",
        "x.hpp:1:1: remark:     VGPRs: 100 [-Rpass-analysis=kernel-resource-usage]",
        f"x.hpp:1:1: remark:     Occupancy [waves/SIMD]: {occupancy} [-Rpass-analysis=kernel-resource-usage]",
        f"x.hpp:1:1: remark:     LDS Size [bytes/block]: {lds} [-Rpass-analysis=kernel-resource-usage]",
        f"x.hpp:1:1: remark:     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]",
        f"x.hpp:1:1: remark:     SGPRs Spill: {sspill} [-Rpass-analysis=kernel-resource-usage]",
        f"x.hpp:1:1: remark:     VGPRs Spill: {vspill} [-Rpass-analysis=kernel-resource-usage]",
        "x.hpp:1:1: remark:     Dynamic Stack: False [-Rpass-analysis=kernel-resource-usage]",
    ])


def test_resource_gate():
    assert B.check_resource_usage(_remarks())[0]["name"] == "kern_a"
    assert B.check_resource_usage(_remarks(sspill="9"))[0]["SGPRs Spill"] == "9"   # VGPR lanes, no memory
    with pytest.raises(RuntimeError):
        B.check_resource_usage(_remarks(scratch="16"))
    with pytest.raises(RuntimeError):
        B.check_resource_usage(_remarks(vspill="4"))
    with pytest.raises(RuntimeError):
        B.check_resource_usage("no remarks at all")


def test_attention_kernels_keep_two_work_groups_per_cu():
    """An attention kernel whose LDS leaves room for two work-groups per CU
    must fit two in registers too; other kernels, and attention kernels
    whose LDS holds one, are not held to it."""
    att = "_ZN2ca21cascade_phases_kernelILi128E"
    assert B.check_resource_usage(_remarks(name=att, occupancy="2"))
    with pytest.raises(RuntimeError):
        B.check_resource_usage(_remarks(name=att, occupancy="1"))
    assert B.check_resource_usage(_remarks(name=att, occupancy="1", lds="133120"))
    assert B.check_resource_usage(_remarks(name="kern_a", occupancy="1"))


def _asm(body):
    return "kern:\n" + "\n".join("\t" + x if not x.endswith(":") else x for x in body) + "\n"


def _read(dst, addr, off=0):
    return [";;#ASMSTART", f"ds_read_b64_tr_b16 {dst}, {addr} offset:{off}", ";;#ASMEND"]


WAIT = [";;#ASMSTART", "s_waitcnt lgkmcnt(0)", ";;#ASMEND"]


def test_waited_reads_pass():
    body = _read("v[8:9]", "v2") + _read("v[10:11]", "v2", 4096) + ["v_add_u32_e32 v3, v4, v5"] + WAIT + \
        ["v_mfma_f32_16x16x32_bf16 v[20:23], v[8:11], v[12:15], 0", "s_endpgm"]
    k, n, problems = L.check(_asm(body))
    assert (k, n, problems) == (1, 2, [])


def test_use_before_wait_is_caught():
    body = _read("v[8:9]", "v2") + ["v_mov_b32_e32 v100, v9"] + WAIT + ["s_endpgm"]
    assert len(L.check(_asm(body))[2]) == 1


def test_register_reuse_before_wait_is_caught():
    body = _read("v[8:9]", "v2") + ["v_mov_b32_e32 v8, 0"] + WAIT + ["s_endpgm"]
    assert len(L.check(_asm(body))[2]) == 1


def test_address_in_flight_is_caught():
    body = _read("v[8:9]", "v2") + _read("v[10:11]", "v8") + WAIT + ["s_endpgm"]
    assert len(L.check(_asm(body))[2]) == 1


def test_partial_wait_does_not_count():
    body = _read("v[8:9]", "v2") + ["s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v100, v8", "s_endpgm"]
    assert len(L.check(_asm(body))[2]) == 1


def test_use_along_a_branch_is_caught():
    # the read is in flight on the taken edge; the target uses it first
    body = _read("v[8:9]", "v2") + ["s_cbranch_vccnz .LBB0_2"] + WAIT + ["s_endpgm", ".LBB0_2:",
                                                                         "v_mov_b32_e32 v100, v8", "s_endpgm"]
    problems = L.check(_asm(body))[2]
    assert len(problems) == 1 and "v_mov" in problems[0]


def test_loop_carried_read_is_tracked():
    # a read issued at the end of an iteration and used at the top of the next
    body = [".LBB0_1:", "v_mov_b32_e32 v100, v8"] + _read("v[8:9]", "v2") + ["s_cbranch_scc1 .LBB0_1", "s_endpgm"]
    problems = L.check(_asm(body))[2]
    assert any("v_mov" in p for p in problems)


def test_compiler_reads_are_not_tracked():
    body = ["ds_read_b128 v[8:11], v2", "s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v100, v8", "s_endpgm"]
    assert L.check(_asm(body))[1:] == (0, [])


def test_this_build_passes():
    path = os.path.join(ROOT, "shared_prefix_attention_amd", "_build", "run.hip.s")
    if not os.path.exists(path):
        pytest.skip("no device assembly from a build in this checkout")
    kernels, reads, problems = L.check(open(path).read())
    assert kernels >= 10 and reads > 1000 and problems == []
