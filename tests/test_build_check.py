"""The build's packed-FP32 guard (no GPU): the device-assembly scan finds a
packed FP32 instruction when one is there, ignores comments and other
packed instructions, and the kept assembly of the last build has none."""
import os

import pytest

from moe_expert_routing_amd import build as B


def test_scan_finds_packed_fp32(tmp_path):
    (tmp_path / "x-hip-amdgcn-amd-amdhsa-gfx950.s").write_text(
        "\tv_pk_max_u16 v0, v1, v2\n"
        "\t; v_pk_add_f32 in a comment\n"
        "\tv_add_f32_e32 v0, v1, v2\n"
        "\tv_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]\n")
    (tmp_path / "x-host-x86_64-unknown-linux-gnu.s").write_text("\tv_pk_mul_f32\n")
    assert B.packed_fp32_in_device_asm(str(tmp_path)) == [("x-hip-amdgcn-amd-amdhsa-gfx950.s", 4)]


def test_last_build_has_no_packed_fp32():
    if not os.path.isdir(B.TEMPS):
        pytest.skip("no kept device assembly (library not built here)")
    assert B.packed_fp32_in_device_asm() == []
