"""The library's gfx950 assembly holds no scalar select fed by a stale carry
flag (see isa_audit.py), and the check finds one in a hand-made listing."""
import os
import shutil
import subprocess

import pytest

from isa_audit import stale_scc_selects

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "sparse_gradient_synchronization_amd", "csrc")


def test_audit_finds_a_select_after_a_carry():
    asm = "\n".join([
        "_Zk:", "\ts_add_u32 s0, s2, s0", "\ts_addc_u32 s1, s3, s1", "\tv_cmp_lt_u64_e32 vcc, s[4:5], v[4:5]",
        "\ts_cbranch_vccnz .LBB0_2", "; %bb.1:", "\ts_endpgm", ".LBB0_2:", "\ts_cselect_b32 s8, s4, 0x2000",
        "\ts_endpgm"])
    found = stale_scc_selects(asm)
    assert len(found) == 1 and found[0][2].startswith("s_cselect_b32")
    # the same select after a comparison is fine
    ok = asm.replace("\tv_cmp_lt_u64_e32 vcc, s[4:5], v[4:5]", "\ts_cmp_lt_u32 s4, 0x2000")
    assert stale_scc_selects(ok) == []


@pytest.mark.skipif(not shutil.which("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_library_assembly_has_no_stale_scc_select(tmp_path):
    out = tmp_path / "sg_lib.s"
    cmd = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", "-o", str(out), "sg_lib.hip"]
    r = subprocess.run(cmd, cwd=CSRC, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    found = stale_scc_selects(out.read_text())
    assert found == [], found[:5]
