"""The column substitutions issue `v_fmac_f32_dpp` from inline asm, where
the compiler inserts no wait states.  Compile the kernels that use it to
gfx950 assembly (with the library's flags) and check that no DPP source
register was written by a VALU instruction within the two preceding wait
states.  Also check the checker on planted cases."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

import dpp_hazard
from delta_rule_linear_amd import build as kbuild

SOURCES = ["kla_prefill.hip", "kla_kda.hip", "kla_bwd.hip"]


def test_checker_finds_planted_hazards():
    dpp = " v_fmac_f32_dpp v3, v2, v1 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
    assert dpp_hazard.check("f:\n v_mul_f32_e32 v2, v1, v2\n" + dpp)
    assert dpp_hazard.check("f:\n v_mul_f32_e32 v2, v1, v2\n s_waitcnt vmcnt(0)\n" + dpp)
    assert dpp_hazard.check("f:\n v_permlane32_swap_b32_e32 v5, v2\n" + dpp)  # both operands written
    assert dpp_hazard.check("f:\n v_mov_b64 v[2:3], v[6:7]\n" + dpp)
    assert not dpp_hazard.check("f:\n v_mul_f32_e32 v2, v1, v2\n s_nop 1\n" + dpp)
    assert not dpp_hazard.check("f:\n v_mul_f32_e32 v2, v1, v2\n v_add_f32 v8, v1, v1\n v_add_f32 v9, v1, v1\n" + dpp)
    assert not dpp_hazard.check("f:\n v_mul_f32_e32 v4, v1, v2\n" + dpp)


@pytest.mark.skipif(not shutil.which(kbuild.HIPCC) and not os.path.exists(kbuild.HIPCC), reason="hipcc not found")
def test_no_dpp_read_after_valu_write(tmp_path):
    def asm(src):
        out = tmp_path / (src + ".s")
        cmd = [kbuild.HIPCC] + kbuild.flags(src) + ["-x", "hip", "--cuda-device-only", "-S",
                                                os.path.join(kbuild.CSRC, src), "-o", str(out)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return src, out.read_text()

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        results = list(ex.map(asm, SOURCES))
    for src, text in results:
        n_dpp = text.count("v_fmac_f32_dpp")
        assert n_dpp > 0, f"{src}: no DPP substitution found (the check would be vacuous)"
        bad = dpp_hazard.check(text)
        assert not bad, f"{src}: DPP read within two wait states of a VALU write: {bad[:3]}"
