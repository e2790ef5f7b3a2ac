"""The inline-asm MFMA / v_dot2c wait states of the 64-query-wave and persistent kernels, checked
on the code the compiler generates for gfx950 (no GPU needed), and the checker itself on planted
cases."""
import os
import shutil
import subprocess

import pytest

from tests.isa_hazards import check_asm, compiler_source_war_pairs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_checker_finds_planted_hazards():
    asm = "\n".join([
        "_Zplanted:",
        "\tv_cvt_pk_bf16_f32 v10, v1, v2",
        "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[20:23], v[8:11], a[0:15]",
        "\tv_accvgpr_read_b32 v5, a3",
        "\tv_dot2c_f32_bf16 v30, 0x3f803f80, v9",
        "\tv_add_f32_e32 v31, v30, v30",
        "\ts_nop 1",
        "\tv_mfma_f32_32x32x16_bf16 a[16:31], v[20:23], v[8:11], a[16:31]",
        "\ts_nop 7",
        "\ts_nop 7",
        "\tv_accvgpr_read_b32 v6, a17",
        "\tv_dot2c_f32_bf16 v40, 0x3f803f80, v9",
        "\tv_dot2c_f32_bf16 v40, 0x3f803f80, v10",
        "\ts_nop 2",
        "\tv_add_f32_e32 v41, v40, v40",
    ])
    bad = check_asm(asm)["_Zplanted"]
    assert len(bad) == 3, bad   # cvt -> mfma, mfma -> accvgpr read, dot2c -> add


def test_checker_separates_source_war_by_operand():
    """A VALU write right after an MFMA: harmless to SrcA/SrcB, a hazard to a VGPR SrcC that is
    not also the destination, and a result read (not this rule) when SrcC is the destination."""
    asm = "\n".join([
        "_Zwar:",
        "\tv_mfma_f32_32x32x16_bf16 v[40:55], v[20:23], v[8:11], v[40:55]",
        "\tv_mov_b32_e32 v20, 0",                                  # SrcA: fine
        "\tv_mov_b32_e32 v9, 0",                                   # SrcB: fine
        "\ts_nop 7",
        "\ts_nop 7",
        "\tv_mfma_f32_32x32x16_bf16 v[60:75], v[20:23], v[8:11], v[80:95]",
        "\tv_mov_b32_e32 v81, 0",                                  # SrcC, not the destination
        "\ts_nop 7",
        "\ts_nop 7",
        "\tv_mov_b32_e32 v82, 0",                                  # 17 wait states later: fine
    ])
    bad = check_asm(asm)["_Zwar"]
    assert len(bad) == 1 and "v81" in bad[0], bad


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
@pytest.mark.parametrize("src_name, kernel", [("sdpa_bf16_d128_w64.hip", "attn_fwd_w_kernel"),
                                              ("sdpa_bf16_d128_p.hip", "attn_fwd_p_kernel"),
                                              ("sdpa_f16_d64.hip", "attn_fwd_kernel")])
def test_generated_code_has_no_inline_asm_hazards(tmp_path, src_name, kernel):
    from exact_attention_forward_flash_amd.build import HIPCC, flags_for, CSRC
    src = os.path.join(CSRC, src_name)
    out = tmp_path / "k.s"
    cmd = [HIPCC, *flags_for(src), "--cuda-device-only", "-S", src, "-o", str(out)]
    subprocess.run([c for c in cmd if c != "-fPIC"], check=True, capture_output=True)
    text = out.read_text()
    res = check_asm(text)
    kernels = [k for k in res if kernel in k]
    assert kernels, f"no {kernel} in the listing"
    for k in kernels:
        assert not res[k], (k, res[k][:5])
    # the compiler's own schedule writes MFMA A/B registers in the very next instruction, which
    # the inline asm relies on as well (no wait states for write-after-read of SrcA/SrcB)
    assert compiler_source_war_pairs(text.splitlines()) > 0
