"""The built library's device code: no MFMA result is read through a branch with fewer
wait states than the compiler leaves for the same read within one basic block
(kv_cache_flashattention_attn_amd/hazard_scan.py explains the check and the defect it
guards against)."""
import os

import pytest

from kv_cache_flashattention_attn_amd import build, hazard_scan


def _asm():
    if not os.path.exists(build.ASM_PATH):
        pytest.skip("device assembly not built (python -m kv_cache_flashattention_attn_amd.build)")
    return open(build.ASM_PATH).read()


def test_no_mfma_result_read_early_across_a_branch():
    need, bad = hazard_scan.scan(_asm())
    assert need, "no MFMA result reads found: the scan is not seeing the kernels"
    assert not bad, "\n".join(f"{k[:80]}: {op}, {w} wait states to {t}" for k, op, w, _, t in bad[:10])


def test_scan_catches_a_read_one_instruction_after_the_mfma():
    """Teeth: the pattern of the defect (a branch, then the read) is reported."""
    text = "\n".join([
        "_Zkernel:",
        "\tv_mfma_f32_16x16x32_f16 v[4:7], v[8:11], v[12:15], 0",
        "\ts_nop 7",
        "\tv_max_f32_e32 v1, v7, v7",
        "\tv_mfma_f32_16x16x32_f16 v[4:7], v[8:11], v[12:15], 0",
        "\ts_cbranch_scc1 .LBB0_2",
        "\ts_nop 7",
        "\tv_max_f32_e32 v1, v7, v7",
        ".LBB0_2:",
        "\tv_max_f32_e32 v2, v7, v7",
        "\ts_endpgm",
        ".Lfunc_end0:",
    ])
    need, bad = hazard_scan.scan(text)
    assert need == {"v_mfma_f32_16x16x32_f16": 8}
    assert len(bad) == 1 and bad[0][2] == 1 and "v2" in bad[0][4]


def test_scan_ends_a_path_where_the_result_registers_are_overwritten():
    """A read after a load (or another write) into every result register reads that
    value, not the MFMA's: not reported.  A read of a register still holding the
    result is."""
    text = "\n".join([
        "_Zkernel:",
        "\tv_mfma_f32_16x16x32_f16 v[4:7], v[8:11], v[12:15], 0",
        "\ts_nop 7",
        "\tv_max_f32_e32 v1, v7, v7",
        "\tv_mfma_f32_16x16x32_f16 v[4:7], v[8:11], v[12:15], 0",
        "\ts_cbranch_scc1 .LBB0_2",
        "\tglobal_load_dwordx4 v[4:7], v[20:21], off",
        "\ts_waitcnt vmcnt(0)",
        "\tv_mov_b64_e32 v[30:31], v[4:5]",
        ".LBB0_2:",
        "\tv_mov_b32_e32 v6, 0",
        "\tv_max_f32_e32 v2, v6, v6",
        "\tv_max_f32_e32 v3, v7, v7",
        "\ts_endpgm",
        ".Lfunc_end0:",
    ])
    need, bad = hazard_scan.scan(text)
    assert need == {"v_mfma_f32_16x16x32_f16": 8}
    # only the read of v7 on the path that skipped the load: v6 was rewritten first
    assert len(bad) == 1 and "v3" in bad[0][4], bad
