"""The inline-assembly MFMAs of gemm_m16_kernel against the rules its source
states (no accumulator access next to an MFMA the compiler cannot see, no
VALU-written MFMA operand without wait states), checked on the assembly of
gemm_mfma.hip compiled with the library's own flags.  Runs on the CPU
(hipcc cross-compiles for gfx950); the checker itself is first tested on
small hand-written listings."""
import os
import subprocess
import tempfile

import pytest

import asm_rules
from all_gather_gemm_agmm_amd import _build

HEADER = "_Z4testv:\n"
FOOTER = "\ts_endpgm\n.Lfunc_end0:\n"


def _listing(body: str) -> str:
    out = []
    for line in body.strip().split("\n"):
        t = line.strip()
        out.append((t if t.startswith((".", ";;")) else "\t" + t) + "\n")
    return HEADER + "".join(out) + FOOTER


def _check(body: str):
    (_, lines), = list(asm_rules.functions(_listing(body)))
    return asm_rules.check_function(lines)


MFMA = ";;#ASMSTART\nv_mfma_f32_16x16x32_bf16 a[0:3], v[4:7], v[8:11], a[0:3]\n;;#ASMEND"
DRAIN = ";;#ASMSTART\ns_nop 7\ns_nop 7\ns_nop 7\ns_nop 7\n;;#ASMEND"


def test_checker_accepts_drained_code():
    n, bad = _check(f"""
        ds_read_b128 v[4:7], v1
        ds_read_b128 v[8:11], v2
        s_waitcnt lgkmcnt(0)
        {MFMA}
        {MFMA}
        {DRAIN}
        v_accvgpr_read_b32 v20, a0
    """)
    assert n == 2 and bad == []


def test_checker_flags_accumulator_read_before_drain():
    n, bad = _check(f"""
        {MFMA}
        v_accvgpr_read_b32 v20, a0
        {DRAIN}
    """)
    assert n == 1 and len(bad) == 1 and "after an MFMA" in bad[0][0]


def test_checker_flags_accumulator_write_before_mfma():
    _, bad = _check(f"""
        v_accvgpr_write_b32 a1, 0
        {MFMA}
        {DRAIN}
    """)
    assert len(bad) == 1 and "AGPR write" in bad[0][0]


def test_checker_flags_valu_written_operand():
    _, bad = _check(f"""
        {DRAIN}
        v_mov_b32 v9, v30
        {MFMA}
        {DRAIN}
    """)
    assert len(bad) == 1 and "VALU write" in bad[0][0]


def test_checker_follows_branches():
    # the drain sits on one path only: the read after the join is flagged
    _, bad = _check(f"""
        {MFMA}
        s_cbranch_scc1 .LBB0_2
        {DRAIN}
    .LBB0_2:
        v_accvgpr_read_b32 v20, a0
    """)
    assert len(bad) == 1
    # a loop whose back edge carries an undrained MFMA into an AGPR write
    _, bad = _check(f"""
        {DRAIN}
    .LBB0_1:
        v_accvgpr_write_b32 a5, v3
        {DRAIN}
        {MFMA}
        s_cbranch_scc1 .LBB0_1
        {DRAIN}
    """)
    assert len(bad) == 1 and "after an MFMA" in bad[0][0]


@pytest.fixture(scope="module")
def gemm_asm():
    try:
        hipcc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(_build.CSRC, "gemm_mfma.hip")
    with tempfile.TemporaryDirectory(prefix="agmm_asm_") as tmp:
        out = os.path.join(tmp, "gemm_mfma.s")
        cmd = [hipcc, *_build.COMMON, *_build.SOURCES["gemm_mfma.hip"], "--cuda-device-only", "-S",
               "-o", out, src]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            yield f.read()


def test_mfma16_kernels_keep_the_inline_asm_rules(gemm_asm):
    checked = 0
    for sym, lines in asm_rules.functions(gemm_asm):
        if "gemm_m16_kernel" not in sym:
            continue
        n_asm, bad = asm_rules.check_function(lines)
        assert bad == [], f"{sym}: {bad[:5]}"
        checked += n_asm
    assert checked > 0, "no inline-asm MFMA found: the check would be vacuous"
