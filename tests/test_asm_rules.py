"""The inline-assembly MFMAs of gemm_m16_kernel against the rules its source
states (no accumulator access next to an MFMA the compiler cannot see, no
VALU-written MFMA operand without wait states), and its grouped LDS-DMA
loads against theirs (M0 written only by inline assembly), checked on the assembly of
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


SETLOAD = (";;#ASMSTART\ns_mov_b32 m0, s4\ns_nop 0\nbuffer_load_dwordx4 v1, s[8:11], s5 offen offset:0 lds\n"
           ";;#ASMEND")
LOAD = ";;#ASMSTART\nbuffer_load_dwordx4 v2, s[8:11], s5 offen offset:0x400 lds\n;;#ASMEND"


def _check_m0(body: str):
    (_, lines), = list(asm_rules.functions(_listing(body)))
    return asm_rules.check_m0(lines)


def test_m0_checker_accepts_a_shared_write():
    n, bad = _check_m0(f"""
        {SETLOAD}
        v_add_u32_e32 v3, v4, v5
        {LOAD}
        {LOAD}
    """)
    assert n == 3 and bad == []


def test_m0_checker_rejects_a_compiler_write():
    n, bad = _check_m0(f"""
        {SETLOAD}
        s_mov_b32 m0, s6
        {LOAD}
    """)
    assert [v[0] for v in bad] == ["M0 written outside inline assembly",
                                   "LDS-DMA load without an inline-assembly M0 write before it"]


def test_m0_checker_rejects_a_load_with_no_write_before_it():
    n, bad = _check_m0(f"""
        {LOAD}
        {SETLOAD}
    """)
    assert len(bad) == 1 and "without an inline-assembly M0 write" in bad[0][0]
    # the flat form of the DMA load too
    n, bad = _check_m0("""
        ;;#ASMSTART
        global_load_lds_dwordx4 v[2:3], off offset:1024
        ;;#ASMEND
    """)
    assert n == 1 and len(bad) == 1


def test_m0_checker_follows_every_path():
    # one path reaches the load through the inline-assembly write, the other
    # does not write M0 at all
    n, bad = _check_m0(f"""
        s_cbranch_scc1 .LBB0_2
        {SETLOAD}
        .LBB0_2:
        {LOAD}
    """)
    assert len(bad) == 1
    n, bad = _check_m0(f"""
        {SETLOAD}
        .LBB0_1:
        {LOAD}
        s_cbranch_scc1 .LBB0_1
    """)
    assert bad == []


def _device_asm(source):
    try:
        hipcc = _build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(_build.CSRC, source)
    with tempfile.TemporaryDirectory(prefix="agmm_asm_") as tmp:
        out = os.path.join(tmp, os.path.splitext(source)[0] + ".s")
        cmd = [hipcc, *_build.COMMON, *_build.SOURCES[source], "--cuda-device-only", "-S",
               "-o", out, src]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        with open(out) as f:
            return f.read()


@pytest.fixture(scope="module")
def gemm_asm():
    return _device_asm("gemm_mfma.hip")



def test_mfma16_kernels_keep_the_inline_asm_rules(gemm_asm):
    checked = 0
    for sym, lines in asm_rules.functions(gemm_asm):
        if "gemm_m16_kernel" not in sym:
            continue
        n_asm, bad = asm_rules.check_function(lines)
        assert bad == [], f"{sym}: {bad[:5]}"
        checked += n_asm
    assert checked > 0, "no inline-asm MFMA found: the check would be vacuous"


def test_gemm_kernels_write_m0_only_in_inline_asm(gemm_asm):
    """The grouped buffer loads of gemm_m16_kernel rely on the compiler never
    writing M0: checked on every GEMM kernel of the library's build."""
    checked = 0
    for sym, lines in asm_rules.functions(gemm_asm):
        if "gemm" not in sym:
            continue
        n, bad = asm_rules.check_m0(lines)
        assert bad == [], f"{sym}: {bad[:5]}"
        checked += n
    assert checked > 0, "no LDS-DMA load found: the check would be vacuous"

