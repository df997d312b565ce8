"""Host-only checks of the C ABI (no GPU): the library loads, exports every
symbol include/agmm.h declares, and rejects malformed problems with the
documented status codes and messages."""
import ctypes
import os
import re

import pytest

import all_gather_gemm_agmm_amd as agmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "agmm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(agmm_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = agmm.load_library()
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), f"{name} declared in agmm.h but not exported"
    # ...and the Python binding covers exactly the declared set
    assert sorted(n for n, _, _ in agmm.EXPORTS) == names


def test_version():
    assert "gfx950" in agmm.agmm_version()


def test_validate_accepts_the_workloads():
    from all_gather_gemm_agmm_amd import inputs as I
    for w in I.WORKLOADS.values():
        assert agmm.agmm_plan_validate(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype,
                                       w.rhs_transpose) == agmm.AGMM_OK


@pytest.mark.parametrize("args,status,fragment", [
    ((0, 4, 8, 8, 0, 0), agmm.AGMM_ERR_INVALID_ARG, "num_shards"),
    ((65, 4, 8, 8, 0, 0), agmm.AGMM_ERR_UNSUPPORTED, "maximum"),
    ((2, 0, 8, 8, 0, 0), agmm.AGMM_ERR_INVALID_ARG, "sizes"),
    ((2, 4, 0, 8, 0, 0), agmm.AGMM_ERR_INVALID_ARG, "sizes"),
    ((2, 4, 8, -1, 0, 0), agmm.AGMM_ERR_INVALID_ARG, "sizes"),
    ((2, 4, 8, 8, 7, 0), agmm.AGMM_ERR_INVALID_ARG, "dtype"),
    ((2, 4, 8, 8, 0, 2), agmm.AGMM_ERR_INVALID_ARG, "rhs_transpose"),
    ((2, 1 << 29, 8, 8, 0, 0), agmm.AGMM_ERR_UNSUPPORTED, "too large"),
])
def test_validate_rejects(args, status, fragment):
    assert agmm.load_library().agmm_plan_validate(*args) == status
    assert agmm.agmm_last_status() == status
    assert fragment in agmm.agmm_last_error()


@pytest.mark.parametrize("args,ok", [
    ((64, 1, 8, 8), True),                        # the most shards
    ((1, (1 << 30) - 1, 1, 1), True),             # m just below 2^30
    ((2, 1 << 29, 1, 1), False),                  # m = 2^30
    ((1, 1, (1 << 30) - 1, 1), True),             # k just below 2^30
    ((1, 1, 1, 1 << 30), False),                  # n = 2^30
    ((1, 1 << 20, (1 << 20) - 1, 8), True),       # m*k just below 2^40
    ((1, 1 << 20, 1 << 20, 8), False),            # m*k = 2^40
    ((4, 1 << 18, 8, 1 << 20), False),            # m*n = 2^40
    ((1, 8, 1 << 20, (1 << 20) - 1), True),       # k*n just below 2^40
])
def test_validate_size_limits(args, ok):
    """m, k and n_local below 2^30 and their products below 2^40, exactly at
    the boundaries."""
    st = agmm.load_library().agmm_plan_validate(*args, 0, 0)
    if ok:
        assert st == agmm.AGMM_OK, agmm.agmm_last_error()
    else:
        assert st == agmm.AGMM_ERR_UNSUPPORTED and "too large" in agmm.agmm_last_error()


def test_validate_accepts_ragged_and_odd_shapes():
    assert agmm.agmm_plan_validate(3, 100, 200, 136, 0, 0) == agmm.AGMM_OK
    assert agmm.agmm_plan_validate(3, 100, 200, 130, 1, 1) == agmm.AGMM_OK  # n free with B^T
    assert agmm.agmm_plan_validate(2, 5, 7, 3, 2, 0) == agmm.AGMM_OK        # fp32: any shape
    # 16-bit rows that are not whole 16-byte vectors run on zero-padded copies
    assert agmm.agmm_plan_validate(2, 4, 12, 8, 0, 1) == agmm.AGMM_OK
    assert agmm.agmm_plan_validate(2, 4, 16, 12, 1, 0) == agmm.AGMM_OK
    assert agmm.agmm_plan_validate(3, 7, 13, 5, 1, 0) == agmm.AGMM_OK
    assert agmm.agmm_last_status() == agmm.AGMM_OK and agmm.agmm_last_error() == ""


def test_null_handles_are_rejected_without_touching_the_gpu():
    lib = agmm.load_library()
    assert lib.agmm_run(None, None, None, None, None) == agmm.AGMM_ERR_INVALID_ARG
    assert "plan is NULL" in agmm.agmm_last_error()
    assert lib.agmm_gather(None, None, None, None) == agmm.AGMM_ERR_INVALID_ARG
    assert lib.agmm_run_gathered(None, None, None, None, None) == agmm.AGMM_ERR_INVALID_ARG
    assert lib.agmm_plan_set_int(None, b"pvalue", 2) == agmm.AGMM_ERR_INVALID_ARG
    v = ctypes.c_int64(0)
    assert lib.agmm_plan_get_int(None, b"pvalue", ctypes.byref(v)) == agmm.AGMM_ERR_INVALID_ARG
    assert lib.agmm_plan_workspace_bytes(None) == 0
    assert not lib.agmm_plan_slot_ptr(None, 0)
    assert lib.agmm_plan_tile_order(None, 0, None, 0) == -1
    assert lib.agmm_plan_timing_begin(None) == agmm.AGMM_ERR_INVALID_ARG
    lib.agmm_plan_destroy(None)  # no-op


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        agmm.load_library(str(tmp_path / "libagmm.so"))


def _header_rule_statuses(N, m_s, k, n, dtype, rt):
    """Statuses the header's agmm_plan_validate rules give a problem (an empty
    set: accepted)."""
    out = set()
    if N < 1 or min(m_s, k, n) < 1 or dtype not in (0, 1, 2) or rt not in (0, 1):
        out.add(agmm.AGMM_ERR_INVALID_ARG)
    if N > 64:
        out.add(agmm.AGMM_ERR_UNSUPPORTED)
    if not out:
        m = N * m_s
        if max(m, k, n) >= 1 << 30 or max(m * k, k * n, m * n) >= 1 << 40:
            out.add(agmm.AGMM_ERR_UNSUPPORTED)
    return out


def test_validate_follows_the_header_rules():
    """agmm_plan_validate against the header's rules, restated here, on drawn
    problems: sizes around 1, around the 2^30 and 2^40 limits and anywhere in
    between, in- and out-of-range dtypes, layout flags and shard counts."""
    hyp = pytest.importorskip("hypothesis")
    st = hyp.strategies
    size = st.one_of(st.integers(-2, 3), st.integers(1, 1 << 12),
                     st.integers((1 << 20) - 2, (1 << 20) + 2), st.integers((1 << 30) - 2, (1 << 30) + 1),
                     st.integers(1, (1 << 31) - 1))
    lib = agmm.load_library()

    @hyp.settings(max_examples=3000, deadline=None, derandomize=True)
    @hyp.given(N=st.integers(-1, 70), m_s=size, k=size, n=size, dtype=st.integers(-1, 3),
               rt=st.integers(-1, 2))
    def check(N, m_s, k, n, dtype, rt):
        want = _header_rule_statuses(N, m_s, k, n, dtype, rt)
        got = lib.agmm_plan_validate(N, m_s, k, n, dtype, rt)
        if want:
            assert got in want, (N, m_s, k, n, dtype, rt, got, agmm.agmm_last_error())
            assert agmm.agmm_last_status() == got and agmm.agmm_last_error() != ""
        else:
            assert got == agmm.AGMM_OK, (N, m_s, k, n, dtype, rt, agmm.agmm_last_error())
            assert agmm.agmm_last_error() == ""

    check()


def test_status_is_per_thread():
    """The header's status rule on the CPU: each host thread reads the
    status and message of its own most recent call, whatever other threads
    do meanwhile (8 threads alternating accepted and rejected problems)."""
    import threading
    lib = agmm.load_library()
    errors = []
    start = threading.Barrier(8)

    def worker(i):
        try:
            start.wait()
            for it in range(2000):
                bad = (i + it) % 2 == 0
                st = lib.agmm_plan_validate(2, 4, 8, 8, 7 if bad else 0, 0)
                want = agmm.AGMM_ERR_INVALID_ARG if bad else agmm.AGMM_OK
                got_st, got_msg = lib.agmm_last_status(), lib.agmm_last_error().decode()
                if st != want or got_st != want or (bad != ("unknown dtype 7" in got_msg)) or (not bad and got_msg):
                    errors.append((i, it, st, got_st, got_msg))
                    return
        except Exception as e:   # pragma: no cover - reported below
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert errors == []
