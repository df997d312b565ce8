"""The no-allocation entry point (agmm_run_noalloc) through the C ABI.

Its output is checked against agmm_run on a default plan for the same
problem (bit-identical: same tile, same k split, only the tile visit order
differs, which does not change values) and against the oracle's tolerance,
on two calls in a row, the second smaller, both using split-K partial sums in
the library's scratch.  A problem whose partial sums do not fit the scratch
is refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import oracle
import all_gather_gemm_agmm_amd as agmm
from all_gather_gemm_agmm_amd import inputs as I
from gpu_util import BOUND, rel_err, to_bits, to_device, torch_dtype

pytestmark = pytest.mark.gpu

BF16, FP16 = I.DTYPE_BF16, I.DTYPE_FP16

# N, m_per_shard, k, n_local, dtype, rhs_transpose; the second call is smaller
CASES = [
    (4, 48, 4096, 1024, BF16, True),   # m 192: the split-K 128x64 skinny tile, 8 k ranges
    (2, 64, 2048, 256, FP16, False),   # m 128, B k x n: the 128x128 tile, 16 k ranges
    (4, 16, 8192, 1024, BF16, True),   # m 64: the skinny 32x32 tile, 4 k ranges
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    agmm.load_library()


def test_noalloc_matches_agmm_run_twice_in_a_row():
    for i, (N, m_s, k, n, dtype, rt) in enumerate(CASES):
        w = I.custom_workload(N, m_s, k, n, dtype, rt, wid=3100 + i)
        shards, B = I.make_inputs(w)
        sd = [to_device(x, dtype) for x in shards]
        bd = to_device(B, dtype)
        plan = agmm.Plan(N, m_s, k, n, dtype, rt)
        try:
            splits = plan.get("splits")
            assert splits > 1, "the case must use split-K partial sums (the scratch)"
            assert splits * w.m * n * 4 <= agmm.NOALLOC_SCRATCH_BYTES
            C_ref = plan.run(sd, bd)
            torch.cuda.synchronize()
        finally:
            plan.close()
        C = torch.full((w.m, n), float("nan"), dtype=torch_dtype(dtype), device="cuda")
        agmm.agmm_run_noalloc(N, m_s, k, n, dtype, rt, [x.data_ptr() for x in sd], bd.data_ptr(),
                              C.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        got_bits = to_bits(C)
        assert np.array_equal(got_bits, to_bits(C_ref)), f"call {i}: differs from agmm_run"
        ref = oracle.agmm_f64(shards, B, dtype, rt)
        err = rel_err(oracle.decode(got_bits, dtype), ref)
        assert err <= BOUND[dtype], f"call {i}: max rel err {err:.3e}"


def test_noalloc_refuses_problems_beyond_its_scratch():
    """4 x 512 x 8192 -> 4096 bf16: a default plan splits k in two, 64 MiB of
    partial sums, more than the scratch holds; the call fails and C is
    untouched."""
    N, m_s, k, n = 4, 512, 8192, 4096
    plan = agmm.Plan(N, m_s, k, n, BF16, False)
    try:
        need = plan.get("splits") * N * m_s * n * 4
    finally:
        plan.close()
    assert need > agmm.NOALLOC_SCRATCH_BYTES
    sd = [torch.zeros((m_s, k), dtype=torch.bfloat16, device="cuda") for _ in range(N)]
    bd = torch.zeros((k, n), dtype=torch.bfloat16, device="cuda")
    C = torch.full((N * m_s, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(agmm.AgmmError) as ei:
        agmm.run_noalloc(sd, bd, C, False)
    assert ei.value.status == agmm.AGMM_ERR_UNSUPPORTED
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.isnan(C.float()).all().item()


def test_noalloc_refuses_padded_shapes():
    """Rows that are not whole 16-byte vectors need a plan's padded copies."""
    sd = [torch.zeros((8, 13), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    bd = torch.zeros((24, 13), dtype=torch.bfloat16, device="cuda")
    C = torch.full((16, 24), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(agmm.AgmmError) as ei:
        agmm.run_noalloc(sd, bd, C, True)
    assert ei.value.status == agmm.AGMM_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(C.float()).all().item()
