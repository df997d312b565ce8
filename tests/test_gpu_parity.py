"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerance (stated for the all-gather matmul workloads): per element
|C_gpu - C_ref| / (|C_ref| + 1e-3) <= 2e-2 for bf16/fp16 inputs and <= 1e-5
for fp32 inputs, C_ref being the oracle's float64 result.  Gathered operands
and schedule-invariance checks are bit-exact.
"""
import time

import numpy as np
import pytest
import torch

import oracle
import all_gather_gemm_agmm_amd as agmm
from all_gather_gemm_agmm_amd import inputs as I
from gpu_util import BOUND, block_rows, rel_err, sample_rows, to_bits, to_device, torch_dtype

pytestmark = pytest.mark.gpu

BF16, FP16, FP32 = I.DTYPE_BF16, I.DTYPE_FP16, I.DTYPE_FP32


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    agmm.load_library()


def make_case(N, m_s, k, n, dtype, rt, seed, dist="normal"):
    w = I.custom_workload(N, m_s, k, n, dtype, rt, dist=dist, wid=seed)
    shards, B = I.make_inputs(w)
    return w, shards, B


def run_variant(w, shards_d, B_d, variant, **settings):
    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose,
                     variant=variant, **settings)
    try:
        C = plan.run(shards_d, B_d)
        torch.cuda.synchronize()
        return C, plan.get("variant_used")
    finally:
        plan.close()


def check_against_oracle(w, shards, B, C_d, rows=None):
    ref = oracle.agmm_f64(shards, B, w.dtype, w.rhs_transpose, rows=rows)
    Cb = to_bits(C_d if rows is None else C_d[torch.tensor(rows, device=C_d.device)])
    got = oracle.decode(Cb, w.dtype)
    err = rel_err(got, ref)
    assert np.all(np.isfinite(got))
    assert err <= BOUND[w.dtype], f"max rel err {err:.3e} > {BOUND[w.dtype]}"
    return err


# ---------------------------------------------------------------- small and ragged
SMALL = [
    # N, m_s, k, n, dtype, rhs_transpose
    (2, 64, 256, 128, FP32, False),
    (3, 100, 200, 136, BF16, False),
    (3, 100, 200, 130, FP16, True),
    (2, 300, 136, 264, BF16, True),
    (4, 77, 520, 96, FP16, False),
    (1, 513, 64, 257, BF16, True),
    (5, 1, 8, 8, BF16, False),
    (2, 33, 36, 5, FP32, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:4])) + f"_{I.DTYPE_NAMES[c[4]]}_rt{int(c[5])}")
@pytest.mark.parametrize("variant", ["fused", "staged", "unfused", "skinny"])
def test_small_ragged(case, variant):
    N, m_s, k, n, dtype, rt = case
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=17 + N + m_s)
    shards_d = [to_device(s, dtype) for s in shards]
    B_d = to_device(B, dtype)
    settings = {"pvalue": 1} if variant == "staged" else {}
    C, used = run_variant(w, shards_d, B_d, variant, **settings)
    check_against_oracle(w, shards, B, C)


@pytest.mark.parametrize("tile", list(range(agmm.NUM_TILES)))
@pytest.mark.parametrize("dtype,rt", [(BF16, False), (BF16, True), (FP16, False), (FP16, True)])
@pytest.mark.parametrize("k", [328, 384])
def test_tiles_ragged(tile, dtype, rt, k):
    """Every tile shape against the oracle on ragged m and n; k = 328 leaves a
    ragged last k-tile, k = 384 is whole 64-deep k-tiles, so interior tiles
    take the unmasked load path."""
    if tile in agmm.TILES_NEED_BT and not rt:
        pytest.skip("the 128x64 and skinny tiles take B stored n x k only")
    w, shards, B = make_case(3, 200, k, 392, dtype, rt, seed=900 + tile + k)
    shards_d = [to_device(s, dtype) for s in shards]
    B_d = to_device(B, dtype)
    C, _ = run_variant(w, shards_d, B_d, "fused", tile=tile)
    check_against_oracle(w, shards, B, C)


# ------------------------------------------- skinny kernel, whole k or k ranges
SKINNY_FULLK = [
    # N, m_s, k, n, dtype, extra plan settings
    (3, 50, 1000, 200, FP16, {}),       # 3 row blocks of 64 (the last ragged), ragged k-tile, ragged n
    (1, 7, 72, 33, BF16, {}),           # a single short k-tile: waves 2, 3 have none
    (8, 16, 4096, 1792, BF16, {}),      # the decode-like workload's shape
    (9, 30, 640, 130, FP16, {}),        # 9 shards, row blocks across shard boundaries
    (2, 100, 3000, 520, BF16, {"splits": 4}),   # 4 k ranges of 768 (the last 696)
    (3, 40, 264, 100, BF16, {"lda": 272, "ldb": 280, "ldc": 103}),
    (5, 13, 8, 16, BF16, {}),           # k = 8: one chunk of one k-tile
]


@pytest.mark.parametrize("split_mode", ["whole_k", "auto"])
@pytest.mark.parametrize("shape", [0, 1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("case", SKINNY_FULLK, ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}-d{c[4]}-{len(c[5])}")
def test_skinny_fullk_tile(case, shape, split_mode):
    """The skinny tile (wave-private LDS rings), every tile shape (64x16,
    32x32, 32x16, 16x32, 64x32, 64x64), over the whole of k and with the
    automatic k split (fp32 partial sums of each k range, then the
    fixed-order reduction), against the oracle on ragged m, n and k, strided
    operands; C's row padding untouched; a second run bit-identical."""
    N, m_s, k, n, dtype, extra = case
    extra = dict(extra)
    if split_mode == "whole_k":
        extra.setdefault("splits", 1)
    w, shards, B = make_case(N, m_s, k, n, dtype, True, seed=2200 + N + m_s + k + n)
    lda, ldb, ldc = extra.get("lda", k), extra.get("ldb", k), extra.get("ldc", n)
    dt = torch_dtype(dtype)
    sd = []
    for x in shards:
        buf = torch.full((m_s, lda), float("nan"), dtype=dt, device="cuda")
        buf[:, :k] = to_device(x, dtype)
        sd.append(buf[:, :k])
    bfull = torch.full((n, ldb), float("nan"), dtype=dt, device="cuda")
    bfull[:, :k] = to_device(B, dtype)
    C = torch.full((N * m_s, ldc), float("nan"), dtype=dt, device="cuda")
    plan = agmm.Plan(N, m_s, k, n, dtype, True, variant="skinny", tile=agmm.TILE_SKINNY, skinny_shape=shape, **extra)
    try:
        assert plan.get("tile") == agmm.TILE_SKINNY and plan.get("skinny_shape") == shape
        if "splits" in extra:
            assert plan.get("splits") == min(extra["splits"], -(-k // 64))
        plan.run(sd, bfull[:, :k], C[:, :n])
        torch.cuda.synchronize()
        first = to_bits(C[:, :n])
        check_against_oracle(w, shards, B, C[:, :n])
        if ldc > n:
            assert torch.isnan(C[:, n:].float()).all(), "wrote past n into the row padding"
        plan.run(sd, bfull[:, :k], C[:, :n])
        torch.cuda.synchronize()
        assert np.array_equal(first, to_bits(C[:, :n]))
    finally:
        plan.close()


@pytest.mark.parametrize("shape,tile,skinny_shape,splits", [
    ((8, 16, 4096, 1792), 10, 5, 1),       # 224 tiles of 32 x 32: whole k
    ((2, 16, 4096, 1024), 10, 5, 8),       # 32 tiles: 8 k ranges of 512
    ((4, 16, 8192, 1024), 10, 5, 4),       # 64 tiles: 4 k ranges
    ((2, 16, 4096, 256), 10, 5, 8),        # 8 tiles: k ranges of at least one k-tile per wave
    ((8, 16, 14336, 4096), 10, 7, 2),      # 512 tiles of 32 x 32, 128 of 64 x 64: 2 k ranges
    ((8, 16, 8192, 8192), 10, 7, 1),       # 256 tiles of 64 x 64: whole k
    ((16, 16, 4096, 1792), 7, None, None)])
def test_skinny_automatic_choice(shape, tile, skinny_shape, splits):
    """The skinny variant's automatic tile: for m <= 128 the skinny kernel,
    32 x 32 with k split into as many ranges as fill the CUs (each at least
    one 64-deep k-tile per wave), or 64 x 64 where 32 x 32 tiles would take
    more than one round of workgroups; the split-K 128x64 part ring for
    128 < m <= 256."""
    plan = agmm.Plan(*shape, BF16, True, variant="skinny")
    try:
        assert plan.get("tile") == tile
        if skinny_shape is not None:
            assert plan.get("skinny_shape") == skinny_shape
        if splits is not None:
            assert plan.get("splits") == splits
    finally:
        plan.close()


@pytest.mark.parametrize("dims,dtype", [((8, 16, 14336, 4096), BF16), ((4, 16, 8192, 1024), FP16)])
def test_skinny_split_large_against_oracle(dims, dtype):
    """Decode-like shapes on which the automatic skinny choice splits k
    (64 x 64 tiles with 2 k ranges; 32 x 32 with 4), checked in full against
    the oracle, and the second run bit-identical."""
    w, shards, B = make_case(*dims, dtype, True, seed=2400 + dims[2])
    sd = [to_device(x, dtype) for x in shards]
    bd = to_device(B, dtype)
    plan = agmm.Plan(*dims, dtype, True)
    try:
        assert plan.get("tile") == agmm.TILE_SKINNY and plan.get("splits") > 1
        C = torch.full((w.m, dims[3]), float("nan"), dtype=torch_dtype(dtype), device="cuda")
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
        first = to_bits(C)
        check_against_oracle(w, shards, B, C)
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
        assert np.array_equal(first, to_bits(C))
    finally:
        plan.close()


@pytest.mark.parametrize("shape,variant,want", [
    ((8, 1024, 8192, 3584, FP16, True), "fused", 11), ((8, 1024, 8192, 3584, FP16, True), "staged", 11),
    ((8, 4096, 8192, 7168, BF16, False), "fused", 8), ((8, 4096, 8192, 7168, BF16, True), "fused", 8)])
def test_tile_choice_fills_rounds(shape, variant, want):
    """The automatic tile: 256x224 (B stored n x k) where 256x256 tiles would
    leave a partial last round of workgroups (8192 x 3584: 448 tiles, 1.75
    rounds, against 512 tiles, 2 rounds; a staged chunk of 4096 rows: 224
    against 256 tiles, one round each), 256x256 otherwise."""
    settings = {"pvalue": 2, "nbuf": 2} if variant == "staged" else {}
    plan = agmm.Plan(*shape, variant=variant, **settings)
    try:
        assert plan.get("tile") == want
    finally:
        plan.close()


def test_skinny_fullk_needs_transposed_b():
    plan = agmm.Plan(2, 16, 64, 64, BF16, False, variant="skinny")
    try:
        with pytest.raises(agmm.AgmmError):
            plan.set("tile", agmm.TILE_SKINNY)
    finally:
        plan.close()


def test_skinny_fullk_in_staged_chunks():
    """The skinny tile under the staged variant: chunk launches map their rows to C
    through the chunk's row offset."""
    w, shards, B = make_case(3, 200, 384, 130, BF16, True, seed=2300)
    C, _ = run_variant(w, [to_device(x, BF16) for x in shards], to_device(B, BF16), "staged",
                       pvalue=1, tile=agmm.TILE_SKINNY)
    check_against_oracle(w, shards, B, C)


# ------------------------------------------------------------- the five workloads
def workload_inputs(wid):
    w = I.WORKLOADS[wid]
    shards, B = I.make_inputs(w)
    return w, shards, B, [to_device(s, w.dtype) for s in shards], to_device(B, w.dtype)


@pytest.mark.parametrize("variant", ["auto", "fused", "staged", "unfused"])
def test_workload1_fp32(variant):
    w, shards, B, sd, bd = workload_inputs(1)
    C, _ = run_variant(w, sd, bd, variant)
    check_against_oracle(w, shards, B, C)


@pytest.mark.parametrize("variant", ["auto", "fused", "staged", "unfused", "skinny"])
def test_workload2(variant):
    w, shards, B, sd, bd = workload_inputs(2)
    C, _ = run_variant(w, sd, bd, variant)
    check_against_oracle(w, shards, B, C)


@pytest.mark.parametrize("variant", ["auto", "fused", "skinny", "unfused"])
def test_workload3_skinny(variant):
    w, shards, B, sd, bd = workload_inputs(3)
    C, used = run_variant(w, sd, bd, variant)
    if variant == "auto":
        assert used == agmm.AGMM_VARIANT_SKINNY
    check_against_oracle(w, shards, B, C)


@pytest.mark.parametrize("variant", ["staged", "fused", "unfused"])
def test_workload4_sampled(variant):
    w, shards, B, sd, bd = workload_inputs(4)
    settings = {"pvalue": w.pvalue, "nbuf": w.nbuf} if variant == "staged" else {}
    C, _ = run_variant(w, sd, bd, variant, **settings)
    rows = sample_rows(w.num_shards, w.m_per_shard, per_shard=3, seed=4)
    check_against_oracle(w, shards, B, C, rows=rows)


def test_workload4_every_tile():
    """Workload 4 (fp16, B n x k): two rows of every 256-row block, one in
    each 128-row wave half, all columns, so every 256 x 256 output tile and
    every wave's sub-tile is compared with the oracle; fused and unfused
    (same tile, same k order per element) are bit-identical."""
    w, shards, B, sd, bd = workload_inputs(4)
    outs = {}
    for variant in ("fused", "unfused"):
        plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose,
                         variant=variant)
        try:
            C = torch.full((w.m, w.n_local), float("nan"), dtype=torch_dtype(w.dtype), device="cuda")
            plan.run(sd, bd, C)
            torch.cuda.synchronize()
            outs[variant] = (C, plan.get("tile"), plan.get("splits"))
        finally:
            plan.close()
    C = outs["fused"][0]
    assert not torch.isnan(C.float()).any().item(), "some outputs were never written"
    check_against_oracle(w, shards, B, C, rows=block_rows(w.m, seed=4))
    assert outs["fused"][1:] == outs["unfused"][1:]
    assert torch.equal(C.view(torch.int16), outs["unfused"][0].view(torch.int16))


@pytest.mark.parametrize("wid", [2, 3])
def test_workload_graph_of_calls_over_buffer_sets(wid):
    """Workloads 2 and 3 in the form their short steps are timed: 20 calls
    of one plan (the automatic path: split-K 128x128 tiles, the skinny
    kernel) captured into one HIP graph on a side stream, each call on the
    next of several buffer sets.  Here every set holds its own seeded inputs,
    so a call that read another set's operands or wrote another set's output
    would show: two replays, every set's C against the oracle and
    bit-identical to an eager call on that set."""
    w = I.WORKLOADS[wid]
    nsets, calls = 8, 20
    sets, host = [], []
    for i in range(nsets):
        shards, B = I.make_inputs(w, seed_base=5000 + 10 * wid + i)
        host.append((shards, B))
        sets.append(([to_device(x, w.dtype) for x in shards], to_device(B, w.dtype),
                     torch.empty((w.m, w.n_local), dtype=torch_dtype(w.dtype), device="cuda")))
    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose)
    try:
        assert plan.get("splits") > 1 or plan.get("tile") == agmm.TILE_SKINNY
        eager = []
        for sd, bd, _ in sets:
            eager.append(to_bits(plan.run(sd, bd)))
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for c in range(calls):
                    sd, bd, C = sets[c % nsets]
                    plan.run(sd, bd, C, stream=side)
        torch.cuda.synchronize()
        for rep in range(2):
            for _, _, C in sets:
                C.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for i, ((shards, B), (_, _, C)) in enumerate(zip(host, sets)):
                bits = to_bits(C)
                assert np.array_equal(bits, eager[i]), f"replay {rep}, set {i}: differs from eager"
                if rep == 0:
                    check_against_oracle(w, shards, B, C)
        del g
    finally:
        plan.close()


@pytest.mark.parametrize("wid", [2, 4])
def test_staged_one_call_graphs_over_buffer_sets(wid):
    """Workloads 2 and 4 staged (pvalue 2, two slots) in the form their
    steps are timed: one HIP graph per buffer set, each holding one staged
    call, the graphs replayed in turn.  Every set has its own inputs; every
    replay of every set matches an eager call bit for bit, and the oracle
    (workload 2 in full, workload 4 on two rows of every 256-row block)."""
    w = I.WORKLOADS[wid]
    nsets = 4
    host, sets = [], []
    for i in range(nsets):
        shards, B = I.make_inputs(w, seed_base=5100 + 10 * wid + i)
        host.append((shards, B))
        sets.append(([to_device(x, w.dtype) for x in shards], to_device(B, w.dtype),
                     torch.empty((w.m, w.n_local), dtype=torch_dtype(w.dtype), device="cuda")))
    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose,
                     variant="staged", pvalue=2, nbuf=2)
    try:
        assert plan.get("num_chunks") <= plan.get("num_slots")
        eager = [to_bits(plan.run(sd, bd)) for sd, bd, _ in sets]
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        for sd, bd, C in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    plan.run(sd, bd, C, stream=side)
            graphs.append(g)
        torch.cuda.synchronize()
        for rep in range(2):
            for _, _, C in sets:
                C.fill_(float("nan"))
            torch.cuda.synchronize()
            for g in graphs:
                g.replay()
            torch.cuda.synchronize()
            for i, ((shards, B), (_, _, C)) in enumerate(zip(host, sets)):
                assert np.array_equal(to_bits(C), eager[i]), f"replay {rep}, set {i}"
                if rep == 0:
                    check_against_oracle(w, shards, B, C,
                                         rows=None if wid == 2 else block_rows(w.m, seed=i))
        del graphs
    finally:
        plan.close()


def test_workload5_every_tile_every_variant():
    """Workload 5, the benchmarked configuration (8 x 4096 x 8192 -> 7168
    bf16), through the fused, staged (pvalue 2, 2 slots: 8 chunks, each slot
    reused four times) and unfused paths.  C starts as NaN and no NaN may
    remain.  The oracle checks two rows of every 256-row block (one in each
    128-row wave half, at offsets that vary from block to block) over all
    7168 columns: every one of the 3584 output tiles and every wave's
    sub-tile.  The three paths use tiles of the 16x16x32 ring (the staged
    chunks may take 256x224 tiles where the fused launch takes 256x256), which
    share the k order per element, and the same splits, so their outputs must
    also be bit-identical, which covers every element of the staged and
    unfused outputs."""
    w, shards, B, sd, bd = workload_inputs(5)
    rows = block_rows(w.m, seed=5)
    outs = {}
    for variant in ("fused", "staged", "unfused"):
        settings = {"pvalue": 2, "nbuf": 2} if variant == "staged" else {}
        plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose,
                         variant=variant, **settings)
        try:
            if variant == "staged":
                assert plan.get("num_chunks") == 8 and plan.get("num_slots") == 2
            C = torch.full((w.m, w.n_local), float("nan"), dtype=torch_dtype(w.dtype), device="cuda")
            plan.run(sd, bd, C)
            torch.cuda.synchronize()
            outs[variant] = (plan.get("tile"), plan.get("splits"))
        finally:
            plan.close()
        assert not torch.isnan(C.float()).any().item(), f"{variant}: some outputs were never written"
        check_against_oracle(w, shards, B, C, rows=rows)
        if variant == "fused":
            C_fused = C
        else:
            ring16 = {agmm.TILES["256x256_m16"], agmm.TILES["128x128_m16"], agmm.TILES["256x224_m16"]}
            assert {outs[variant][0], outs["fused"][0]} <= ring16, (variant, outs)
            assert outs[variant][1] == outs["fused"][1], (variant, outs)
            assert torch.equal(C.view(torch.int16), C_fused.view(torch.int16)), variant
            del C


# ---------------------------------------------------------------- gather, exact
@pytest.mark.parametrize("dtype", [BF16, FP16, FP32])
def test_gather_bit_exact(dtype):
    w, shards, B = make_case(5, 37, 264, 8, dtype, False, seed=77)
    sd = [to_device(s, dtype) for s in shards]
    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, dtype, False)
    try:
        G = plan.gather(sd)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert np.array_equal(to_bits(G), oracle.gather(shards, dtype))


DEGENERATE = [
    # N, m_s, k, n, dtype, rhs_transpose
    (1, 1, 8, 1, BF16, True),      # one output element, one 16-byte chunk of k
    (1, 1, 1, 1, FP32, False),     # one multiply
    (3, 1, 16, 1, FP16, True),     # one column, one row per shard
    (1, 1, 7, 1, BF16, False),     # padded k and n
    (2, 1, 3000, 1, BF16, True),   # one column over a long k
    (1, 300, 8, 1, FP16, True),    # one tall column, k of one chunk
]


@pytest.mark.parametrize("variant", ["auto", "fused", "staged", "unfused", "skinny"])
@pytest.mark.parametrize("case", DEGENERATE, ids=lambda c: "x".join(map(str, c[:4])) + f"_{I.DTYPE_NAMES[c[4]]}_rt{int(c[5])}")
def test_degenerate_shapes(case, variant):
    """Single rows, single columns and single elements through every variant
    (the skinny variant falls back to the fused path for fp32) against the
    oracle; C's bits identical on a second run."""
    N, m_s, k, n, dtype, rt = case
    if variant == "skinny" and N * m_s > 256:
        pytest.skip("the skinny variant is for m <= 256")
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=3300 + k + n + m_s)
    sd = [to_device(x, dtype) for x in shards]
    bd = to_device(B, dtype)
    plan = agmm.Plan(N, m_s, k, n, dtype, rt, variant=variant)
    try:
        C = plan.run(sd, bd)
        torch.cuda.synchronize()
        first = to_bits(C)
        check_against_oracle(w, shards, B, C)
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
        assert np.array_equal(first, to_bits(C))
    finally:
        plan.close()


@pytest.mark.parametrize("variant,dtype,rt,m_s,settings", [
    ("fused", BF16, False, 5, {}), ("fused", FP16, True, 9, {"tile": 11}),
    ("staged", BF16, True, 7, {"pvalue": 1, "nbuf": 2}), ("unfused", FP16, False, 3, {}),
    ("skinny", BF16, True, 2, {}), ("skinny", BF16, True, 1, {"splits": 3}),
    ("skinny", FP16, True, 4, {"skinny_shape": 7, "splits": 2}), ("fused", FP32, False, 3, {})])
def test_most_shards(variant, dtype, rt, m_s, settings):
    """64 shards, the largest pointer table a call can pass: every variant
    (with the skinny kernel over whole k and over k ranges) against the
    oracle, and the gather of all 64 bit-exact."""
    N, k, n = 64, 328, 136
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=3100 + m_s)
    sd = [to_device(x, dtype) for x in shards]
    C, _ = run_variant(w, sd, to_device(B, dtype), variant, **settings)
    check_against_oracle(w, shards, B, C)
    plan = agmm.Plan(N, m_s, k, n, dtype, rt)
    try:
        G = plan.gather(sd)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert np.array_equal(to_bits(G), oracle.gather(shards, dtype))


@pytest.mark.parametrize("dtype,k,lda", [
    (BF16, 8, 0), (BF16, 56, 0), (BF16, 264, 0), (BF16, 2040, 0), (BF16, 2048, 0),
    (BF16, 2056, 0), (FP16, 8000, 0), (FP32, 4, 0), (FP32, 1028, 0), (BF16, 264, 280)])
def test_gather_row_shapes_bit_exact(dtype, k, lda):
    """The gather copy's work split: rows shorter than 256 16-byte chunks
    packed several to a workgroup (with a partial last workgroup), rows of
    exactly 256 chunks, rows with a partial last 256-chunk block, and a
    row-strided source (lda > k, NaN in the gaps)."""
    N, m_s = 5, 37
    w, shards, B = make_case(N, m_s, k, 8, dtype, False, seed=990 + k)
    tdt = torch_dtype(dtype)
    if lda:
        sd = []
        for x in shards:
            t = torch.full((m_s, lda), float("nan"), dtype=tdt, device="cuda")
            t[:, :k] = to_device(x, dtype)
            sd.append(t[:, :k])
    else:
        sd = [to_device(x, dtype) for x in shards]
    plan = agmm.Plan(N, m_s, k, 8, dtype, False, **({"lda": lda} if lda else {}))
    try:
        G = torch.full((N * m_s, k), float("nan"), dtype=tdt, device="cuda")
        plan.gather(sd, G)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert np.array_equal(to_bits(G), oracle.gather(shards, dtype))


def test_gather_capped_grid_strides_bit_exact():
    """A copy whose grid is capped below its work items (the side copy of
    agmm_run_gather_out with copy_wgs 3) walks the items in strides: the
    gathered output is still the bit-exact concatenation, and C matches."""
    N, m_s, k, n, dtype = 4, 300, 2056, 72, BF16
    w, shards, B = make_case(N, m_s, k, n, dtype, True, seed=995)
    sd = [to_device(x, dtype) for x in shards]
    plan = agmm.Plan(N, m_s, k, n, dtype, True, variant="fused", gather_out=1, copy_wgs=3)
    try:
        C, G = plan.run_gather_out(sd, to_device(B, dtype))
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert np.array_equal(to_bits(G), np.concatenate(shards, axis=0))
    check_against_oracle(w, shards, B, C)


def test_gather_larger_than_mall_bit_exact():
    """A gather above 256 MiB (workload 5's 8 shards x 4096 x 8192 bf16 =
    512 MiB; the copy then uses non-temporal stores): bit-exact against the
    concatenation, checked in full on the device and on sampled rows
    against the host inputs."""
    w = I.WORKLOADS[5]
    shards, _ = I.make_inputs(w)
    sd = [to_device(x, w.dtype) for x in shards]
    G = torch.empty((w.m, w.k), dtype=torch_dtype(w.dtype), device="cuda")
    G.fill_(float("nan"))
    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose)
    try:
        plan.gather(sd, G)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert torch.equal(G.view(torch.int16), torch.cat(sd, 0).view(torch.int16))
    for r in sample_rows(w.num_shards, w.m_per_shard, per_shard=2, seed=5):
        s_, i = divmod(r, w.m_per_shard)
        assert np.array_equal(to_bits(G[r:r + 1])[0], shards[s_][i])
    del G, sd


@pytest.mark.parametrize("copy_engine", [0, 1])
def test_staged_slots_bit_exact(copy_engine):
    """debug_keep_slots: every chunk keeps its own slot; each equals the
    oracle gather's rows of that chunk, whether the gather kernel or the
    SDMA engines copied it."""
    w, shards, B = make_case(3, 300, 128, 64, BF16, True, seed=78)
    sd = [to_device(s, BF16) for s in shards]
    bd = to_device(B, BF16)
    plan = agmm.Plan(3, 300, 128, 64, BF16, True, variant="staged", pvalue=1, tile=1,
                     debug_keep_slots=1, copy_engine=copy_engine)
    try:
        C = plan.run(sd, bd)
        torch.cuda.synchronize()
        R = plan.get("rows_per_chunk")
        nch = plan.get("num_chunks")
        assert R == 128 and nch == 3
        G = oracle.gather(shards, BF16)
        for c in range(nch):
            ptr = agmm.agmm_plan_slot_ptr(plan.handle, c)
            rows_c = min(R, 300 - c * R)
            nbytes = 3 * rows_c * 128 * 2
            host = np.empty(nbytes // 2, dtype=np.uint16)
            import ctypes
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
            assert hip.hipMemcpy(host.ctypes.data, ptr, nbytes, 2) == 0  # device -> host
            host = host.reshape(3, rows_c, 128)
            for r in range(3):
                want = G[r * 300 + c * R: r * 300 + c * R + rows_c]
                assert np.array_equal(host[r], want), (c, r)
    finally:
        plan.close()
    check_against_oracle(w, shards, B, C)


# -------------------------------------------------- schedule invariance, exact
def test_schedule_orders_bit_identical():
    w, shards, B = make_case(4, 384, 256, 512, BF16, False, seed=79)
    sd = [to_device(s, BF16) for s in shards]
    bd = to_device(B, BF16)
    outs = []
    for order, r0 in [(1, 0), (0, 0), (0, 1), (0, 3)]:
        C, _ = run_variant(w, sd, bd, "fused", order=order, local_shard=r0, tile=0)
        outs.append(to_bits(C))
    for o in outs[1:]:
        assert np.array_equal(outs[0], o)
    # same microkernel and tile: fused, staged and unfused agree bit for bit
    Cs, _ = run_variant(w, sd, bd, "staged", pvalue=1, tile=0)
    Cu, _ = run_variant(w, sd, bd, "unfused", tile=0)
    assert np.array_equal(outs[0], to_bits(Cs))
    assert np.array_equal(outs[0], to_bits(Cu))
    check_against_oracle(w, shards, B, Cs)


def test_ring_order_table():
    plan = agmm.Plan(4, 512, 64, 128, BF16, False, variant="fused", tile=0, local_shard=1)
    try:
        order = plan.tile_order()
    finally:
        plan.close()
    # 4 shards x 2 row blocks of 256: top halves are row blocks 2r, bottom 2r+1.
    # step 0: top of shard 1, bottom of shard 1; step 1: top of 2, bottom of 0;
    # step 2: top of 3, bottom of 3; step 3: top of 0, bottom of 2.
    assert order == [2, 3, 4, 1, 6, 7, 0, 5]


def test_identity_returns_gathered_exactly():
    for dtype, rt in [(BF16, False), (FP16, True), (FP32, False)]:
        N, m_s, k = 3, 70, 64
        w, shards, _ = make_case(N, m_s, k, k, dtype, rt, seed=80)
        eye = I.to_storage_bits(np.eye(k, dtype=np.float32), dtype)
        sd = [to_device(s, dtype) for s in shards]
        C, _ = run_variant(w, sd, to_device(eye, dtype), "fused")
        assert np.array_equal(to_bits(C), oracle.gather(shards, dtype))


def test_fp16_subnormal_outputs():
    """Outputs deep in the fp16 subnormal range must not be flushed."""
    N, m_s, k, n = 2, 64, 64, 64
    rng = np.random.default_rng(81)
    shards = [I.to_storage_bits((rng.standard_normal((m_s, k)) * 2e-3).astype(np.float32), FP16)
              for _ in range(N)]
    B = I.to_storage_bits((rng.standard_normal((k, n)) * 2e-3).astype(np.float32), FP16)
    w = I.custom_workload(N, m_s, k, n, FP16, False)
    C, _ = run_variant(w, [to_device(s, FP16) for s in shards], to_device(B, FP16), "fused")
    ref = oracle.agmm_f64(shards, B, FP16, False)
    got = oracle.decode(to_bits(C), FP16)
    assert (np.abs(ref) < 2.0 ** -14).mean() > 0.5      # mostly subnormal outputs
    assert (np.abs(got) > 0).mean() > 0.9                # and they survived
    assert rel_err(got, ref) <= BOUND[FP16]


@pytest.mark.parametrize("tile,splits", [(3, 4), (3, 7), (1, 3), (2, 2), (0, 11), (4, 9), (6, 3), (7, 5)])
def test_split_k_ragged(tile, splits):
    """Split-K partials + fixed-order reduction, with a ragged last k range."""
    rt = tile in agmm.TILES_NEED_BT
    w, shards, B = make_case(2, 50, 968, 200 if rt else 208, FP16, rt, seed=400 + tile + splits)
    C, used = run_variant(w, [to_device(s, FP16) for s in shards], to_device(B, FP16), "skinny",
                          tile=tile, splits=splits)
    assert used == agmm.AGMM_VARIANT_SKINNY
    check_against_oracle(w, shards, B, C)


@pytest.mark.parametrize("tile", [8, 9, 11])
@pytest.mark.parametrize("dtype,rt", [(BF16, False), (BF16, True), (FP16, False), (FP16, True)])
@pytest.mark.parametrize("splits,k", [(1, 1024), (3, 1024), (1, 1000)])
def test_mfma16_tiles(tile, dtype, rt, splits, k):
    """The 16x16x32-MFMA tiles on whole interior tiles (m, n multiples of the
    tile, whole k-tiles in every k range: the unmasked loop with its pinned
    interleave), with split-K, and with a ragged k (masked loop).  Tile 11
    (256x224, B stored n x k) has 7 column blocks per wave: halves of 4 and
    3 blocks, and C rows of 28 16-byte chunks in the staged epilogue."""
    if tile in agmm.TILES_NEED_BT and not rt:
        pytest.skip("B stored n x k only")
    n = 448 if tile == 11 else 512
    w, shards, B = make_case(2, 512, k, n, dtype, rt, seed=1600 + tile + splits + k)
    C, _ = run_variant(w, [to_device(s, dtype) for s in shards], to_device(B, dtype), "fused",
                       tile=tile, splits=splits)
    check_against_oracle(w, shards, B, C)


@pytest.mark.parametrize("variant,tile,splits,rt,pvalue", [
    ("fused", 5, 3, False, None), ("fused", 1, 0, False, None), ("unfused", 6, 2, True, None),
    ("fused", 0, 2, True, None), ("fused", 5, 0, True, None),
    ("staged", 6, 2, False, 1), ("staged", 7, 0, True, 1)])
def test_split_k_variants(variant, tile, splits, rt, pvalue):
    """Split-K on the fused, unfused and staged variants (explicit and
    automatic k ranges; staged: per chunk, two chunks with a ragged second
    one), ragged m, n and a ragged last k range."""
    w, shards, B = make_case(2, 200, 2248, 264, BF16, rt, seed=450 + tile + splits)
    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, BF16, rt, variant=variant,
                     tile=tile, splits=splits, pvalue=pvalue)
    try:
        assert plan.get("splits") > 1
        C = plan.run([to_device(s, BF16) for s in shards], to_device(B, BF16))
        torch.cuda.synchronize()
        check_against_oracle(w, shards, B, C)
    finally:
        plan.close()


@pytest.mark.parametrize("dtype,rt", [(BF16, False), (FP16, True)])
def test_staged_slot_reuse_alternating_streams(dtype, rt):
    """Four chunks through two ring slots (each slot reused), chunk GEMMs
    alternating between the plan's two GEMM streams: same bits as the fused
    path with the same tile, and the oracle's values."""
    w, shards, B = make_case(3, 400, 256, 264, dtype, rt, seed=500 + dtype)
    sd = [to_device(x, dtype) for x in shards]
    bd = to_device(B, dtype)
    out = {}
    for variant, extra in (("staged", {"pvalue": 1, "nbuf": 2}), ("fused", {})):
        plan = agmm.Plan(3, 400, 256, 264, dtype, rt, variant=variant, tile=6, splits=1, **extra)
        try:
            if variant == "staged":
                assert plan.get("num_chunks") == 4
            for _ in range(2):      # twice: the second run reuses the ring and events
                out[variant] = plan.run(sd, bd)
            torch.cuda.synchronize()
        finally:
            plan.close()
    assert np.array_equal(to_bits(out["staged"]), to_bits(out["fused"]))
    check_against_oracle(w, shards, B, out["staged"])


def strided(t, ld):
    """A copy of the 2-D tensor t as a row-strided view (rows ld elements apart)."""
    big = torch.full((t.shape[0], ld), float("nan"), dtype=t.dtype, device=t.device)
    big[:, :t.shape[1]] = t
    return big[:, :t.shape[1]]


@pytest.mark.parametrize("variant,dtype,rt,lds", [
    ("fused", BF16, False, (264, 208, 216)), ("fused", FP16, True, (320, 264, 200)),
    ("staged", BF16, True, (256, 312, 136)), ("unfused", FP16, False, (248, 144, 200)),
    ("skinny", BF16, True, (248, 248, 129)), ("fused", FP32, False, (252, 132, 131))])
def test_strided_inputs(variant, dtype, rt, lds):
    """Row strides for the shards (lda), B (ldb) and C (ldc) on every path;
    padding columns hold NaN, so reading them would show in C, and C's own
    padding must stay untouched."""
    lda, ldb, ldc = lds
    m_s = 40 if variant == "skinny" else 200
    w, shards, B = make_case(3, m_s, 240, 128, dtype, rt, seed=510 + lda)
    plan = agmm.Plan(3, m_s, 240, 128, dtype, rt, variant=variant,
                     **({"pvalue": 1, "tile": 6} if variant == "staged" else {}))
    try:
        plan.set("lda", lda)
        plan.set("ldb", ldb)
        plan.set("ldc", ldc)
        assert (plan.get("lda"), plan.get("ldb"), plan.get("ldc")) == (lda, ldb, ldc)
        sd = [strided(to_device(x, dtype), lda) for x in shards]
        bd = strided(to_device(B, dtype), ldb)
        c_full = torch.full((w.m, ldc), float("nan"), dtype=sd[0].dtype, device="cuda")
        C = plan.run(sd, bd, c_full[:, :w.n_local])
        C2, G = plan.run_gather_out(sd, bd)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert C2.stride() == (ldc, 1)
    assert bool(torch.isnan(c_full[:, w.n_local:].float()).all())   # C's padding untouched
    assert np.array_equal(to_bits(G), np.concatenate(shards, axis=0))
    assert np.array_equal(to_bits(C), to_bits(C2))
    check_against_oracle(w, shards, B, C)


PADDED = [
    # N, m_s, k, n, dtype, rhs_transpose: rows that are not whole 16-byte vectors
    (3, 50, 100, 130, BF16, False),    # k % 8 == 4, n % 8 == 2 with B stored k x n
    (2, 33, 257, 65, FP16, True),      # odd k
    (4, 64, 1000, 300, BF16, False),   # n % 8 == 4 only (k whole)
    (1, 7, 13, 5, FP16, False),        # everything tiny and odd
    (2, 40, 2051, 96, BF16, True),     # a long ragged k (split-K over the padded k)
]


@pytest.mark.parametrize("variant", ["auto", "fused", "staged", "skinny"])
@pytest.mark.parametrize("case", PADDED, ids=lambda c: "x".join(map(str, c[:4])) + f"_{I.DTYPE_NAMES[c[4]]}_rt{int(c[5])}")
def test_padded_shapes(case, variant):
    """bf16/fp16 problems whose rows are not whole 16-byte vectors run on
    zero-padded copies of A and B (every requested variant resolves to that
    gather-then-GEMM form): the oracle's values; C's padding untouched."""
    N, m_s, k, n, dtype, rt = case
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=2800 + N + m_s + k + n)
    sd = [to_device(x, dtype) for x in shards]
    bd = to_device(B, dtype)
    plan = agmm.Plan(N, m_s, k, n, dtype, rt, variant=variant)
    try:
        assert plan.get("variant_used") == agmm.VARIANTS["unfused"]
        c_full = torch.full((w.m, n + 3), float("nan"), dtype=torch_dtype(dtype), device="cuda")
        plan.set("ldc", n + 3)
        C = plan.run(sd, bd, c_full[:, :n])
        C2, G = plan.run_gather_out(sd, bd)
        C3 = plan.run_gathered(G, bd)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert bool(torch.isnan(c_full[:, n:].float()).all())
    assert np.array_equal(to_bits(G), np.concatenate(shards, axis=0))
    assert np.array_equal(to_bits(C), to_bits(C2)) and np.array_equal(to_bits(C), to_bits(C3))
    check_against_oracle(w, shards, B, C)


def test_padded_strided_and_split():
    """A padded problem with row strides that are not 16-byte multiples
    (allowed where rows go through the element copy) and explicit split-K."""
    N, m_s, k, n, dtype, rt = 3, 70, 1003, 77, FP16, True
    lda, ldb = 1005, 1010
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=2900)
    plan = agmm.Plan(N, m_s, k, n, dtype, rt, splits=2)
    try:
        plan.set("lda", lda)
        plan.set("ldb", ldb)
        assert plan.get("splits") == 2
        sd = [strided(to_device(x, dtype), lda) for x in shards]
        bd = strided(to_device(B, dtype), ldb)
        C = plan.run(sd, bd)
        G = plan.gather(sd)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert np.array_equal(to_bits(G), np.concatenate(shards, axis=0))
    check_against_oracle(w, shards, B, C)


@pytest.mark.parametrize("dtype,k", [(BF16, 13), (FP16, 302), (FP32, 37)])
def test_gather_any_row_length(dtype, k):
    """agmm_gather with rows that are not whole 16-byte vectors (the element
    copy): bit-exact."""
    w, shards, _ = make_case(4, 29, k, 8, dtype, True, seed=3000 + k)
    sd = [to_device(x, dtype) for x in shards]
    plan = agmm.Plan(4, 29, k, 8, dtype, True)
    try:
        G = plan.gather(sd)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert np.array_equal(to_bits(G), oracle.gather(shards, dtype))


def test_stride_keys_validated():
    plan = agmm.Plan(2, 16, 64, 40, BF16, True)
    try:
        for key, bad in (("lda", 63), ("lda", 68), ("ldb", 60), ("ldb", 66), ("ldc", 39)):
            with pytest.raises(agmm.AgmmError):
                plan.set(key, bad)
        plan.set("lda", 72)
        plan.set("ldc", 41)
        plan.set("lda", 0)
        assert plan.get("lda") == 64 and plan.get("ldc") == 41 and plan.get("ldb") == 64
    finally:
        plan.close()


@pytest.mark.parametrize("variant,dtype,rt", [("fused", BF16, False), ("skinny", FP16, True),
                                              ("staged", BF16, True), ("fused", FP32, True)])
def test_autotune_keeps_a_correct_configuration(variant, dtype, rt):
    """agmm_plan_autotune times its candidates, keeps one, and the plan then
    computes the oracle's values (the tuned C too)."""
    m_s = 24 if variant == "skinny" else 200
    w, shards, B = make_case(3, m_s, 320, 136, dtype, rt, seed=530 + dtype)
    sd = [to_device(x, dtype) for x in shards]
    bd = to_device(B, dtype)
    plan = agmm.Plan(3, m_s, 320, 136, dtype, rt, variant=variant)
    try:
        C_tuned = torch.empty((w.m, w.n_local), dtype=sd[0].dtype, device="cuda")
        best = plan.autotune(sd, bd, C_tuned, iters=2)
        assert best > 0
        assert plan.get("variant_used") == agmm.VARIANTS[variant]
        C = plan.run(sd, bd)
        torch.cuda.synchronize()
    finally:
        plan.close()
    check_against_oracle(w, shards, B, C)
    check_against_oracle(w, shards, B, C_tuned)


def _random_cases(count, seed):
    """Seeded random problems across the plan's settings (shapes kept small
    enough for the oracle)."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < count:
        dtype = int(rng.choice([BF16, FP16, FP32]))
        rt = bool(rng.integers(2))
        N = int(rng.integers(1, 10))
        m_s = int(rng.choice([1, 2, 7, 16, 33, 64, 100, 129, 256, 300]))
        k = 8 * int(rng.integers(1, 70))
        n = int(rng.integers(1, 300))
        if dtype != FP32 and not rt:
            n = 8 * max(1, n // 8)
        variant = str(rng.choice(["auto", "fused", "staged", "unfused", "skinny"]))
        if variant == "skinny" and (N * m_s > 256 or dtype == FP32):
            variant = "fused"
        settings = {"variant": variant}
        if dtype != FP32 and rng.random() < 0.6:
            tiles = [0, 1, 2, 5, 6, 8, 9] + (list(agmm.TILES_NEED_BT) if rt else [])
            settings["tile"] = int(rng.choice(tiles))
            if variant in ("fused", "unfused", "skinny", "staged") and rng.random() < 0.5:
                settings["splits"] = int(rng.integers(1, 6))
            if settings["tile"] == agmm.TILE_SKINNY:
                settings["skinny_shape"] = int(rng.integers(0, 8))
        if variant == "staged":
            settings["pvalue"] = int(rng.integers(1, 3))
            settings["nbuf"] = int(rng.integers(1, 4))
        if N * m_s * k * n > 6e7:
            continue
        cases.append((N, m_s, k, n, dtype, rt, settings))
    return cases


@pytest.mark.parametrize("case", _random_cases(96, 2024), ids=lambda c: f"{c[0]}x{c[1]}x{c[2]}x{c[3]}-d{c[4]}-t{int(c[5])}-{c[6]}")
def test_random_problems(case):
    """Randomized cross-check of every variant, tile and split setting against
    the oracle on small ragged problems (fixed seed, so failures reproduce)."""
    N, m_s, k, n, dtype, rt, settings = case
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=sum(case[:4]) + dtype)
    C, _ = run_variant(w, [to_device(x, dtype) for x in shards], to_device(B, dtype), **settings)
    check_against_oracle(w, shards, B, C)


def test_repeated_runs_fresh_inputs():
    """Back-to-back runs with new inputs (staged ring reuse, split-K counters
    reset): every run matches its own oracle."""
    for variant, settings in [("staged", {"pvalue": 1, "tile": 1, "nbuf": 2}), ("skinny", {})]:
        plan = None
        try:
            for it in range(3):
                w, shards, B = make_case(4, 160 if variant == "staged" else 24, 192, 256, BF16,
                                         True, seed=300 + it)
                if plan is None:
                    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, BF16, True,
                                     variant=variant, **settings)
                C = plan.run([to_device(s, BF16) for s in shards], to_device(B, BF16))
                torch.cuda.synchronize()
                check_against_oracle(w, shards, B, C)
        finally:
            if plan is not None:
                plan.close()


@pytest.mark.parametrize("variant,settings", [
    ("fused", {}), ("skinny", {}), ("unfused", {}), ("fused", {"splits": 3}),
    ("skinny", {"splits": 3}),                                   # the skinny kernel's k ranges + reduction
    ("staged", {"pvalue": 1, "tile": 1, "nbuf": 2}),
    ("staged", {"pvalue": 1, "tile": 6, "nbuf": 2, "splits": 2})])
def test_graph_capture_replays(variant, settings):
    """agmm_run captured into a HIP graph (launches, and for the staged plan
    the copy stream and second GEMM stream joined through events) and
    replayed on new inputs written into the captured buffers: every replay
    matches the oracle and is bit-identical to an eager run."""
    m_s = 24 if variant == "skinny" else 160
    N, k, n, dtype, rt = 4, 384, 264, BF16, True
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=900)
    plan = agmm.Plan(N, m_s, k, n, dtype, rt, variant=variant, **settings)
    try:
        sd = [to_device(s, dtype) for s in shards]
        bd = to_device(B, dtype)
        C = torch.empty((N * m_s, n), dtype=torch.bfloat16, device="cuda")
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.run(sd, bd, C)
        torch.cuda.synchronize()
        assert plan.get("captured") == 1
        with pytest.raises(agmm.AgmmError) as ei:
            plan.set("group_m", 8)          # the graph holds the current layout
        assert ei.value.status == agmm.AGMM_ERR_UNSUPPORTED
        for rep in range(3):
            w2, sh2, B2 = make_case(N, m_s, k, n, dtype, rt, seed=901 + rep)
            for d, h in zip(sd, sh2):
                d.copy_(to_device(h, dtype))
            bd.copy_(to_device(B2, dtype))
            C.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            check_against_oracle(w2, sh2, B2, C)
            C_eager = plan.run(sd, bd)
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(C), to_bits(C_eager))
        del g
    finally:
        plan.close()


def test_graph_capture_refuses_untested_staged_forms():
    """Under graph capture a staged plan accepts one call per graph with at
    most as many chunks as ring slots; a plan that refills slots within a call,
    or a second staged call in the same capture, is refused before anything is
    enqueued, and the capture and the plan stay usable."""
    N, k, n, dtype, rt = 4, 256, 136, BF16, True
    # (a) 4 chunks over 2 slots: eager runs work, capture refuses
    w, shards, B = make_case(N, 400, k, n, dtype, rt, seed=940)
    plan = agmm.Plan(N, 400, k, n, dtype, rt, variant="staged", pvalue=1, tile=1, nbuf=2)
    try:
        assert plan.get("num_chunks") == 4 and plan.get("num_slots") == 2
        sd = [to_device(x, dtype) for x in shards]
        bd = to_device(B, dtype)
        C = torch.empty((N * 400, n), dtype=torch.bfloat16, device="cuda")
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            with pytest.raises(agmm.AgmmError) as ei:
                plan.run(sd, bd, C)
            assert ei.value.status == agmm.AGMM_ERR_UNSUPPORTED
            C.fill_(0.0)                  # the capture goes on
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert not torch.any(C).item()
        del g
        C2 = plan.run(sd, bd)             # still usable eagerly
        torch.cuda.synchronize()
        check_against_oracle(w, shards, B, C2)
    finally:
        plan.close()
    # (b) 2 chunks over 2 slots: the first call is captured, a second is refused
    w, shards, B = make_case(N, 160, k, n, dtype, rt, seed=941)
    plan = agmm.Plan(N, 160, k, n, dtype, rt, variant="staged", pvalue=1, tile=1, nbuf=2)
    try:
        assert plan.get("num_chunks") == 2 and plan.get("num_slots") == 2
        sd = [to_device(x, dtype) for x in shards]
        bd = to_device(B, dtype)
        C = torch.empty((N * 160, n), dtype=torch.bfloat16, device="cuda")
        C_other = torch.empty_like(C)
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.run(sd, bd, C)
            with pytest.raises(agmm.AgmmError) as ei:
                plan.run(sd, bd, C_other)
            assert ei.value.status == agmm.AGMM_ERR_UNSUPPORTED
        torch.cuda.synchronize()
        C.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        check_against_oracle(w, shards, B, C)
        del g
    finally:
        plan.close()


# ------------------------------------------- transposed copy of B (stored k x n)
@pytest.mark.parametrize("variant,dtype,settings", [
    ("fused", BF16, {"tile": 9}), ("fused", FP16, {"tile": 8}), ("fused", BF16, {"tile": 9, "splits": 2}),
    ("unfused", BF16, {"tile": 9}), ("staged", FP16, {"tile": 9, "pvalue": 1}),
    ("fused", BF16, {"tile": 1})])
@pytest.mark.parametrize("k", [384, 328])
def test_b_transposed_copy_bit_identical(variant, dtype, settings, k):
    """B stored k x n with the plan's transposed copy (b_transpose 1): the GEMM
    reads B^T as n x k.  Same tile and k order as reading B directly, so the
    output is bit-identical to b_transpose 0, and it matches the oracle (ragged
    m, n and tiles, whole and ragged last k-tiles (k = 328: the transpose's
    last row tile is partial too); also the 32x32 stage-ring tile)."""
    N, m_s, n = 3, 200, 392
    w, shards, B = make_case(N, m_s, k, n, dtype, False, seed=960 + len(variant))
    sd = [to_device(x, dtype) for x in shards]
    bd = to_device(B, dtype)
    outs = []
    for bt in (1, 0):
        plan = agmm.Plan(N, m_s, k, n, dtype, False, variant=variant, b_transpose=bt, **settings)
        try:
            assert plan.get("b_transposed") == bt
            outs.append(plan.run(sd, bd))
            torch.cuda.synchronize()
        finally:
            plan.close()
    check_against_oracle(w, shards, B, outs[0])
    assert np.array_equal(to_bits(outs[0]), to_bits(outs[1]))


def test_b_transposed_copy_graph_capture():
    """A plan that copies B transposed, captured into a HIP graph (the
    transpose and the GEMM are both in it) and replayed on new inputs: every
    replay matches the oracle and is bit-identical to an eager run."""
    N, m_s, k, n, dtype = 2, 256, 512, 264, BF16
    w, shards, B = make_case(N, m_s, k, n, dtype, False, seed=980)
    plan = agmm.Plan(N, m_s, k, n, dtype, False, variant="fused", b_transpose=1)
    try:
        assert plan.get("b_transposed") == 1
        sd = [to_device(x, dtype) for x in shards]
        bd = to_device(B, dtype)
        C = torch.empty((N * m_s, n), dtype=torch.bfloat16, device="cuda")
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.run(sd, bd, C)
        torch.cuda.synchronize()
        for rep in range(3):
            w2, sh2, B2 = make_case(N, m_s, k, n, dtype, False, seed=981 + rep)
            for d, h in zip(sd, sh2):
                d.copy_(to_device(h, dtype))
            bd.copy_(to_device(B2, dtype))
            C.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            check_against_oracle(w2, sh2, B2, C)
            C_eager = plan.run(sd, bd)
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(C), to_bits(C_eager))
        del g
    finally:
        plan.close()


def test_b_transposed_copy_strided_and_gathered_calls():
    """The transposed copy with a row-strided B (ldb > n, NaN in the gaps), the
    n x k-only 256x224 tile, and through agmm_run_gathered / agmm_run_gather_out."""
    N, m_s, k, n, dtype = 2, 300, 512, 456, BF16
    w, shards, B = make_case(N, m_s, k, n, dtype, False, seed=971)
    sd = [to_device(x, dtype) for x in shards]
    ldb = n + 24
    Bp = torch.full((k, ldb), float("nan"), dtype=torch.bfloat16, device="cuda")
    Bp[:, :n] = to_device(B, dtype)
    bview = Bp[:, :n]
    plan = agmm.Plan(N, m_s, k, n, dtype, False, variant="fused", b_transpose=1, ldb=ldb,
                     tile=agmm.TILES["256x224_m16"])
    try:
        assert plan.get("b_transposed") == 1 and plan.get("tile") == agmm.TILES["256x224_m16"]
        C = plan.run(sd, bview)
        torch.cuda.synchronize()
        check_against_oracle(w, shards, B, C)
        C2, G = plan.run_gather_out(sd, bview)
        C3 = plan.run_gathered(G, bview)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(G), np.concatenate(shards, axis=0))
        assert np.array_equal(to_bits(C2), to_bits(C))
        assert np.array_equal(to_bits(C3), to_bits(C))
    finally:
        plan.close()


def test_b_transposed_copy_automatic_choice():
    """Automatic: B stored k x n is copied transposed for large m only (never
    for B stored n x k, skinny plans or fp32), and a tile that reads B as
    n x k only is refused on B k x n without the copy."""
    big = agmm.Plan(8, 4096, 8192, 7168, BF16, False)
    small = agmm.Plan(4, 512, 4096, 1024, BF16, False)
    nk = agmm.Plan(8, 4096, 8192, 7168, BF16, True)
    try:
        assert big.get("b_transposed") == 1
        assert small.get("b_transposed") == 0 and nk.get("b_transposed") == 0
        with pytest.raises(agmm.AgmmError):
            small.set("tile", agmm.TILES["256x224_m16"])
        small.set("b_transpose", 1)
        small.set("tile", agmm.TILES["256x224_m16"])
        assert small.get("b_transposed") == 1
    finally:
        big.close()
        small.close()
        nk.close()


SPECIAL_BITS = {BF16: (0x7F80, 0xFF80, 0x7FC0), FP16: (0x7C00, 0xFC00, 0x7E00),
                FP32: (0x7F800000, 0xFF800000, 0x7FC00000)}   # +inf, -inf, NaN


@pytest.mark.parametrize("variant,dtype,rt,k,settings", [
    ("fused", BF16, False, 384, {}), ("fused", FP16, True, 384, {"splits": 3}),
    ("staged", BF16, True, 384, {"pvalue": 1}), ("unfused", FP16, False, 384, {}),
    ("skinny", BF16, True, 384, {}), ("skinny", FP16, True, 1024, {"splits": 4}),
    ("fused", BF16, False, 13, {}), ("fused", FP32, False, 200, {})])
def test_special_values_propagate(variant, dtype, rt, k, settings):
    """IEEE specials in A (+inf, -inf, both in one row, NaN) give the
    oracle's specials in C: an output is NaN, +inf or -inf exactly where
    the fp64 oracle's is, whatever the summation order; every other output
    is within the usual bound."""
    N, m_s, n = 3, 40, 136
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=3700 + k + dtype)
    pinf, ninf, nan = SPECIAL_BITS[dtype]
    shards = [s.copy() for s in shards]
    shards[0][1, 3] = pinf          # row 1: +-inf by the sign of B's row 3
    shards[0][5, 2] = ninf          # row 5: -+inf
    shards[1][7, 0] = pinf          # row m_s + 7: +inf and -inf: NaN where both terms meet
    shards[1][7, k - 1] = ninf
    shards[2][9, k // 2] = nan      # row 2 m_s + 9: all NaN
    sd = [to_device(x, dtype) for x in shards]
    C, _ = run_variant(w, sd, to_device(B, dtype), variant, **settings)
    ref = oracle.agmm_f64(shards, B, dtype, rt)
    got = oracle.decode(to_bits(C), dtype)
    for cls in (np.isnan, np.isposinf, np.isneginf):
        assert np.array_equal(cls(got), cls(ref)), f"{cls.__name__} positions differ"
    assert np.isnan(ref).any() and np.isposinf(ref).any() and np.isneginf(ref).any()
    fin = np.isfinite(ref)
    err = rel_err(got[fin], ref[fin])
    assert err <= BOUND[dtype], f"max rel err {err:.3e}"


@pytest.mark.parametrize("dtype,rt", [(BF16, False), (FP16, True), (FP32, False)])
def test_all_gather_matmul_one_call(dtype, rt):
    """The one-call form: the same bits as a plan's run, the plan created
    once and reused for the same problem, a new one for another shape."""
    w, shards, B = make_case(3, 40, 264, 136, dtype, rt, seed=3500 + dtype)
    sd = [to_device(x, dtype) for x in shards]
    bd = to_device(B, dtype)
    agmm.clear_plan_cache()
    try:
        C1 = agmm.all_gather_matmul(sd, bd, rhs_transpose=rt)
        C2 = agmm.all_gather_matmul(sd, bd, rhs_transpose=rt)
        torch.cuda.synchronize()
        assert len(agmm._PLAN_CACHE) == 1
        with agmm.Plan(3, 40, 264, 136, dtype, rt) as plan:
            C_ref = plan.run(sd, bd)
            torch.cuda.synchronize()
        assert np.array_equal(to_bits(C1), to_bits(C_ref)) and np.array_equal(to_bits(C2), to_bits(C_ref))
        check_against_oracle(w, shards, B, C1)
        agmm.all_gather_matmul(sd[:2], bd, rhs_transpose=rt)
        torch.cuda.synchronize()
        assert len(agmm._PLAN_CACHE) == 2
    finally:
        agmm.clear_plan_cache()
    assert len(agmm._PLAN_CACHE) == 0


def test_run_gathered_matches_fused():
    w, shards, B = make_case(2, 256, 512, 256, FP16, True, seed=82)
    sd = [to_device(s, FP16) for s in shards]
    bd = to_device(B, FP16)
    plan = agmm.Plan(2, 256, 512, 256, FP16, True, variant="fused", tile=1)
    try:
        G = plan.gather(sd)
        C1 = plan.run_gathered(G, bd)
        C2 = plan.run(sd, bd)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert np.array_equal(to_bits(C1), to_bits(C2))
    check_against_oracle(w, shards, B, C1)


@pytest.mark.parametrize("variant,dtype,rt,settings", [
    ("fused", BF16, False, {"tile": 6}), ("staged", FP16, True, {"pvalue": 1, "tile": 6}),
    ("unfused", BF16, True, {}), ("skinny", BF16, True, {}), ("fused", FP32, False, {}),
    ("fused", BF16, True, {"copy_engine": 1, "gather_out": 1}), ("fused", BF16, False, {"gather_out": 1}),
    ("fused", FP16, True, {"gather_out": 2}), ("skinny", BF16, True, {"gather_out": 2}),
    ("staged", BF16, False, {"pvalue": 1, "copy_engine": 1}),
    ("unfused", BF16, False, {"copy_engine": 1})])
def test_run_gather_out(variant, dtype, rt, settings):
    """C and the gathered operand from one call: the gathered buffer is the
    bit-exact concatenation, C is bit-identical to agmm_run's, and the
    gathered buffer feeds a second product against another B ("split n")."""
    m_s = 24 if variant == "skinny" else 200
    w, shards, B = make_case(3, m_s, 320, 136, dtype, rt, seed=470 + len(variant))
    _, _, B2 = make_case(3, m_s, 320, 136, dtype, rt, seed=471 + len(variant))
    sd = [to_device(x, dtype) for x in shards]
    plan = agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, dtype, rt, variant=variant,
                     **settings)
    try:
        assert plan.get("variant_used") == agmm.VARIANTS[variant]
        C, G = plan.run_gather_out(sd, to_device(B, dtype))
        C_ref = plan.run(sd, to_device(B, dtype))
        C2 = plan.run_gathered(G, to_device(B2, dtype))
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert np.array_equal(to_bits(G), np.concatenate(shards, axis=0))
    assert np.array_equal(to_bits(C), to_bits(C_ref))
    check_against_oracle(w, shards, B, C)
    check_against_oracle(w, shards, B2, C2)


@pytest.mark.parametrize("copy_engine", [0, 1])
@pytest.mark.parametrize("nbuf", [1, 2, 3])
def test_staged_copy_engines(copy_engine, nbuf):
    """The staged pipeline with its chunk copies on the gather kernel or the
    SDMA engines, ring slots reused (more chunks than slots), two calls in a
    row: the oracle's values, and the same bits whichever engine copied."""
    w, shards, B = make_case(3, 520, 256, 200, BF16, True, seed=480 + nbuf)
    sd = [to_device(x, BF16) for x in shards]
    bd = to_device(B, BF16)
    outs = []
    for ce in (0, copy_engine):
        plan = agmm.Plan(3, 520, 256, 200, BF16, True, variant="staged", pvalue=1, tile=6,
                         nbuf=nbuf, copy_engine=ce)
        try:
            assert plan.get("num_chunks") == 5 and plan.get("copy_engine") == ce
            for _ in range(2):
                C = plan.run(sd, bd)
            torch.cuda.synchronize()
            outs.append(to_bits(C))
        finally:
            plan.close()
    assert np.array_equal(outs[0], outs[1])
    check_against_oracle(w, shards, B, C)


@pytest.mark.parametrize("shape,want", [((8, 1024, 8192, 3584, FP16, True), 8),
                                        ((8, 4096, 8192, 7168, BF16, False), 4)])
def test_group_m_automatic(shape, want):
    """The automatic row-block group: the count whose tiles on one XCD touch
    the fewest A row blocks plus B column blocks (8 for 32 x 14 tiles of
    256 x 256, 4 on ties); an explicit setting wins."""
    plan = agmm.Plan(*shape, variant="fused")
    try:
        assert plan.get("group_m") == 0
        assert plan.get("group_m_used") == want
        plan.set("group_m", 2)
        assert plan.get("group_m_used") == 2
    finally:
        plan.close()


@pytest.mark.parametrize("local_shard", [0, 1, 3])
@pytest.mark.parametrize("settings", [{"pvalue": 1, "nbuf": 2, "tile": 6},
                                      {"pvalue": 2, "nbuf": 1, "tile": 1},
                                      {"pvalue": 1, "nbuf": 2, "tile": 6, "splits": 2},
                                      {"pvalue": 1, "nbuf": 3, "tile": 6, "gemm_streams": 1}])
def test_staged_local_first(local_shard, settings):
    """The staged variant with the local shard's rows computed first from
    its own buffer (local_first 1) against the same plan without (0): the
    same bits (same tile, same k order per element), and the oracle's
    values; C from agmm_run_gather_out too, with its gathered operand."""
    w, shards, B = make_case(4, 300, 256, 136, BF16, True, seed=2400 + local_shard)
    sd = [to_device(x, BF16) for x in shards]
    bd = to_device(B, BF16)
    outs = []
    for lf in (0, 1):
        plan = agmm.Plan(4, 300, 256, 136, BF16, True, variant="staged", local_shard=local_shard,
                         local_first=lf, **settings)
        try:
            assert plan.get("local_first") == lf
            C = plan.run(sd, bd)
            C2, G = plan.run_gather_out(sd, bd)
            torch.cuda.synchronize()
            assert np.array_equal(to_bits(C), to_bits(C2))
            assert np.array_equal(to_bits(G), np.concatenate(shards, axis=0))
            outs.append(to_bits(C))
        finally:
            plan.close()
    assert np.array_equal(outs[0], outs[1])
    check_against_oracle(w, shards, B, C)


def test_copy_engine_validated():
    plan = agmm.Plan(2, 64, 64, 64, BF16, True, variant="staged")
    try:
        for bad in (-1, 2):
            with pytest.raises(agmm.AgmmError):
                plan.set("copy_engine", bad)
        plan.set("copy_engine", 1)
        assert plan.get("copy_engine") == 1
    finally:
        plan.close()


def test_run_rejects_misaligned_pointer():
    w, shards, B = make_case(2, 8, 64, 64, BF16, False, seed=83)
    sd = [to_device(s, BF16) for s in shards]
    bd = to_device(B, BF16)
    C = torch.empty((16, 64), dtype=torch.bfloat16, device="cuda")
    plan = agmm.Plan(2, 8, 64, 64, BF16, False)
    try:
        with pytest.raises(agmm.AgmmError) as ei:
            agmm.agmm_run(plan.handle, [sd[0].data_ptr() + 2, sd[1].data_ptr()], bd.data_ptr(),
                          C.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert ei.value.status == agmm.AGMM_ERR_UNSUPPORTED
        with pytest.raises(agmm.AgmmError) as ei:
            agmm.agmm_run(plan.handle, [sd[0].data_ptr(), 0], bd.data_ptr(), C.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
        assert ei.value.status == agmm.AGMM_ERR_INVALID_ARG
    finally:
        plan.close()


def test_binding_rejects_misplaced_tensors():
    """The torch binding's host checks: a tensor on the CPU, of another
    dtype or shape, or a short shard list is refused with an exception before
    any pointer reaches the library (which would otherwise read host memory
    or past the pointer table on the GPU)."""
    w, shards, B = make_case(2, 8, 64, 64, BF16, True, seed=85)
    sd = [to_device(s, BF16) for s in shards]
    bd = to_device(B, BF16)
    C = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    plan = agmm.Plan(2, 8, 64, 64, BF16, True)
    try:
        with pytest.raises(ValueError, match="expected 2 shards"):
            plan.gather(sd[:1])
        with pytest.raises(ValueError, match="on the GPU"):
            plan.run([sd[0], sd[1].cpu()], bd)
        with pytest.raises(ValueError, match="on the GPU"):
            plan.run_gathered(torch.zeros((16, 64), dtype=torch.bfloat16), bd)
        with pytest.raises(TypeError, match="dtype"):
            plan.run(sd, bd.half())
        with pytest.raises(ValueError, match="shape"):
            plan.run(sd, bd[:, :32])
    finally:
        plan.close()
    # the plan-free entry point
    with pytest.raises(ValueError, match="on cuda"):
        agmm.run_noalloc(sd, bd, C.cpu(), True)
    with pytest.raises(TypeError, match="dtype"):
        agmm.run_noalloc(sd, bd, C.half(), True)
    with pytest.raises(ValueError, match="every shard"):
        agmm.run_noalloc([sd[0], sd[1][:4]], bd, C, True)
    with pytest.raises(ValueError, match="does not match k"):
        agmm.run_noalloc(sd, bd[:, :32].contiguous(), C, True)
    with pytest.raises(ValueError, match="on the GPU"):
        agmm.run_noalloc([s.cpu() for s in sd], bd.cpu(), C.cpu(), True)
    # the checks above changed nothing: a correct call still runs
    agmm.run_noalloc(sd, bd, C, True)
    torch.cuda.synchronize()
    check_against_oracle(w, shards, B, C)


def test_set_int_rejection_keeps_the_plan():
    """A rejected setting (the skinny tile on a plan whose B is
    stored k x n) leaves every setting as it was: the plan still runs with
    its previous tile and computes the oracle's values."""
    w, shards, B = make_case(2, 16, 64, 64, BF16, False, seed=84)
    plan = agmm.Plan(2, 16, 64, 64, BF16, False, variant="skinny")
    try:
        tile0, ws0 = plan.get("tile"), plan.workspace_bytes()
        with pytest.raises(agmm.AgmmError) as ei:
            plan.set("tile", agmm.TILE_SKINNY)
        assert ei.value.status == agmm.AGMM_ERR_UNSUPPORTED
        assert plan.get("tile") == tile0 and plan.get("usable") == 1
        assert plan.workspace_bytes() == ws0
        C = plan.run([to_device(x, BF16) for x in shards], to_device(B, BF16))
        torch.cuda.synchronize()
    finally:
        plan.close()
    check_against_oracle(w, shards, B, C)


def test_set_int_oom_restores_previous_layout(monkeypatch):
    """A reconfiguration whose workspace cannot be allocated (test hook: no
    allocation larger than the current workspace) fails with AGMM_ERR_OOM
    and leaves the plan with its previous settings and a workspace for them:
    runs stay correct."""
    w, shards, B = make_case(3, 200, 256, 136, BF16, True, seed=85)
    sd = [to_device(x, BF16) for x in shards]
    bd = to_device(B, BF16)
    plan = agmm.Plan(3, 200, 256, 136, BF16, True, variant="unfused")
    try:
        assert plan.get("splits") == 1
        # split-K adds [2][600][136] fp32 partial sums to the [600, 256] operand
        monkeypatch.setenv("AGMM_TEST_FAIL_ALLOC", str(plan.workspace_bytes()))
        with pytest.raises(agmm.AgmmError) as ei:
            plan.set("splits", 2)
        assert ei.value.status == agmm.AGMM_ERR_OOM
        monkeypatch.delenv("AGMM_TEST_FAIL_ALLOC")
        assert plan.get("usable") == 1
        assert plan.get("variant_used") == agmm.VARIANTS["unfused"] and plan.get("splits") == 1
        C = torch.full((w.m, w.n_local), float("nan"), dtype=torch.bfloat16, device="cuda")
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
    finally:
        plan.close()
    check_against_oracle(w, shards, B, C)


def test_set_int_oom_unrecoverable_plan_refuses_runs(monkeypatch):
    """When neither the new nor the previous workspace can be allocated the
    plan is marked unusable: every later call fails with the allocation's
    status and launches nothing (C keeps its NaN fill)."""
    w, shards, B = make_case(2, 300, 256, 128, BF16, False, seed=86)
    sd = [to_device(x, BF16) for x in shards]
    bd = to_device(B, BF16)
    plan = agmm.Plan(2, 300, 256, 128, BF16, False, variant="unfused")
    try:
        monkeypatch.setenv("AGMM_TEST_FAIL_ALLOC", "1")
        with pytest.raises(agmm.AgmmError) as ei:
            plan.set("splits", 2)          # a larger workspace: ring plus partials
        assert ei.value.status == agmm.AGMM_ERR_OOM
        monkeypatch.delenv("AGMM_TEST_FAIL_ALLOC")
        assert plan.get("usable") == 0
        C = torch.full((w.m, w.n_local), float("nan"), dtype=torch.bfloat16, device="cuda")
        for call in (lambda: plan.run(sd, bd, C), lambda: plan.run_gathered(torch.cat(sd), bd, C),
                     lambda: plan.run_gather_out(sd, bd, C), lambda: plan.set("splits", 1)):
            with pytest.raises(agmm.AgmmError) as ei:
                call()
            assert ei.value.status == agmm.AGMM_ERR_OOM
        torch.cuda.synchronize()
        assert torch.isnan(C.float()).all().item()
    finally:
        plan.close()


def test_autotune_under_allocation_limits(monkeypatch):
    """Autotune when workspace allocations fail (test hook).  With no
    allocation larger than the plan's current workspace, the candidates that
    need more are skipped and the plan keeps a correct configuration that
    fits.  With every allocation failing, a candidate that needs a larger
    workspace leaves the plan without one: autotune stops, reports
    AGMM_ERR_OOM, and the plan then refuses runs."""
    w, shards, B = make_case(3, 200, 512, 136, BF16, True, seed=87)
    sd = [to_device(x, BF16) for x in shards]
    bd = to_device(B, BF16)
    plan = agmm.Plan(3, 200, 512, 136, BF16, True, variant="unfused")
    try:
        limit = plan.workspace_bytes()
        monkeypatch.setenv("AGMM_TEST_FAIL_ALLOC", str(limit))
        C = torch.full((w.m, w.n_local), float("nan"), dtype=torch.bfloat16, device="cuda")
        plan.autotune(sd, bd, C, iters=1)
        monkeypatch.delenv("AGMM_TEST_FAIL_ALLOC")
        assert plan.get("usable") == 1 and plan.workspace_bytes() <= limit
        C2 = plan.run(sd, bd)
        torch.cuda.synchronize()
        check_against_oracle(w, shards, B, C)
        check_against_oracle(w, shards, B, C2)
    finally:
        plan.close()
    plan = agmm.Plan(3, 200, 512, 136, BF16, True, variant="unfused")
    try:
        monkeypatch.setenv("AGMM_TEST_FAIL_ALLOC", "1")
        with pytest.raises(agmm.AgmmError) as ei:
            plan.autotune(sd, bd, iters=1)
        assert ei.value.status == agmm.AGMM_ERR_OOM
        monkeypatch.delenv("AGMM_TEST_FAIL_ALLOC")
        assert plan.get("usable") == 0
        C = torch.full((w.m, w.n_local), float("nan"), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(agmm.AgmmError) as ei:
            plan.run(sd, bd, C)
        assert ei.value.status == agmm.AGMM_ERR_OOM
        torch.cuda.synchronize()
        assert torch.isnan(C.float()).all().item()
    finally:
        plan.close()


def _spin_cycles_per_ms():
    """Rate of torch's bounded spin kernel (torch.cuda._sleep) on this GPU.
    The kernel runs once untimed first: the first launch in a process also
    loads its code, and that host-side delay would land between the events."""
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    torch.cuda._sleep(4_000_000)
    e.record()
    torch.cuda.synchronize()
    return 4_000_000 / max(s.elapsed_time(e), 1e-3)


@pytest.mark.parametrize("variant,settings", [
    ("staged", {"pvalue": 1, "nbuf": 2, "tile": 6}),            # 4 chunks through 2 slots
    ("fused", {"tile": 1, "splits": 3}),                         # split-K partials
    ("skinny", {"tile": 7, "splits": 4}),
    ("skinny", {"tile": 10, "splits": 4})])                      # the skinny kernel's k ranges
def test_serial_calls_on_two_streams_are_ordered(variant, settings):
    """Call 1 on stream s1 (queued behind a ~150 ms spin kernel), then at once
    call 2 with other inputs on stream s2, no host synchronisation between
    them.  The plan orders call 2 after call 1 (it shares the ring slots or
    the split-K partials), so call 2 cannot have finished while s1 is still
    spinning, and both outputs match their own oracle."""
    m_s = 24 if variant == "skinny" else 400
    cases = [make_case(3, m_s, 512, 264, BF16, True, seed=2500 + i) for i in range(2)]
    dev = [([to_device(x, BF16) for x in sh], to_device(B, BF16)) for _, sh, B in cases]
    plan = agmm.Plan(3, m_s, 512, 264, BF16, True, variant=variant, **settings)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    Cs = [torch.full((3 * m_s, 264), float("nan"), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    try:
        if variant == "staged":
            assert plan.get("num_chunks") == 4 and plan.get("num_slots") == 2
        else:
            assert plan.get("splits") > 1
        cycles = int(150 * _spin_cycles_per_ms())
        torch.cuda.synchronize()
        done2 = torch.cuda.Event()
        with torch.cuda.stream(s1):
            torch.cuda._sleep(cycles)
            plan.run(dev[0][0], dev[0][1], Cs[0], stream=s1)
        with torch.cuda.stream(s2):
            plan.run(dev[1][0], dev[1][1], Cs[1], stream=s2)
            done2.record(s2)
        time.sleep(0.03)
        assert not done2.query(), "call 2 finished while call 1 was still queued behind the spin"
        torch.cuda.synchronize()
    finally:
        plan.close()
    for (w, sh, B), C in zip(cases, Cs):
        check_against_oracle(w, sh, B, C)


def test_concurrent_plans_from_host_threads():
    """Three host threads, each with its own plan (fused split-K, skinny k
    ranges, staged) and its own stream, call at the same time; every output
    is bit-identical to the same call made alone, and each thread's error
    status stays its own (a rejected call in one thread does not disturb
    the others)."""
    import threading
    specs = [((3, 100, 512, 264, BF16, True), {"variant": "fused", "splits": 3}),
             ((4, 16, 2048, 512, BF16, True), {"variant": "skinny"}),
             ((2, 300, 384, 136, FP16, False), {"variant": "staged", "pvalue": 1, "nbuf": 2})]
    cases = []
    for i, ((N, m_s, k, n, dtype, rt), settings) in enumerate(specs):
        w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=3900 + i)
        cases.append((w, [to_device(x, dtype) for x in shards], to_device(B, dtype), settings))
    refs = []
    for w, sd, bd, settings in cases:
        with agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose, **settings) as plan:
            refs.append(to_bits(plan.run(sd, bd)))
            torch.cuda.synchronize()
    errors, outs = [], [None] * len(cases)
    start = threading.Barrier(len(cases))

    def worker(i):
        try:
            w, sd, bd, settings = cases[i]
            stream = torch.cuda.Stream()
            with agmm.Plan(w.num_shards, w.m_per_shard, w.k, w.n_local, w.dtype, w.rhs_transpose,
                           **settings) as plan:
                C = torch.empty((w.m, w.n_local), dtype=torch_dtype(w.dtype), device="cuda")
                start.wait()
                for it in range(30):
                    plan.run(sd, bd, C, stream=stream)
                    if i == 0 and it == 10:
                        # rejected here, in this thread only (the C call alone:
                        # the binding's own follow-up calls would reset it)
                        st = agmm.load_library().agmm_plan_set_int(plan.handle, b"tile", 99)
                        assert st == agmm.AGMM_ERR_INVALID_ARG
                        time.sleep(0.01)   # the other threads' calls succeed meanwhile
                        assert agmm.agmm_last_status() == agmm.AGMM_ERR_INVALID_ARG
                        assert "tile" in agmm.agmm_last_error()
                stream.synchronize()
                outs[i] = to_bits(C)
        except Exception as e:   # reported on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    for i, (out, ref) in enumerate(zip(outs, refs)):
        assert out is not None and np.array_equal(out, ref), f"thread {i}: output differs"


def test_runs_allocate_nothing(monkeypatch):
    """Once the plans exist, every workspace allocation is made to fail
    (the test hook): runs on every path, the gather, the gathered-output
    and already-gathered entry points all still succeed and match the
    oracle, so none of them allocates."""
    specs = [((3, 100, 512, 264, BF16, False), {"variant": "fused"}),
             ((3, 100, 512, 264, FP16, True), {"variant": "staged", "pvalue": 1, "nbuf": 2}),
             ((3, 100, 512, 264, BF16, True), {"variant": "unfused"}),
             ((4, 16, 2048, 512, BF16, True), {"variant": "skinny"}),
             ((2, 50, 13, 20, BF16, False), {}),                        # padded copies
             ((2, 64, 200, 96, FP32, False), {"variant": "fused"})]
    made = []
    try:
        for i, ((N, m_s, k, n, dtype, rt), settings) in enumerate(specs):
            w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=4000 + i)
            plan = agmm.Plan(N, m_s, k, n, dtype, rt, **settings)
            made.append((w, shards, B, plan, [to_device(x, dtype) for x in shards], to_device(B, dtype)))
        monkeypatch.setenv("AGMM_TEST_FAIL_ALLOC", "1")
        for w, shards, B, plan, sd, bd in made:
            C = plan.run(sd, bd)
            C2, G = plan.run_gather_out(sd, bd)
            torch.cuda.synchronize()
            check_against_oracle(w, shards, B, C)
            assert np.array_equal(to_bits(C2), to_bits(C))
            assert np.array_equal(to_bits(G), oracle.gather(shards, w.dtype))
            C3 = plan.run_gathered(G, bd)
            G2 = plan.gather(sd)
            torch.cuda.synchronize()
            check_against_oracle(w, shards, B, C3)
            assert np.array_equal(to_bits(G2), to_bits(G))
        # the hook is live: a new plan that needs a workspace fails to get one
        with pytest.raises(agmm.AgmmError) as ei:
            agmm.Plan(2, 512, 256, 256, BF16, False, variant="unfused")
        assert ei.value.status == agmm.AGMM_ERR_OOM
    finally:
        monkeypatch.delenv("AGMM_TEST_FAIL_ALLOC", raising=False)
        for m in made:
            m[3].close()


def test_oom_hook_reports_status(monkeypatch):
    monkeypatch.setenv("AGMM_TEST_FAIL_ALLOC", "1")
    with pytest.raises(agmm.AgmmError) as ei:
        agmm.Plan(2, 512, 256, 256, BF16, False, variant="unfused")
    assert ei.value.status == agmm.AGMM_ERR_OOM


# -------------------------------- randomized sweep of layouts and copies of B
def _random_layout_case(seed):
    """A seeded random problem for the layout-related settings the sweep above
    leaves out: the transposed copy of B (b_transpose), row strides (lda,
    ldb) and padded shapes (k not a multiple of 8), across variants, tiles
    and k splits."""
    rng = np.random.default_rng(7000 + seed)
    dtype = [BF16, FP16, BF16, FP32][seed % 4]
    variant = ["fused", "staged", "unfused", "fused", "skinny", "auto"][seed % 6]
    rt = bool(rng.integers(0, 2)) and seed % 3 != 0
    N = int(rng.integers(1, 7))
    m_s = int(rng.integers(1, 32)) if variant == "skinny" else int(rng.integers(1, 170))
    k = int(rng.integers(1, 66)) * 8
    n = int(rng.integers(1, 300))
    if dtype != FP32 and not rt:
        n = max(8, n - n % 8)          # whole 16-byte B rows
    padded = dtype != FP32 and seed % 7 == 3
    if padded:
        k += int(rng.integers(1, 8))   # rows that are not 16-byte vectors
    settings = {}
    if dtype != FP32 and variant not in ("skinny", "auto"):
        bt = not rt and not padded and rng.random() < 0.8
        if bt:
            settings["b_transpose"] = 1    # first, so that n x k-only tiles are allowed
        tiles = [0, 1, 2, 5, 6, 8, 9] + ([3, 4, 7, 11] if (rt or bt) else [])
        settings["tile"] = int(rng.choice(tiles))
        settings["splits"] = int(rng.integers(0, 4))
    if variant == "staged":
        settings["pvalue"] = int(rng.integers(1, 4))
        settings["nbuf"] = int(rng.integers(1, 4))
    e = 4 if dtype == FP32 else 2
    lda = ldb = 0
    if not padded and rng.integers(0, 2) == 0:
        # at least the row length, and a whole number of 16-byte vectors
        vec = 16 // e
        lda = k + vec * int(rng.integers(1, 4))
        row_b = k if rt else n
        ldb = row_b + (-row_b) % vec + vec * int(rng.integers(1, 4))
    return variant, dtype, rt, N, m_s, k, n, settings, lda, ldb


@pytest.mark.parametrize("seed", list(range(24)))
def test_randomized_layouts_against_oracle(seed):
    variant, dtype, rt, N, m_s, k, n, settings, lda, ldb = _random_layout_case(seed)
    w, shards, B = make_case(N, m_s, k, n, dtype, rt, seed=8000 + seed)
    plan = agmm.Plan(N, m_s, k, n, dtype, rt, variant=variant, **settings)
    try:
        if lda:
            plan.set("lda", lda)
        if ldb:
            plan.set("ldb", ldb)
        sd = [to_device(x, dtype) for x in shards]
        bd = to_device(B, dtype)
        if lda:
            sd = [strided(t, lda) for t in sd]
        if ldb:
            bd = strided(bd, ldb)
        C = torch.full((w.m, n), float("nan"), dtype=torch_dtype(dtype), device="cuda")
        plan.run(sd, bd, C)
        torch.cuda.synchronize()
        desc = (f"{variant} dtype {dtype} rt {int(rt)} {N}x{m_s}x{k}->{n} {settings} lda {lda} ldb {ldb} "
                f"-> tile {plan.get('tile')} splits {plan.get('splits')} variant_used "
                f"{plan.get('variant_used')} b_transposed {plan.get('b_transposed')}")
    finally:
        plan.close()
    assert not torch.isnan(C.float()).any().item(), desc
    try:
        check_against_oracle(w, shards, B, C)
    except AssertionError as err:
        raise AssertionError(f"{desc}: {err}") from None
