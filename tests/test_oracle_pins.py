"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: exact
rational brute force, numpy/torch conversions and matmul, hand-worked values,
and invariants the definition implies.  `test_pins_catch_planted_mistakes`
rebuilds the oracle with deliberate mistakes (on the CPU) and requires every
one of them to be caught by the pins below.
"""
import json
import os
import shutil
import subprocess
import tempfile
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import Oracle
from all_gather_gemm_agmm_amd import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "handworked.json")
DTYPES = [I.DTYPE_BF16, I.DTYPE_FP16, I.DTYPE_FP32]


# ----------------------------------------------------------------- helpers
def dyadic_bits(shape, seed, dtype):
    """Values j/4 with |j| <= 12: exact in bf16/fp16/fp32, exact sums in fp64."""
    rng = np.random.default_rng(seed)
    x = (rng.integers(-12, 13, size=shape) / 4.0).astype(np.float32)
    return I.to_storage_bits(x, dtype)


def exact_value(bits, dtype):
    return [[Fraction(float(v)) for v in row] for row in I.bits_to_f64(bits, dtype)]


def brute_force(shards, B, dtype, rhs_transpose):
    """Exact rational C, straight from the definition (pure Python loops)."""
    A = []
    for s in shards:
        A.extend(exact_value(s, dtype))
    Bv = exact_value(B, dtype)
    k = len(A[0])
    n = len(Bv) if rhs_transpose else len(Bv[0])
    C = []
    for row in A:
        out = []
        for j in range(n):
            acc = Fraction(0)
            for t in range(k):
                b = Bv[j][t] if rhs_transpose else Bv[t][j]
                acc += row[t] * b
            out.append(acc)
        C.append(out)
    return C


# The pin checks, parameterised by the oracle build so that planted mistakes
# can be run through the very same checks.
def pin_brute_force(orc, dtype, rhs_transpose, N, m_s, k, n, seed):
    shards = [dyadic_bits((m_s, k), seed + r, dtype) for r in range(N)]
    B = dyadic_bits((n, k) if rhs_transpose else (k, n), seed + 99, dtype)
    got = orc.agmm_f64(shards, B, dtype, rhs_transpose)
    want = brute_force(shards, B, dtype, rhs_transpose)
    assert got.shape == (N * m_s, n)
    for i in range(N * m_s):
        for j in range(n):
            assert Fraction(float(got[i, j])) == want[i][j], (i, j)


def pin_numpy_matmul(orc, dtype, rhs_transpose, seed=3):
    N, m_s, k, n = 3, 7, 40, 9
    shards = [I.to_storage_bits(I.draw((m_s, k), seed + r, "normal", k), dtype) for r in range(N)]
    B = I.to_storage_bits(I.draw((n, k) if rhs_transpose else (k, n), seed + 50, "normal", k), dtype)
    A = np.concatenate([I.bits_to_f64(s, dtype) for s in shards], axis=0)
    Bf = I.bits_to_f64(B, dtype)
    ref = A @ (Bf.T if rhs_transpose else Bf)
    got = orc.agmm_f64(shards, B, dtype, rhs_transpose)
    scale = np.abs(A) @ np.abs(Bf.T if rhs_transpose else Bf)
    assert np.all(np.abs(got - ref) <= 1e-12 * scale + 1e-300)


def pin_row_blocks(orc, dtype, rhs_transpose, seed=11):
    N, m_s, k, n = 4, 5, 24, 6
    shards = [I.to_storage_bits(I.draw((m_s, k), seed + r, "normal", k), dtype) for r in range(N)]
    B = I.to_storage_bits(I.draw((n, k) if rhs_transpose else (k, n), seed + 50, "normal", k), dtype)
    full = orc.agmm_f64(shards, B, dtype, rhs_transpose)
    for r in range(N):
        one = orc.agmm_f64([shards[r]], B, dtype, rhs_transpose)
        assert np.array_equal(full[r * m_s:(r + 1) * m_s], one)


def pin_permutation(orc, dtype, rhs_transpose, seed=21):
    N, m_s, k, n = 5, 3, 16, 4
    shards = [I.to_storage_bits(I.draw((m_s, k), seed + r, "normal", k), dtype) for r in range(N)]
    B = I.to_storage_bits(I.draw((n, k) if rhs_transpose else (k, n), seed + 50, "normal", k), dtype)
    base = orc.agmm_f64(shards, B, dtype, rhs_transpose)
    perm = [3, 0, 4, 1, 2]
    got = orc.agmm_f64([shards[p] for p in perm], B, dtype, rhs_transpose)
    for pos, p in enumerate(perm):
        assert np.array_equal(got[pos * m_s:(pos + 1) * m_s], base[p * m_s:(p + 1) * m_s])


def identity_bits(k, n, dtype, rhs_transpose):
    eye = np.eye(k, n, dtype=np.float32)           # [I 0] or [I; 0]
    if rhs_transpose:
        eye = np.ascontiguousarray(eye.T)
    return I.to_storage_bits(eye, dtype)


def pin_identity(orc, dtype, rhs_transpose, seed=31):
    N, m_s = 3, 4
    for k, n in [(8, 8), (8, 5), (5, 8)]:
        shards = [I.to_storage_bits(I.draw((m_s, k), seed + r, "normal", k), dtype) for r in range(N)]
        got = orc.agmm_f64(shards, identity_bits(k, n, dtype, rhs_transpose), dtype, rhs_transpose)
        A = np.concatenate([I.bits_to_f64(s, dtype) for s in shards], axis=0)
        want = np.zeros((N * m_s, n))
        c = min(k, n)
        want[:, :c] = A[:, :c]
        assert np.array_equal(got, want), (k, n)


def pin_linearity(orc, dtype, rhs_transpose, seed=41):
    N, m_s, k, n = 2, 3, 12, 5
    shards = [I.small_int_bits((m_s, k), seed + r, dtype) for r in range(N)]
    shape = (n, k) if rhs_transpose else (k, n)
    rng = np.random.default_rng(seed + 7)
    B1 = rng.integers(-4, 5, size=shape).astype(np.float32)
    B2 = rng.integers(-4, 5, size=shape).astype(np.float32)
    alpha, beta = 2.0, -3.0
    C1 = orc.agmm_f64(shards, I.to_storage_bits(B1, dtype), dtype, rhs_transpose)
    C2 = orc.agmm_f64(shards, I.to_storage_bits(B2, dtype), dtype, rhs_transpose)
    C12 = orc.agmm_f64(shards, I.to_storage_bits(alpha * B1 + beta * B2, dtype), dtype, rhs_transpose)
    assert np.array_equal(C12, alpha * C1 + beta * C2)


def pin_transpose(orc, dtype, seed=51):
    N, m_s, k, n = 3, 4, 20, 7
    shards = [I.to_storage_bits(I.draw((m_s, k), seed + r, "normal", k), dtype) for r in range(N)]
    B = I.to_storage_bits(I.draw((k, n), seed + 50, "normal", k), dtype)
    Bt = np.ascontiguousarray(B.T)
    assert np.array_equal(orc.agmm_f64(shards, B, dtype, False),
                          orc.agmm_f64(shards, Bt, dtype, True))


def pin_golden(orc):
    with open(GOLDEN) as f:
        data = json.load(f)
    for case in data["cases"]:
        dtype = I.DTYPE_BY_NAME[case["dtype"]]
        if "shards_bits" in case:
            wbits = np.uint32 if dtype == I.DTYPE_FP32 else np.uint16
            shards = [np.array(s, dtype=wbits) for s in case["shards_bits"]]
            B = np.array(case["B_bits"], dtype=wbits)
        else:
            shards = [I.to_storage_bits(np.array(s, dtype=np.float32), dtype) for s in case["shards"]]
            B = I.to_storage_bits(np.array(case["B"], dtype=np.float32), dtype)
        got = orc.agmm_f64(shards, B, dtype, case["rhs_transpose"])
        assert np.array_equal(got, np.array(case["C"], dtype=np.float64)), case["name"]


def pin_gather(orc, dtype, seed=61):
    N, m_s, k = 4, 6, 10
    shards = [I.to_storage_bits(I.draw((m_s, k), seed + r, "normal", k), dtype) for r in range(N)]
    got = orc.gather(shards, dtype)
    assert np.array_equal(got, np.concatenate(shards, axis=0))


def pin_sampled_rows(orc, dtype, rhs_transpose, seed=71):
    N, m_s, k, n = 3, 5, 16, 6
    shards = [I.to_storage_bits(I.draw((m_s, k), seed + r, "normal", k), dtype) for r in range(N)]
    B = I.to_storage_bits(I.draw((n, k) if rhs_transpose else (k, n), seed + 50, "normal", k), dtype)
    full = orc.agmm_f64(shards, B, dtype, rhs_transpose)
    rows = [14, 0, 7, 5, 5]
    assert np.array_equal(orc.agmm_f64(shards, B, dtype, rhs_transpose, rows=rows), full[rows])


def run_all_pins(orc):
    """Every pin; raises AssertionError on the first one that fails."""
    pin_golden(orc)
    for dtype in DTYPES:
        pin_gather(orc, dtype)
        pin_transpose(orc, dtype)
        for rt in (False, True):
            pin_brute_force(orc, dtype, rt, 2, 3, 7, 4, seed=5)
            pin_numpy_matmul(orc, dtype, rt)
            pin_row_blocks(orc, dtype, rt)
            pin_permutation(orc, dtype, rt)
            pin_identity(orc, dtype, rt)
            pin_linearity(orc, dtype, rt)
            pin_sampled_rows(orc, dtype, rt)


# ------------------------------------------------------------------- tests
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rhs_transpose", [False, True])
@pytest.mark.parametrize("N,m_s,k,n", [(1, 1, 1, 1), (2, 2, 3, 4), (3, 5, 7, 9),
                                       (2, 1, 16, 1), (3, 2, 16, 4)])
def test_brute_force_exact(dtype, rhs_transpose, N, m_s, k, n):
    pin_brute_force(oracle.default(), dtype, rhs_transpose, N, m_s, k, n,
                    seed=100 * N + 10 * m_s + k)


def test_brute_force_general_floats():
    """Random fp32 values: oracle within the fp64 summation bound of the exact sum."""
    dtype = I.DTYPE_FP32
    N, m_s, k, n = 2, 3, 17, 4
    shards = [I.to_storage_bits(I.draw((m_s, k), 900 + r, "uniform", k), dtype) for r in range(N)]
    B = I.to_storage_bits(I.draw((k, n), 950, "uniform", k), dtype)
    got = oracle.agmm_f64(shards, B, dtype, False)
    exact = brute_force(shards, B, dtype, False)
    A = np.concatenate([I.bits_to_f64(s, dtype) for s in shards])
    bound = k * 2.0 ** -53 * (np.abs(A) @ np.abs(I.bits_to_f64(B, dtype)))
    for i in range(N * m_s):
        for j in range(n):
            err = abs(Fraction(float(got[i, j])) - exact[i][j])
            assert err <= Fraction(float(bound[i, j])), (i, j)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rhs_transpose", [False, True])
def test_numpy_matmul(dtype, rhs_transpose):
    pin_numpy_matmul(oracle.default(), dtype, rhs_transpose)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rhs_transpose", [False, True])
def test_row_blocks_match_single_shard(dtype, rhs_transpose):
    pin_row_blocks(oracle.default(), dtype, rhs_transpose)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rhs_transpose", [False, True])
def test_shard_permutation(dtype, rhs_transpose):
    pin_permutation(oracle.default(), dtype, rhs_transpose)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rhs_transpose", [False, True])
def test_identity_returns_gathered(dtype, rhs_transpose):
    pin_identity(oracle.default(), dtype, rhs_transpose)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rhs_transpose", [False, True])
def test_linearity_in_B(dtype, rhs_transpose):
    pin_linearity(oracle.default(), dtype, rhs_transpose)


@pytest.mark.parametrize("dtype", DTYPES)
def test_transpose_consistency(dtype):
    pin_transpose(oracle.default(), dtype)


@pytest.mark.parametrize("dtype", DTYPES)
def test_gather_is_concatenation(dtype):
    pin_gather(oracle.default(), dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rhs_transpose", [False, True])
def test_sampled_rows(dtype, rhs_transpose):
    pin_sampled_rows(oracle.default(), dtype, rhs_transpose)


def test_handworked_golden():
    pin_golden(oracle.default())


SPECIALS = {I.DTYPE_BF16: (0x7F80, 0xFF80, 0x7FC0), I.DTYPE_FP16: (0x7C00, 0xFC00, 0x7E00),
            I.DTYPE_FP32: (0x7F800000, 0xFF800000, 0x7FC00000)}   # +inf, -inf, NaN


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("rhs_transpose", [False, True])
def test_special_values_follow_ieee(dtype, rhs_transpose):
    """Infinities and NaN in A: the oracle's outputs equal a plain Python
    float loop over the same decoded values (IEEE double arithmetic), NaN
    where that loop gives NaN; finite values are small integers, so every
    finite output is exact.  B holds zeros too, so inf * 0 = NaN is met."""
    N, m_s, k, n = 2, 3, 4, 5
    shards = [I.small_int_bits((m_s, k), 40 + r, dtype, lo=-3, hi=3) for r in range(N)]
    bshape = (n, k) if rhs_transpose else (k, n)
    B = I.small_int_bits(bshape, 47, dtype, lo=-2, hi=2)
    pinf, ninf, nan = SPECIALS[dtype]
    shards[0][0, 1] = pinf
    shards[0][2, 0] = ninf
    shards[1][1, 0] = pinf
    shards[1][1, 3] = ninf
    shards[1][2, 2] = nan
    got = oracle.agmm_f64(shards, B, dtype, rhs_transpose)
    A = np.concatenate([I.bits_to_f64(x, dtype) for x in shards])
    Bv = I.bits_to_f64(B, dtype)
    for i in range(N * m_s):
        for j in range(n):
            acc = 0.0
            for t in range(k):
                b = float(Bv[j, t] if rhs_transpose else Bv[t, j])
                acc += float(A[i, t]) * b
            if acc != acc:
                assert np.isnan(got[i, j]), (i, j)
            else:
                assert got[i, j] == acc, (i, j, got[i, j], acc)
    assert np.isnan(got).any() and np.isinf(got).any()


def test_decode_fp16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, I.DTYPE_FP16)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_decode_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(bits, I.DTYPE_BF16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_decode_fp32_random_patterns():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    got = oracle.decode(bits, I.DTYPE_FP32)
    want = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_storage_rounding_matches_torch():
    """The input generator's bf16 rounding equals torch's (round to nearest even)."""
    x = I.draw((4096,), 5, "normal", 1) * np.float32(1000.0)
    x = np.concatenate([x, np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39,
                                     np.float32(np.inf)], dtype=np.float32)])
    mine = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_fp16_subnormals_kept_in_inputs():
    """A workload-4 shaped draw holds fp16 subnormals and they survive storage."""
    x = I.draw((64, 8192), 4000, "normal", 8192)
    bits = I.to_storage_bits(x, I.DTYPE_FP16)
    v = oracle.decode(bits, I.DTYPE_FP16)
    sub = (np.abs(v) > 0) & (np.abs(v) < 2.0 ** -14)
    assert sub.mean() > 1e-3


def test_rejects_bad_arguments():
    s = [np.zeros((2, 3), np.uint16)]
    with pytest.raises(ValueError):
        oracle.agmm_f64(s, np.zeros((4, 2), np.uint16), I.DTYPE_BF16, False)
    with pytest.raises(ValueError):
        oracle.agmm_f64(s, np.zeros((3, 2), np.uint16), I.DTYPE_BF16, False, rows=[2])
    with pytest.raises(TypeError):
        oracle.agmm_f64(s, np.zeros((3, 2), np.float32), I.DTYPE_BF16, False)


# Plausible mistakes, each planted by a textual edit of a copy of the oracle
# source.  Every one must make at least one pin fail.
MUTANTS = {
    "transposed_B_operand": ("Bd[t * n + j] = rhs_transpose ? tmp[j * k + t] : tmp[t * n + j];",
                             "Bd[t * n + j] = rhs_transpose ? tmp[t * n + j] : tmp[j * k + t];"),
    "wrong_sign": ("out[j] += a * brow[j];", "out[j] -= a * brow[j];"),
    "dropped_last_term": ("for (int64_t t = 0; t < k; ++t) {", "for (int64_t t = 0; t + 1 < k; ++t) {"),
    "dropped_first_term": ("for (int64_t t = 0; t < k; ++t) {", "for (int64_t t = (k > 1); t < k; ++t) {"),
    "wrong_shard_index": ("int64_t r = row / m_s;       /* owning shard */",
                          "int64_t r = row % num_shards; /* owning shard */"),
    "wrong_local_row": ("int64_t i = row - r * m_s;   /* row inside the shard */",
                        "int64_t i = row % (m_s > 1 ? m_s - 1 : 1);"),
    "fp16_subnormal_flush": ("v = ldexp((double)frac, -24);", "v = 0.0 * frac;"),
    "fp16_bias_off_by_one": ("v = ldexp((double)(frac + 1024), e - 25);",
                             "v = ldexp((double)(frac + 1024), e - 24);"),
    "bf16_wrong_shift": ("uint32_t u = ((uint32_t)h) << 16;", "uint32_t u = ((uint32_t)h) << 15;"),
    "gather_rows_reversed": ("memcpy(out + ((size_t)r * m_s + i) * row_bytes,",
                             "memcpy(out + ((size_t)r * m_s + (m_s - 1 - i)) * row_bytes,"),
    "output_row_off_by_one": ("double *out = C + (size_t)q * (size_t)n;",
                              "double *out = C + (size_t)((q + 1) % nout) * (size_t)n;"),
}


def test_pins_pass_on_real_oracle():
    run_all_pins(oracle.default())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name):
    src_path = os.path.join(os.path.dirname(oracle.__file__), "agmm_oracle.c")
    with open(src_path) as f:
        src = f.read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new, 1)
    tmp = tempfile.mkdtemp(prefix="oracle_mutant_")
    try:
        c_path = os.path.join(tmp, "m.c")
        so_path = os.path.join(tmp, f"lib_{name}.so")
        with open(c_path, "w") as f:
            f.write(src)
        subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                        "-ffp-contract=off", "-o", so_path, c_path, "-lm"], check=True)
        mutant = Oracle(so_path)
        with pytest.raises(AssertionError):
            run_all_pins(mutant)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
