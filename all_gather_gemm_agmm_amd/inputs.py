"""Seeded synthetic inputs for the all-gather matmul workloads.

This module is shared by the HIP path's tests/benchmark and by the CPU
oracle's tests.  It holds no arithmetic of the method itself: it only draws
random numbers, rounds them to the storage dtype and hands out raw bit
arrays, so both sides see exactly the same bits.

The five workloads are the per-GPU shares of the all-gather matmul described
by the tpu-inference page ("all_gather_matmul.py", `all_gather_matmul`
docstring: all-gather(x, axis=0) @ y, with x row-sharded over the ring and y
column-sharded so each device owns n_local columns) and by the
Triton-distributed-Ascend tutorial "AllGather-GEMM" (`run_test_distributed`).
No public dataset exists for this op; these seeded tensors stand in for
activations (A shards) and weights (B).

Value recipe:
  * fp32 workload: U[-1, 1] drawn in float32.
  * bf16/fp16 workloads: N(0, sigma) with sigma = 1/sqrt(k), drawn in
    float32, then rounded to the storage type with round-to-nearest-even,
    subnormals kept.
  * seeds: shard r uses 1000*w + r, B uses 1000*w + 999 (w = workload id).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Tuple

import numpy as np

DTYPE_BF16 = 0
DTYPE_FP16 = 1
DTYPE_FP32 = 2

DTYPE_NAMES = {DTYPE_BF16: "bf16", DTYPE_FP16: "fp16", DTYPE_FP32: "fp32"}
DTYPE_BYTES = {DTYPE_BF16: 2, DTYPE_FP16: 2, DTYPE_FP32: 4}
DTYPE_BY_NAME = {v: k for k, v in DTYPE_NAMES.items()}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One all-gather matmul problem as a single GPU sees it."""
    wid: int                # workload id (seed base)
    name: str
    num_shards: int
    m_per_shard: int
    k: int
    n_local: int
    dtype: int
    rhs_transpose: bool
    dist: str               # "uniform" or "normal"
    pvalue: Optional[int] = None
    nbuf: Optional[int] = None
    variant: str = "auto"

    @property
    def m(self) -> int:
        return self.num_shards * self.m_per_shard

    @property
    def elem_bytes(self) -> int:
        return DTYPE_BYTES[self.dtype]

    def flops(self) -> int:
        """2*m*k*n: the work the tpu-inference page's cost estimate assigns."""
        return 2 * self.m * self.k * self.n_local

    def algorithmic_bytes(self) -> int:
        """itemsize*(m*k + k*n + m*n): read A and B once, write C once."""
        e = self.elem_bytes
        return e * (self.m * self.k + self.k * self.n_local + self.m * self.n_local)

    def gather_bytes(self) -> int:
        return self.elem_bytes * self.m * self.k

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "num_shards": self.num_shards,
            "m_per_shard": self.m_per_shard,
            "k": self.k,
            "n_local": self.n_local,
            "dtype": DTYPE_NAMES[self.dtype],
            "rhs_transpose": self.rhs_transpose,
            "values": ("U[-1,1]" if self.dist == "uniform"
                       else "N(0, sigma=1/sqrt(k))"),
        }


WORKLOADS = {
    1: Workload(1, "agmm_s2_m64_k256_n128_fp32", 2, 64, 256, 128, DTYPE_FP32,
                False, "uniform"),
    2: Workload(2, "agmm_s4_m512_k4096_n1024_bf16", 4, 512, 4096, 1024,
                DTYPE_BF16, False, "normal"),
    3: Workload(3, "agmm_s8_m16_k4096_n1792_bf16_rhsT", 8, 16, 4096, 1792,
                DTYPE_BF16, True, "normal"),
    4: Workload(4, "agmm_s8_m1024_k8192_n3584_fp16_rhsT", 8, 1024, 8192, 3584,
                DTYPE_FP16, True, "normal", pvalue=2, nbuf=2,
                variant="staged"),
    5: Workload(5, "agmm_s8_m4096_k8192_n7168_bf16", 8, 4096, 8192, 7168,
                DTYPE_BF16, False, "normal", variant="fused"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + bias) >> 16).astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def to_storage_bits(x: np.ndarray, dtype: int) -> np.ndarray:
    """float32 array -> raw storage bits (uint16 for bf16/fp16, uint32 for fp32)."""
    if dtype == DTYPE_BF16:
        return f32_to_bf16_bits(x)
    if dtype == DTYPE_FP16:
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == DTYPE_FP32:
        return np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    raise ValueError(f"unknown dtype {dtype}")


def bits_to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Widen storage bits to float64 with numpy's own conversions (test helper)."""
    if dtype == DTYPE_BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == DTYPE_FP16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == DTYPE_FP32:
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype}")


def draw(shape: Tuple[int, ...], seed: int, dist: str, k: int) -> np.ndarray:
    """Seeded float32 draw: U[-1,1] or N(0, 1/sqrt(k))."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    if dist == "normal":
        x = rng.standard_normal(size=shape, dtype=np.float32)
        x *= np.float32(1.0 / math.sqrt(k))
        return x
    raise ValueError(f"unknown distribution {dist}")


def b_shape(w: Workload) -> Tuple[int, int]:
    """B as stored: [n_local, k] when rhs_transpose, else [k, n_local]."""
    return (w.n_local, w.k) if w.rhs_transpose else (w.k, w.n_local)


def make_inputs(w: Workload, seed_base: Optional[int] = None
                ) -> Tuple[List[np.ndarray], np.ndarray]:
    """Return (shards, B) as raw storage-bit arrays for workload `w`.

    shards[r] has shape [m_per_shard, k]; B has the stored shape b_shape(w).
    """
    base = 1000 * (w.wid if seed_base is None else seed_base)
    shards = [to_storage_bits(draw((w.m_per_shard, w.k), base + r, w.dist, w.k), w.dtype)
              for r in range(w.num_shards)]
    B = to_storage_bits(draw(b_shape(w), base + 999, w.dist, w.k), w.dtype)
    return shards, B


def custom_workload(num_shards: int, m_per_shard: int, k: int, n_local: int,
                    dtype: int, rhs_transpose: bool, dist: str = "normal",
                    wid: int = 0, name: str = "custom") -> Workload:
    return Workload(wid, name, num_shards, m_per_shard, k, n_local, dtype,
                    rhs_transpose, dist)


def small_int_bits(shape: Tuple[int, ...], seed: int, dtype: int, lo: int = -4,
                   hi: int = 4) -> np.ndarray:
    """Small integers (exactly representable in every dtype) as storage bits."""
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return to_storage_bits(x, dtype)
