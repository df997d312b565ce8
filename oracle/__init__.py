"""CPU oracle for the all-gather matmul — TEST INFRASTRUCTURE ONLY.

Only `tests/`, `__graft_entry__.smoke()` and the CPU-baseline leg of
`bench.py` may import this package.  The HIP library never calls it, and it
imports nothing from the HIP package: both sides only receive the same raw
input bits from the seeded generators.

The arithmetic lives in `agmm_oracle.c` (plain C, double precision, OpenMP
over output rows).  This module is a thin ctypes wrapper around it that takes
numpy arrays of raw storage bits.

Definition followed (tpu-inference "all_gather_matmul.py", `all_gather_matmul`
docstring; Triton-distributed-Ascend "AllGather-GEMM", golden
`torch_allgather_gemm`):

    C[r*m_s + i, j] = sum_t A_r[i, t] * (B[t, j]  or, with rhs_transpose, B[j, t])

Parity pins: see tests/test_oracle_pins.py (brute force in exact rationals,
numpy float64 matmul, row-block / permutation / identity / linearity /
transpose invariants, decoder checks).  No function here is unpinned.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

BF16, FP16, FP32 = 0, 1, 2


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _check_bits(a: np.ndarray, dtype: int) -> np.ndarray:
    want = np.uint32 if dtype == FP32 else np.uint16
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        raise TypeError(f"expected raw {np.dtype(want).name} bits for dtype {dtype}, got {a.dtype}")
    return a


class Oracle:
    """ctypes view of one build of the oracle library (the default build, or
    a deliberately broken copy that the pin tests use to show the pins bite)."""

    def __init__(self, lib_path: str = _LIB_PATH):
        if lib_path == _LIB_PATH and not os.path.exists(lib_path):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(lib_path)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.agmm_oracle_decode.argtypes = [ci, vp, i64, vp]
        lib.agmm_oracle_decode.restype = ci
        lib.agmm_oracle_gather.argtypes = [ci, i64, i64, ci, ctypes.POINTER(vp), vp]
        lib.agmm_oracle_gather.restype = ci
        lib.agmm_oracle_f64.argtypes = [ci, i64, i64, i64, ci, ci, ctypes.POINTER(vp), vp,
                                        ctypes.POINTER(i64), i64, vp]
        lib.agmm_oracle_f64.restype = ci
        lib.agmm_oracle_num_threads.argtypes = []
        lib.agmm_oracle_num_threads.restype = ci
        lib.agmm_oracle_set_threads.argtypes = [ci]
        lib.agmm_oracle_set_threads.restype = None
        self.lib = lib
        self.path = lib_path

    def decode(self, bits: np.ndarray, dtype: int) -> np.ndarray:
        """Storage bits -> float64, decoded by the oracle's own C routines."""
        bits = _check_bits(bits, dtype)
        out = np.empty(bits.shape, dtype=np.float64)
        rc = self.lib.agmm_oracle_decode(dtype, _ptr(bits), bits.size, _ptr(out))
        if rc != 0:
            raise ValueError(f"agmm_oracle_decode failed ({rc})")
        return out

    def gather(self, shards: Sequence[np.ndarray], dtype: int) -> np.ndarray:
        """All-gathered A: rows of shard 0, then shard 1, ... (bit copy)."""
        shards = [_check_bits(s, dtype) for s in shards]
        m_s, k = shards[0].shape
        for s in shards:
            if s.shape != (m_s, k):
                raise ValueError("all shards must have the same shape")
        out = np.empty((len(shards) * m_s, k), dtype=shards[0].dtype)
        table = (ctypes.c_void_p * len(shards))(*[s.ctypes.data for s in shards])
        rc = self.lib.agmm_oracle_gather(len(shards), m_s, k, dtype, table, _ptr(out))
        if rc != 0:
            raise ValueError(f"agmm_oracle_gather failed ({rc})")
        return out

    def agmm_f64(self, shards: Sequence[np.ndarray], B: np.ndarray, dtype: int,
                 rhs_transpose: bool, rows: Optional[Sequence[int]] = None) -> np.ndarray:
        """C = concat(shards) @ B (or @ B^T), accumulated and returned in float64.

        `rows` selects global output rows (shard r, local row i -> r*m_s + i);
        None computes all of them.
        """
        shards = [_check_bits(s, dtype) for s in shards]
        B = _check_bits(B, dtype)
        m_s, k = shards[0].shape
        for s in shards:
            if s.shape != (m_s, k):
                raise ValueError("all shards must have the same shape")
        if rhs_transpose:
            n, kb = B.shape
        else:
            kb, n = B.shape
        if kb != k:
            raise ValueError(f"contraction mismatch: shards have k={k}, B has {kb}")
        table = (ctypes.c_void_p * len(shards))(*[s.ctypes.data for s in shards])
        if rows is None:
            nout = len(shards) * m_s
            rows_arr = None
            rows_p = None
        else:
            rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
            nout = rows_arr.size
            rows_p = rows_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        out = np.empty((nout, n), dtype=np.float64)
        rc = self.lib.agmm_oracle_f64(len(shards), m_s, k, n, dtype, int(bool(rhs_transpose)),
                                      table, _ptr(B), rows_p,
                                      nout if rows is not None else 0, _ptr(out))
        if rc != 0:
            raise ValueError(f"agmm_oracle_f64 failed ({rc})")
        return out

    def num_threads(self) -> int:
        return int(self.lib.agmm_oracle_num_threads())

    def set_threads(self, n: int) -> None:
        """Threads of later calls (timing on one core; results are the same)."""
        self.lib.agmm_oracle_set_threads(int(n))


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def decode(bits: np.ndarray, dtype: int) -> np.ndarray:
    return default().decode(bits, dtype)


def gather(shards: Sequence[np.ndarray], dtype: int) -> np.ndarray:
    return default().gather(shards, dtype)


def agmm_f64(shards: Sequence[np.ndarray], B: np.ndarray, dtype: int,
             rhs_transpose: bool, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    return default().agmm_f64(shards, B, dtype, rhs_transpose, rows)


def num_threads() -> int:
    return default().num_threads()


def set_threads(n: int) -> None:
    default().set_threads(n)
