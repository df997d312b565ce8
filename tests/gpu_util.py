"""Helpers shared by the GPU tests: moving raw storage bits to and from torch
device tensors and the parity metric.  No arithmetic of the method here."""
import numpy as np
import torch

from all_gather_gemm_agmm_amd import inputs as I

BOUND = {I.DTYPE_BF16: 2e-2, I.DTYPE_FP16: 2e-2, I.DTYPE_FP32: 1e-5}


def gpu_available() -> bool:
    return torch.cuda.is_available()


def to_device(bits: np.ndarray, dtype: int, device="cuda") -> torch.Tensor:
    if dtype == I.DTYPE_BF16:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    elif dtype == I.DTYPE_FP16:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int32)).view(torch.float32)
    return t.to(device)


def to_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.contiguous().view(torch.int32).cpu().numpy().view(np.uint32)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / (|ref| + 1e-3) over all elements."""
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + 1e-3)))


def torch_dtype(dtype: int):
    return {I.DTYPE_BF16: torch.bfloat16, I.DTYPE_FP16: torch.float16,
            I.DTYPE_FP32: torch.float32}[dtype]


def sample_rows(num_shards: int, m_s: int, extra=(), per_shard=4, seed=0):
    """Rows for sampled parity: first/last rows of every shard, shard-half
    boundaries, a few random rows per shard, plus `extra`."""
    rng = np.random.default_rng(seed)
    rows = set()
    for r in range(num_shards):
        base = r * m_s
        for i in (0, m_s - 1, m_s // 2, max(m_s // 2 - 1, 0)):
            rows.add(base + i)
        for i in rng.integers(0, m_s, size=per_shard):
            rows.add(base + int(i))
    for x in extra:
        if 0 <= x < num_shards * m_s:
            rows.add(int(x))
    return sorted(rows)


def block_rows(m: int, block=256, seed=0):
    """Two rows of every `block`-row block of C, one in each half (the two
    128-row wave halves of a 256-row tile), at offsets that vary from block
    to block (so different rows of the 16-row MFMA blocks are hit)."""
    rng = np.random.default_rng(seed)
    rows = []
    for b0 in range(0, m, block):
        half = block // 2
        for lo in (b0, b0 + half):
            hi = min(lo + half, m)
            if lo < hi:
                rows.append(int(rng.integers(lo, hi)))
    return rows
