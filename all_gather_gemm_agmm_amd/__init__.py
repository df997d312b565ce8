"""Python binding of libagmm (all-gather fused matmul for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libagmm.so.  There is no CPU or PyTorch fallback; if the library is
missing or fails to load, every entry point raises.

The functions below carry the names of the C ABI in include/agmm.h and take
plain integers (device addresses, sizes, stream handles).  `Plan` is a small
convenience wrapper that takes torch tensors on the GPU and the current torch
stream.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libagmm.so")

AGMM_BF16, AGMM_FP16, AGMM_FP32 = 0, 1, 2
AGMM_OK, AGMM_ERR_INVALID_ARG, AGMM_ERR_UNSUPPORTED, AGMM_ERR_OOM, AGMM_ERR_HIP = 0, 1, 2, 3, 4
(AGMM_VARIANT_AUTO, AGMM_VARIANT_FUSED, AGMM_VARIANT_STAGED, AGMM_VARIANT_UNFUSED,
 AGMM_VARIANT_SKINNY) = 0, 1, 2, 3, 4
VARIANTS = {"auto": 0, "fused": 1, "staged": 2, "unfused": 3, "skinny": 4}
VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}

# Values of the plan key "tile" (include/agmm.h lists what each one is).
TILES = {"256x256": 0, "128x128": 1, "256x128": 2, "128x64": 3, "128x64_s8": 4,
         "256x256_ring": 5, "128x128_ring": 6, "128x64_ring": 7, "256x256_m16": 8,
         "128x128_m16": 9, "skinny": 10, "256x224_m16": 11}
NUM_TILES = len(TILES)
TILE_SKINNY = TILES["skinny"]
TILES_NEED_BT = (TILES["128x64"], TILES["128x64_s8"], TILES["128x64_ring"], TILE_SKINNY,
                 TILES["256x224_m16"])

# (name, restype, argtypes) of every symbol include/agmm.h declares.
_vp, _i64, _ci, _cc = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_char_p
EXPORTS = [
    ("agmm_plan_validate", _ci, [_ci, _i64, _i64, _i64, _ci, _ci]),
    ("agmm_plan_create", _vp, [_ci, _i64, _i64, _i64, _ci, _ci]),
    ("agmm_run", _ci, [_vp, ctypes.POINTER(_vp), _vp, _vp, _vp]),
    ("agmm_gather", _ci, [_vp, ctypes.POINTER(_vp), _vp, _vp]),
    ("agmm_run_gathered", _ci, [_vp, _vp, _vp, _vp, _vp]),
    ("agmm_run_gather_out", _ci, [_vp, ctypes.POINTER(_vp), _vp, _vp, _vp, _vp]),
    ("agmm_plan_autotune", _ci, [_vp, ctypes.POINTER(_vp), _vp, _vp, _vp, _ci,
                                 ctypes.POINTER(ctypes.c_double)]),
    ("agmm_plan_set_int", _ci, [_vp, _cc, _i64]),
    ("agmm_plan_get_int", _ci, [_vp, _cc, ctypes.POINTER(_i64)]),
    ("agmm_plan_workspace_bytes", ctypes.c_size_t, [_vp]),
    ("agmm_plan_slot_ptr", _vp, [_vp, _ci]),
    ("agmm_plan_tile_order", _ci, [_vp, _ci, ctypes.POINTER(ctypes.c_int32), _ci]),
    ("agmm_plan_timing_begin", _ci, [_vp]),
    ("agmm_plan_timing_read", _ci, [_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_i64)]),
    ("agmm_plan_timing_end", _ci, [_vp]),
    ("agmm_plan_destroy", None, [_vp]),
    ("agmm_run_noalloc", _ci, [_ci, _i64, _i64, _i64, _ci, _ci, ctypes.POINTER(_vp), _vp, _vp, _vp]),
    ("agmm_last_status", _ci, []),
    ("agmm_last_error", _cc, []),
    ("agmm_version", _cc, []),
]

_lib = None


class AgmmError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"agmm error {status}: {message}")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libagmm.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m all_gather_gemm_agmm_amd._build`; "
            "the all-gather matmul has no CPU fallback")
    lib = ctypes.CDLL(path)
    for name, res, args in EXPORTS:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int) -> int:
    if status != AGMM_OK:
        lib = load_library()
        raise AgmmError(status, lib.agmm_last_error().decode())
    return status


def _ptr_table(ptrs: Sequence[int]):
    return (ctypes.c_void_p * len(ptrs))(*[ctypes.c_void_p(int(p)) for p in ptrs])


# ---------------------------------------------------------------- raw C ABI
def agmm_plan_validate(num_shards, m_per_shard, k, n_local, dtype, rhs_transpose) -> int:
    return load_library().agmm_plan_validate(num_shards, m_per_shard, k, n_local, dtype,
                                             int(bool(rhs_transpose)))


def agmm_plan_create(num_shards, m_per_shard, k, n_local, dtype, rhs_transpose) -> int:
    lib = load_library()
    h = lib.agmm_plan_create(num_shards, m_per_shard, k, n_local, dtype, int(bool(rhs_transpose)))
    if not h:
        raise AgmmError(lib.agmm_last_status(), lib.agmm_last_error().decode())
    return h


def agmm_run(plan, shard_ptrs: Sequence[int], B: int, C: int, stream: int) -> int:
    return _check(load_library().agmm_run(plan, _ptr_table(shard_ptrs), B, C, stream))


def agmm_plan_autotune(plan, shard_ptrs: Sequence[int], B: int, C: int, stream: int,
                       iters: int = 3) -> float:
    best = ctypes.c_double(0.0)
    _check(load_library().agmm_plan_autotune(plan, _ptr_table(shard_ptrs), B, C, stream, iters,
                                             ctypes.byref(best)))
    return best.value


def agmm_gather(plan, shard_ptrs: Sequence[int], gathered: int, stream: int) -> int:
    return _check(load_library().agmm_gather(plan, _ptr_table(shard_ptrs), gathered, stream))


def agmm_run_gathered(plan, gathered: int, B: int, C: int, stream: int) -> int:
    return _check(load_library().agmm_run_gathered(plan, gathered, B, C, stream))


def agmm_run_gather_out(plan, shard_ptrs: Sequence[int], B: int, C: int, gathered: int,
                        stream: int) -> int:
    return _check(load_library().agmm_run_gather_out(plan, _ptr_table(shard_ptrs), B, C, gathered,
                                                     stream))


def agmm_plan_set_int(plan, key: str, value: int) -> int:
    return _check(load_library().agmm_plan_set_int(plan, key.encode(), int(value)))


def agmm_plan_get_int(plan, key: str) -> int:
    v = ctypes.c_int64(0)
    _check(load_library().agmm_plan_get_int(plan, key.encode(), ctypes.byref(v)))
    return int(v.value)


def agmm_plan_workspace_bytes(plan) -> int:
    return int(load_library().agmm_plan_workspace_bytes(plan))


def agmm_plan_slot_ptr(plan, slot: int) -> int:
    return int(load_library().agmm_plan_slot_ptr(plan, slot) or 0)


def agmm_plan_tile_order(plan, chunk: int = 0):
    # Chunk 0 is never smaller than a later (clamped) chunk.
    cap = max(agmm_plan_get_int(plan, "num_row_blocks"), 1)
    buf = (ctypes.c_int32 * cap)()
    got = load_library().agmm_plan_tile_order(plan, chunk, buf, cap)
    if got < 0:
        raise AgmmError(agmm_last_status(), agmm_last_error())
    return [int(buf[i]) for i in range(got)]


def agmm_plan_timing_begin(plan) -> int:
    return _check(load_library().agmm_plan_timing_begin(plan))


def agmm_plan_timing_read(plan):
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(load_library().agmm_plan_timing_read(plan, ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def agmm_plan_timing_end(plan) -> int:
    return _check(load_library().agmm_plan_timing_end(plan))


def agmm_plan_destroy(plan) -> None:
    if plan:
        load_library().agmm_plan_destroy(plan)


NOALLOC_SCRATCH_BYTES = 32 << 20


def agmm_run_noalloc(num_shards, m_per_shard, k, n_local, dtype, rhs_transpose,
                     shard_ptrs: Sequence[int], B: int, C: int, stream: int) -> int:
    return _check(load_library().agmm_run_noalloc(num_shards, m_per_shard, k, n_local, dtype,
                                                  int(bool(rhs_transpose)), _ptr_table(shard_ptrs),
                                                  B, C, stream))


def run_noalloc(shards, B, C, rhs_transpose: bool, stream=None):
    """agmm_run_noalloc on torch tensors: dense row-major shards [m_s, k], B
    [k, n] (or [n, k] with rhs_transpose) and a caller-provided C [m, n]."""
    import torch
    if len(shards) == 0:
        raise ValueError("agmm_run_noalloc needs at least one shard")
    tensors = list(shards) + [B, C]
    if not all(isinstance(t, torch.Tensor) for t in tensors):
        raise TypeError("shards, B and C must be torch tensors")
    dtype = {torch.bfloat16: AGMM_BF16, torch.float16: AGMM_FP16,
             torch.float32: AGMM_FP32}.get(B.dtype)
    if dtype is None:
        raise TypeError(f"unsupported dtype {B.dtype}")
    device = B.device
    if device.type != "cuda":
        raise ValueError("B must be on the GPU")
    for t in tensors:
        if t.device != device:
            raise ValueError(f"every tensor must be on {device} (found one on {t.device})")
        if t.dtype != B.dtype:
            raise TypeError(f"every tensor must have dtype {B.dtype} (found {t.dtype})")
        if t.dim() != 2 or not t.is_contiguous():
            raise ValueError("agmm_run_noalloc takes dense row-major 2-D tensors")
    m_s, k = shards[0].shape
    if any(tuple(t.shape) != (m_s, k) for t in shards):
        raise ValueError(f"every shard must have shape {(m_s, k)}")
    n = B.shape[0] if rhs_transpose else B.shape[1]
    if (B.shape[1] if rhs_transpose else B.shape[0]) != k:
        raise ValueError(f"B has shape {tuple(B.shape)}, which does not match k = {k}")
    if tuple(C.shape) != (len(shards) * m_s, n):
        raise ValueError(f"C has shape {tuple(C.shape)}, expected {(len(shards) * m_s, n)}")
    agmm_run_noalloc(len(shards), m_s, k, n, dtype, rhs_transpose, [s.data_ptr() for s in shards],
                     B.data_ptr(), C.data_ptr(), _stream_handle(stream, device.index))
    return C


def agmm_last_status() -> int:
    return int(load_library().agmm_last_status())


def agmm_last_error() -> str:
    return load_library().agmm_last_error().decode()


def agmm_version() -> str:
    return load_library().agmm_version().decode()


# ------------------------------------------------------- torch convenience
def _torch_dtype(dtype: int):
    import torch
    return {AGMM_BF16: torch.bfloat16, AGMM_FP16: torch.float16, AGMM_FP32: torch.float32}[dtype]


def _stream_handle(stream, device_index=None) -> int:
    """The raw hipStream_t of `stream`, or of the current stream of the given
    (else the current) device."""
    import torch
    if stream is None:
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:   # the pointer alone, without a Stream object
            return int(raw(torch.cuda.current_device() if device_index is None else device_index))
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


class Plan:
    """A plan bound to torch tensors.  All checks here are host-side shape,
    dtype and device checks; the computation is the library's."""

    def __init__(self, num_shards: int, m_per_shard: int, k: int, n_local: int, dtype: int,
                 rhs_transpose: bool, **settings):
        self.num_shards, self.m_per_shard, self.k, self.n_local = num_shards, m_per_shard, k, n_local
        self.dtype, self.rhs_transpose = dtype, bool(rhs_transpose)
        self.handle = agmm_plan_create(num_shards, m_per_shard, k, n_local, dtype, rhs_transpose)
        import torch
        self.device = torch.cuda.current_device()   # the device the library created the plan on
        self._tdt = _torch_dtype(dtype)
        self._ptrs = (ctypes.c_void_p * num_shards)()   # shard pointer table, reused per call
        self._read_strides()
        for key, val in settings.items():
            if val is not None:
                self.set(key, VARIANTS[val] if key == "variant" and isinstance(val, str) else val)

    def _read_strides(self):
        # row strides in use, kept here so that per-call checks need no
        # call into the library
        self._ld = {k: agmm_plan_get_int(self.handle, k) for k in ("lda", "ldb", "ldc")}

    @property
    def m(self) -> int:
        return self.num_shards * self.m_per_shard

    def set(self, key: str, value: int) -> None:
        try:
            agmm_plan_set_int(self.handle, key, value)
        finally:
            self._read_strides()

    def get(self, key: str) -> int:
        return agmm_plan_get_int(self.handle, key)

    def _check_tensor(self, t, shape, name, ld_key=None, index=None):
        """Shape / dtype / device checks.  With `ld_key` ("lda", "ldb", "ldc")
        the tensor may be a row-strided view whose row stride is the plan's
        setting for that key; otherwise it must be dense row-major."""
        ld = self._ld[ld_key] if ld_key else shape[1]
        try:   # the common case in a few attribute reads
            st = t.stride()
            if (t.dtype is self._tdt and t.is_cuda and t.get_device() == self.device and
                    t.shape == shape and st[1] == 1 and (shape[0] <= 1 or st[0] == ld)):
                return
        except (AttributeError, TypeError, IndexError):
            pass
        if index is not None:
            name = f"{name}[{index}]"
        import torch
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on the GPU")
        if t.get_device() != self.device:
            raise ValueError(f"{name} is on {t.device}; the plan was created on cuda:{self.device}")
        if t.dtype != _torch_dtype(self.dtype):
            raise TypeError(f"{name} has dtype {t.dtype}, plan expects {_torch_dtype(self.dtype)}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.stride(1) != 1 or (shape[0] > 1 and t.stride(0) != ld):
            raise ValueError(f"{name} must be row-major with rows {ld} elements apart "
                             f"(stride {tuple(t.stride())})")

    def _new_c(self, device):
        """A C buffer with the plan's row stride (a view when ldc > n_local)."""
        import torch
        ldc = self._ld["ldc"]
        return torch.empty((self.m, ldc), dtype=_torch_dtype(self.dtype), device=device)[:, :self.n_local]

    def b_shape(self):
        return (self.n_local, self.k) if self.rhs_transpose else (self.k, self.n_local)

    def run(self, shards, B, C=None, stream=None):
        if len(shards) != self.num_shards:
            raise ValueError(f"expected {self.num_shards} shards, got {len(shards)}")
        shape, ptrs = (self.m_per_shard, self.k), self._ptrs
        for r, s in enumerate(shards):
            self._check_tensor(s, shape, "shards", "lda", r)
            ptrs[r] = s.data_ptr()
        self._check_tensor(B, self.b_shape(), "B", "ldb")
        if C is None:
            C = self._new_c(B.device)
        self._check_tensor(C, (self.m, self.n_local), "C", "ldc")
        _check(load_library().agmm_run(self.handle, ptrs, B.data_ptr(), C.data_ptr(),
                                       _stream_handle(stream, B.device.index)))
        return C

    def run_gather_out(self, shards, B, C=None, gathered=None, stream=None):
        """C = concat(shards) @ B and the gathered operand; returns (C, gathered)."""
        import torch
        if len(shards) != self.num_shards:
            raise ValueError(f"expected {self.num_shards} shards, got {len(shards)}")
        for r, s in enumerate(shards):
            self._check_tensor(s, (self.m_per_shard, self.k), "shards", "lda", r)
        self._check_tensor(B, self.b_shape(), "B", "ldb")
        if C is None:
            C = self._new_c(B.device)
        if gathered is None:
            gathered = torch.empty((self.m, self.k), dtype=_torch_dtype(self.dtype), device=B.device)
        self._check_tensor(C, (self.m, self.n_local), "C", "ldc")
        self._check_tensor(gathered, (self.m, self.k), "gathered")
        agmm_run_gather_out(self.handle, [s.data_ptr() for s in shards], B.data_ptr(), C.data_ptr(),
                            gathered.data_ptr(), _stream_handle(stream, B.device.index))
        return C, gathered

    def autotune(self, shards, B, C=None, iters=3, stream=None) -> float:
        """Time candidate settings on these buffers, keep the fastest; returns
        its mean ms per run (C is overwritten with the product)."""
        if len(shards) != self.num_shards:
            raise ValueError(f"expected {self.num_shards} shards, got {len(shards)}")
        for r, s in enumerate(shards):
            self._check_tensor(s, (self.m_per_shard, self.k), "shards", "lda", r)
        self._check_tensor(B, self.b_shape(), "B", "ldb")
        if C is None:
            C = self._new_c(B.device)
        self._check_tensor(C, (self.m, self.n_local), "C", "ldc")
        return agmm_plan_autotune(self.handle, [s.data_ptr() for s in shards], B.data_ptr(),
                                  C.data_ptr(), _stream_handle(stream, B.device.index), iters)

    def gather(self, shards, out=None, stream=None):
        import torch
        if len(shards) != self.num_shards:
            raise ValueError(f"expected {self.num_shards} shards, got {len(shards)}")
        for r, s in enumerate(shards):
            self._check_tensor(s, (self.m_per_shard, self.k), "shards", "lda", r)
        if out is None:
            out = torch.empty((self.m, self.k), dtype=_torch_dtype(self.dtype), device=shards[0].device)
        self._check_tensor(out, (self.m, self.k), "gathered")
        agmm_gather(self.handle, [s.data_ptr() for s in shards], out.data_ptr(),
                    _stream_handle(stream, out.device.index))
        return out

    def run_gathered(self, gathered, B, C=None, stream=None):
        import torch
        self._check_tensor(gathered, (self.m, self.k), "gathered")
        self._check_tensor(B, self.b_shape(), "B", "ldb")
        if C is None:
            C = self._new_c(B.device)
        self._check_tensor(C, (self.m, self.n_local), "C", "ldc")
        agmm_run_gathered(self.handle, gathered.data_ptr(), B.data_ptr(), C.data_ptr(),
                          _stream_handle(stream, B.device.index))
        return C

    def tile_order(self, chunk: int = 0):
        return agmm_plan_tile_order(self.handle, chunk)

    def workspace_bytes(self) -> int:
        return agmm_plan_workspace_bytes(self.handle)

    def close(self) -> None:
        if getattr(self, "handle", None):
            agmm_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


# ------------------------------------------------ one call, cached plans
_PLAN_CACHE: dict = {}
_PLAN_CACHE_LOCK = None


def all_gather_matmul(shards, B, rhs_transpose: bool = False, C=None, stream=None):
    """C = concat_r(shards[r]) @ B, or @ B^T with rhs_transpose (B stored
    [n_local, k]): the tpu-inference page's `all_gather_matmul` on one GPU,
    with the shards as separate tensors.  The first call for a problem
    shape, dtype and device creates a plan with the automatic settings and
    keeps it (its workspace stays allocated until clear_plan_cache()); later
    calls reuse it.  Returns C [num_shards * m_per_shard, n_local]."""
    import threading
    global _PLAN_CACHE_LOCK
    if _PLAN_CACHE_LOCK is None:
        _PLAN_CACHE_LOCK = threading.Lock()
    if len(shards) == 0:
        raise ValueError("all_gather_matmul needs at least one shard")
    m_s, k = shards[0].shape
    n = B.shape[0] if rhs_transpose else B.shape[1]
    dtype = {"torch.bfloat16": AGMM_BF16, "torch.float16": AGMM_FP16,
             "torch.float32": AGMM_FP32}.get(str(B.dtype))
    if dtype is None:
        raise ValueError(f"unsupported dtype {B.dtype}")
    if B.device.type != "cuda":
        raise ValueError("B must be on the GPU")
    import torch
    key = (len(shards), int(m_s), int(k), int(n), dtype, bool(rhs_transpose), B.device.index)
    with _PLAN_CACHE_LOCK:
        plan = _PLAN_CACHE.get(key)
        if plan is None:
            with torch.cuda.device(B.device):
                plan = Plan(len(shards), int(m_s), int(k), int(n), dtype, bool(rhs_transpose))
            _PLAN_CACHE[key] = plan
    return plan.run(shards, B, C, stream=stream)


def clear_plan_cache() -> None:
    """Destroy the plans all_gather_matmul keeps (after the work queued on
    them has finished: destroying a plan waits for it)."""
    if _PLAN_CACHE_LOCK is None:
        return
    with _PLAN_CACHE_LOCK:
        plans = list(_PLAN_CACHE.values())
        _PLAN_CACHE.clear()
    for p in plans:
        p.close()
