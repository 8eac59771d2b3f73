"""Python binding of libabsa, AB-Attention sampled block-sparse attention for MI355X.

Argument marshalling only: every step runs in the HIP kernels of
sampled_block_sparse_amd/_lib/libabsa.so, whose C interface is
include/absa.h. There is no CPU fallback: if the library is not built, the
first call raises.

The functions carry the C names:
  absa_plan_create(q, k, budget_blocks, seed, ...) -> Plan
  absa_plan_from_scores(scores, N, d, budget_blocks, seed, sampling=...) -> Plan
  absa_plan_import(rowptr, idx, logw, p, B, H, N, d) -> Plan
  absa_plan_scores(plan) -> device address of the retained scores, or 0
  absa_sparse_attention(plan, q, k, v, out=None) -> out
  absa_sparse_attention_noalloc(plan, q, k, v, out) -> out
  absa_dense_attention(q, k, v, out=None) -> out
Tensors are torch CUDA (HIP) tensors, contiguous [B, H, N, d], bfloat16 or
float32; work is queued on torch's current stream unless a stream is given.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "AbsaError", "Plan", "absa_plan_create", "absa_plan_from_scores", "absa_plan_import",
    "absa_plan_scores", "absa_sparse_attention", "absa_sparse_attention_noalloc",
    "absa_dense_attention", "absa_status_string", "absa_last_error",
    "get_lib", "LIB_PATH", "ABSA_OK", "ABSA_ERR_INVALID_ARG", "ABSA_ERR_UNSUPPORTED",
    "ABSA_ERR_OUT_OF_MEMORY", "ABSA_ERR_DEVICE", "ABSA_ERR_PLAN_MISMATCH",
    "INTER_MEAN_KEYS", "INTER_CENTROIDS", "INTER_WEIGHTS", "INTER_SCORES",
    "SAMPLING_POISSON", "SAMPLING_SYSTEMATIC",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libabsa.so")

ABSA_OK, ABSA_ERR_INVALID_ARG, ABSA_ERR_UNSUPPORTED = 0, 1, 2
ABSA_ERR_OUT_OF_MEMORY, ABSA_ERR_DEVICE, ABSA_ERR_PLAN_MISMATCH = 3, 4, 5
ABSA_BF16, ABSA_F32 = 0, 1
INTER_MEAN_KEYS, INTER_CENTROIDS, INTER_WEIGHTS, INTER_SCORES = 0, 1, 2, 3

_i64, _u64, _i32, _vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_int32, ctypes.c_void_p


class _Params(ctypes.Structure):
    _fields_ = [("query_block", _i32), ("kv_block", _i32), ("n_clusters", _i32),
                ("kmeans_iters", _i32), ("budget_blocks", _i64), ("seed", _u64),
                ("keep_intermediates", _i32), ("sampling", _i32), ("fused", _i32)]


# absa_sampling
SAMPLING_POISSON = 0
SAMPLING_SYSTEMATIC = 1
_SAMPLING = {"poisson": SAMPLING_POISSON, "systematic": SAMPLING_SYSTEMATIC}


def _sampling_code(sampling) -> int:
    if isinstance(sampling, str):
        if sampling not in _SAMPLING:
            raise ValueError(f"sampling must be one of {sorted(_SAMPLING)}")
        return _SAMPLING[sampling]
    return int(sampling)


class AbsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def get_lib():
    """Load libabsa.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sampled_block_sparse_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "absa_plan_params_init": (_i32, [ctypes.POINTER(_Params)]),
        "absa_plan_create": (_i32, [_vp, _vp, _i32, _i64, _i64, _i64, _i64,
                                    ctypes.POINTER(_Params), _vp, ctypes.POINTER(_vp)]),
        "absa_plan_from_scores": (_i32, [_vp, _i64, _i64, _i64, _i64, _i64, _u64, _i32, _vp,
                                         ctypes.POINTER(_vp)]),
        "absa_plan_import": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp,
                                    ctypes.POINTER(_vp)]),
        "absa_plan_info": (_i32, [_vp, _vp, _vp, _vp, _vp]),
        "absa_plan_export": (_i32, [_vp, _vp, _vp, _vp, _vp]),
        "absa_plan_export_intermediate": (_i32, [_vp, _i32, _i64, _i64, _vp]),
        "absa_plan_scores": (_i32, [_vp, ctypes.POINTER(_vp)]),
        "absa_sparse_attention": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64,
                                         _i64, _vp]),
        "absa_sparse_attention_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64,
                                                 _i64, _i64, _vp]),
        "absa_dense_attention": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _i64, _i64, _vp]),
        "absa_plan_destroy": (None, [_vp]),
        "absa_release_cached_memory": (_i32, []),
        "absa_status_string": (ctypes.c_char_p, [_i32]),
        "absa_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return get_lib().absa_status_string(status).decode()
    except Exception:
        return f"status {status}"


def absa_status_string(status: int) -> str:
    return get_lib().absa_status_string(status).decode()


def absa_last_error() -> str:
    return get_lib().absa_last_error().decode()


def _check(status: int):
    if status != ABSA_OK:
        raise AbsaError(status, absa_last_error())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ABSA_BF16
    if t.dtype == torch.float32:
        return ABSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _vp(t.data_ptr())


def _stream(stream):
    if stream is None:
        return _vp(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return _vp(stream.cuda_stream)
    return _vp(int(stream))


def _host(a: np.ndarray, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(_vp)


def _shape4(q: torch.Tensor):
    if q.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    return tuple(int(x) for x in q.shape)


class Plan:
    """A library-owned sampling plan (opaque handle)."""

    def __init__(self, handle: int):
        self._h = _vp(handle)

    @property
    def handle(self):
        if not self._h.value:
            raise ValueError("plan was destroyed")
        return self._h

    def info(self):
        shape = (ctypes.c_int64 * 4)()
        rows, M, nnz = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(get_lib().absa_plan_info(self.handle, ctypes.cast(shape, _vp),
                                        ctypes.cast(ctypes.pointer(rows), _vp),
                                        ctypes.cast(ctypes.pointer(M), _vp),
                                        ctypes.cast(ctypes.pointer(nnz), _vp)))
        return dict(shape=tuple(shape), rows=rows.value, M=M.value, nnz=nnz.value)

    def export(self):
        inf = self.info()
        rowptr = np.empty(inf["rows"] + 1, np.int64)
        idx = np.empty(inf["nnz"], np.int32)
        logw = np.empty(inf["nnz"], np.float32)
        p = np.empty(inf["nnz"], np.float64)
        _check(get_lib().absa_plan_export(self.handle, rowptr.ctypes.data_as(_vp),
                                          idx.ctypes.data_as(_vp), logw.ctypes.data_as(_vp),
                                          p.ctypes.data_as(_vp)))
        return dict(rowptr=rowptr, idx=idx, logw=logw, p=p)

    def export_intermediate(self, which: int, offset: int = 0, count: int | None = None):
        if count is None:
            inf = self.info()
            B, H, N, d = inf["shape"]
            QB = (N + 127) // 128
            total = {INTER_MEAN_KEYS: B * H * inf["M"] * d, INTER_SCORES: inf["rows"] * inf["M"]}
            if which not in total:
                raise ValueError("give count for centroids and weights")
            count = total[which] - offset
            del QB
        out = np.empty(count, np.float32)
        _check(get_lib().absa_plan_export_intermediate(self.handle, which, offset, count,
                                                       out.ctypes.data_as(_vp)))
        return out

    def destroy(self):
        if self._h.value:
            get_lib().absa_plan_destroy(self._h)
            self._h = _vp(0)

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def absa_plan_create(q: torch.Tensor, k: torch.Tensor, budget_blocks: int, seed: int,
                     n_clusters: int = 8, kmeans_iters: int = 4,
                     keep_intermediates: bool = False, sampling="poisson", fused: bool = False,
                     stream=None) -> Plan:
    B, H, N, d = _shape4(q)
    if tuple(k.shape) != (B, H, N, d) or k.dtype != q.dtype:
        raise ValueError("q and k must share shape and dtype")
    lib = get_lib()
    prm = _Params()
    _check(lib.absa_plan_params_init(ctypes.byref(prm)))
    prm.n_clusters = n_clusters
    prm.kmeans_iters = kmeans_iters
    prm.budget_blocks = budget_blocks
    prm.seed = seed & 0xFFFFFFFFFFFFFFFF
    prm.keep_intermediates = 1 if keep_intermediates else 0
    prm.sampling = _sampling_code(sampling)
    prm.fused = 1 if fused else 0
    out = _vp()
    _check(lib.absa_plan_create(_dev(q, "q"), _dev(k, "k"), _dtype_code(q), B, H, N, d,
                                ctypes.byref(prm), _stream(stream), ctypes.byref(out)))
    return Plan(out.value)


def absa_plan_from_scores(scores, N: int, d: int, budget_blocks: int, seed: int,
                          sampling="poisson", stream=None, B: int | None = None,
                          H: int | None = None) -> Plan:
    """scores: a float32 GPU tensor [B, H, ceil(N/128), N/4], or the device
    address (int) of such an array, e.g. from absa_plan_scores, with B and H
    given."""
    if isinstance(scores, int):
        if B is None or H is None or not scores:
            raise ValueError("a device address needs B and H (and must not be 0)")
        ptr = _vp(scores)
    else:
        if scores.dtype != torch.float32 or scores.dim() != 4:
            raise ValueError("scores must be float32 [B, H, QB, M]")
        B, H = int(scores.shape[0]), int(scores.shape[1])
        if tuple(scores.shape[2:]) != ((N + 127) // 128, N // 4):
            raise ValueError("scores must be [B, H, ceil(N/128), N/4]")
        ptr = _dev(scores, "scores")
    out = _vp()
    _check(get_lib().absa_plan_from_scores(ptr, B, H, N, d, budget_blocks,
                                           seed & 0xFFFFFFFFFFFFFFFF, _sampling_code(sampling),
                                           _stream(stream), ctypes.byref(out)))
    return Plan(out.value)


def absa_plan_import(rowptr, idx, logw, p, B: int, H: int, N: int, d: int, stream=None) -> Plan:
    """Plan from a host CSR. The C call reads rowptr[0..rows] and then
    rowptr[rows] entries of idx, logw and p, so their lengths are checked
    here first (rows = B*H*ceil(N/128))."""
    rows = B * H * ((N + 127) // 128)
    rowptr, rp = _host(rowptr, np.int64)
    if rowptr.ndim != 1 or rowptr.size != rows + 1:
        raise ValueError(f"rowptr must hold rows + 1 = {rows + 1} entries (got {rowptr.size})")
    nnz = int(rowptr[-1])
    idx, ip = _host(idx, np.int32)
    logw, lp = _host(logw, np.float32)
    for name, a in (("idx", idx), ("logw", logw)):
        if a.ndim != 1 or a.size != nnz:
            raise ValueError(f"{name} must hold rowptr[-1] = {nnz} entries (got {a.size})")
    pp = _vp()
    if p is not None:
        p, pp = _host(p, np.float64)
        if p.ndim != 1 or p.size != nnz:
            raise ValueError(f"p must hold rowptr[-1] = {nnz} entries (got {p.size})")
    out = _vp()
    _check(get_lib().absa_plan_import(rp, ip, lp, pp, B, H, N, d, _stream(stream),
                                      ctypes.byref(out)))
    return Plan(out.value)


def absa_plan_scores(plan: Plan) -> int:
    """Device address of the plan's retained scores [B, H, QB, M] (float32),
    or 0 when the plan did not keep them."""
    ptr = _vp()
    _check(get_lib().absa_plan_scores(plan.handle, ctypes.byref(ptr)))
    return ptr.value or 0


def _attention_args(q, k, v, out):
    B, H, N, d = _shape4(q)
    if out is None:
        out = torch.empty_like(q)
    for t, nm in ((k, "k"), (v, "v"), (out, "out")):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{nm} must match q in shape and dtype")
    return B, H, N, d, out


def absa_sparse_attention(plan: Plan, q, k, v, out=None, stream=None):
    B, H, N, d, out = _attention_args(q, k, v, out)
    _check(get_lib().absa_sparse_attention(plan.handle, _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                           _dev(out, "out"), _dtype_code(q), B, H, N, d,
                                           _stream(stream)))
    return out


def absa_sparse_attention_noalloc(plan: Plan, q, k, v, out, stream=None):
    """The allocation-free variant: out must be given (the C call allocates
    nothing)."""
    B, H, N, d, out = _attention_args(q, k, v, out)
    _check(get_lib().absa_sparse_attention_noalloc(plan.handle, _dev(q, "q"), _dev(k, "k"),
                                                   _dev(v, "v"), _dev(out, "out"),
                                                   _dtype_code(q), B, H, N, d, _stream(stream)))
    return out


def absa_dense_attention(q, k, v, out=None, stream=None):
    B, H, N, d, out = _attention_args(q, k, v, out)
    _check(get_lib().absa_dense_attention(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                          _dev(out, "out"), _dtype_code(q), B, H, N, d,
                                          _stream(stream)))
    return out


def absa_release_cached_memory():
    """Return the library's cached plan memory on the current device to the
    system (waits for the device)."""
    _check(get_lib().absa_release_cached_memory())
