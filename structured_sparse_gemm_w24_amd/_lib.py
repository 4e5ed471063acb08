"""ctypes binding of libssg.so: argument marshalling only.

Pack functions take and return numpy arrays (host memory).  GEMM functions
take torch tensors on the current HIP device and launch on torch's current
stream; outputs are allocated with torch unless ``out`` is given.  Every step
of the computation runs inside the library; a nonzero status raises
``SsgError`` carrying the library's message.  If the library is not built,
every call raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes as ct
import os
import threading
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LOCK = threading.Lock()
_LIB = None

STATUS = {0: "SSG_OK", 1: "SSG_EINVAL", 2: "SSG_ENOT24", 3: "SSG_ENOSPC", 4: "SSG_ENODEV",
          5: "SSG_EARCH", 6: "SSG_EHIP"}
SSG_OK, SSG_EINVAL, SSG_ENOT24, SSG_ENOSPC, SSG_ENODEV, SSG_EARCH, SSG_EHIP = range(7)


class SsgError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


class TwSizes(ct.Structure):
    _fields_ = [("T", ct.c_int64), ("sum_kt", ct.c_int64), ("sum_nt", ct.c_int64), ("vals_elems", ct.c_int64)]


_P = ct.c_void_p
_I64 = ct.c_int64
_I32 = ct.c_int32

# name -> argument types (every function returns int, but ssg_splitk_workspace_bytes: int64)
SIGNATURES = {
    "w24_pack_f16": [_P, _I64, _I64, _P, _P],
    "w24_pack_i8": [_P, _I64, _I64, _P, _P],
    "w24_unpack_f16": [_P, _P, _I64, _I64, _P],
    "w24_unpack_i8": [_P, _P, _I64, _I64, _P],
    "tw_pack_query": [_P, _I64, _I64, _I32, ct.POINTER(TwSizes)],
    "tw_pack_f16": [_P, _I64, _I64, _I32, ct.POINTER(TwSizes), _P, _P, _P, _P, _P, _P, _P],
    "tw_unpack_f16": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _P],
    "tw_pack_query_i8": [_P, _I64, _I64, _I32, ct.POINTER(TwSizes)],
    "tw_pack_i8": [_P, _I64, _I64, _I32, ct.POINTER(TwSizes), _P, _P, _P, _P, _P, _P, _P],
    "tw_unpack_i8": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I32, _P],
    "dense_gemm_f16": [_P, _P, _P, _I64, _I64, _I64, _P],
    "dense_gemm_i8": [_P, _P, _P, _P, _I64, _I64, _I64, _P],
    "w24_gemm_f16": [_P, _P, _P, _P, _I64, _I64, _I64, _P],
    "w24_gemm_i8": [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P],
    "dense_gemm_i8_out": [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P],
    "w24_gemm_i8_out": [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _P],
    "tw_gemm_f16": [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _I64, _I64, _I64, _P],
    "tw_gemm_i8": [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _P, _P, _P, _I32, _I64, _I64, _I64, _P],
    "tw_gemm_f16_ex": [_P, _P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P, _I64, _I64, _I64, _P],
    "ssg_transpose_f16": [_P, _P, _I64, _I64, _P],
    "ssg_device_arch": [ct.c_char_p, _I64],
    "dense_gemm_f16_splitk": [_P, _P, _P, _I64, _I64, _I64, _I32, _P, _I64, _P],
    "w24_gemm_f16_splitk": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P, _I64, _P],
    "dense_gemm_i8_splitk": [_P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _I64, _P],
    "w24_gemm_i8_splitk": [_P, _P, _P, _P, _P, _P, _I32, _I64, _I64, _I64, _I32, _P, _I64, _P],
    "w24_gemm_f16_splitk_static": [_P, _P, _P, _P, _I64, _I64, _I64, _I32, _P],
    "ssg_splitk_suggest": [_I32, _I64, _I64, _I64],
    "ssg_tile_choice": [_I32, _I64, _I64, _I64],
}


def lib_path():
    return os.environ.get("SSG_LIB", os.path.join(_HERE, "libssg.so"))


def load():
    """Load libssg.so once (raises if it has not been built).

    torch (which holds the device memory and streams of the GEMM calls) is
    imported first when it is installed: its wheel carries its own HIP
    runtime, and the library then binds to that one instead of loading the
    system runtime beside it.  Two HIP runtimes initialised in one process
    leave the second without a device (the library's calls fail with
    SSG_ENODEV, or torch reports no GPU), which is what happens when the
    library is loaded before torch."""
    global _LIB
    with _LOCK:
        if _LIB is None:
            try:
                import torch  # noqa: F401
            except ImportError:
                pass
            path = lib_path()
            if not os.path.exists(path):
                raise RuntimeError(f"{path} is missing: build it with "
                                   f"`python -m structured_sparse_gemm_w24_amd.build`")
            lib = ct.CDLL(path, mode=ct.RTLD_LOCAL)
            for name, argtypes in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.argtypes = argtypes
                fn.restype = ct.c_int
            lib.ssg_last_error.argtypes = []
            lib.ssg_last_error.restype = ct.c_char_p
            lib.ssg_version.argtypes = []
            lib.ssg_version.restype = ct.c_char_p
            lib.ssg_splitk_workspace_bytes.argtypes = [_I64, _I64, _I32]
            lib.ssg_splitk_workspace_bytes.restype = ct.c_int64
            _LIB = lib
    return _LIB


def _check(rc):
    if rc != SSG_OK:
        raise SsgError(rc, load().ssg_last_error().decode())


def _np_ptr(a):
    return a.ctypes.data_as(ct.c_void_p) if a is not None else None


def _host(a, dtype, ndim=None):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    if ndim is not None and a.ndim != ndim:
        raise ValueError(f"expected a {ndim}-d array, got shape {a.shape}")
    return a


# ---------------------------------------------------------------- pack stage
def w24_pack_f16(W):
    """W [K, N] float16 (2:4 along K) -> (vals [N, K/2] float16, meta [N, ceil(K/32)] uint32)."""
    W = _host(W, np.float16, 2)
    K, N = W.shape
    vals = np.empty((N, K // 2), np.float16)
    meta = np.empty((N, -(-K // 32)), np.uint32)
    _check(load().w24_pack_f16(_np_ptr(W), K, N, _np_ptr(vals), _np_ptr(meta)))
    return vals, meta


def w24_pack_i8(W):
    W = _host(W, np.int8, 2)
    K, N = W.shape
    vals = np.empty((N, K // 2), np.int8)
    meta = np.empty((N, -(-K // 32)), np.uint32)
    _check(load().w24_pack_i8(_np_ptr(W), K, N, _np_ptr(vals), _np_ptr(meta)))
    return vals, meta


def w24_unpack_f16(vals, meta, K, N):
    vals = _host(vals, np.float16, 2)
    meta = _host(meta, np.uint32, 2)
    if vals.shape != (N, K // 2) or meta.shape != (N, -(-K // 32)):
        raise ValueError("vals/meta shape does not match K, N")
    W = np.empty((K, N), np.float16)
    _check(load().w24_unpack_f16(_np_ptr(vals), _np_ptr(meta), K, N, _np_ptr(W)))
    return W


def w24_unpack_i8(vals, meta, K, N):
    vals = _host(vals, np.int8, 2)
    meta = _host(meta, np.uint32, 2)
    if vals.shape != (N, K // 2) or meta.shape != (N, -(-K // 32)):
        raise ValueError("vals/meta shape does not match K, N")
    W = np.empty((K, N), np.int8)
    _check(load().w24_unpack_i8(_np_ptr(vals), _np_ptr(meta), K, N, _np_ptr(W)))
    return W


@dataclass
class TwPacked:
    """Condensed tile-wise weight (host numpy arrays, or torch tensors after ``to``)."""
    K: int
    N: int
    G: int
    T: int
    vals: object
    offset_k: object
    offset_n: object
    v_ptr: object
    k_ptr: object
    n_ptr: object
    tile_order: object
    max_nt: int = -1  # most kept columns of any tile (-1: not known)

    def arrays(self):
        return dict(vals=self.vals, offset_k=self.offset_k, offset_n=self.offset_n, v_ptr=self.v_ptr,
                    k_ptr=self.k_ptr, n_ptr=self.n_ptr, tile_order=self.tile_order)

    def to(self, device):
        """Copy every array to a torch device (int32 / float16 tensors)."""
        import torch

        def conv(a):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return t.to(device) if t.numel() else torch.zeros(1, dtype=t.dtype, device=device)
        return TwPacked(self.K, self.N, self.G, self.T, *[conv(a) for a in self.arrays().values()],
                        max_nt=self.max_nt)

    def narrow(self):
        """True when every tile is known to keep at most 64 columns (SSG_TW_NARROW)."""
        return 0 <= self.max_nt <= 64


def _tw_fns(dtype):
    dt = np.dtype(dtype)
    if dt == np.float16:
        return np.float16, "tw_pack_query", "tw_pack_f16", "tw_unpack_f16"
    if dt == np.int8:
        return np.int8, "tw_pack_query_i8", "tw_pack_i8", "tw_unpack_i8"
    raise TypeError(f"tile-wise packing takes float16 or int8, got {dt}")


def tw_pack_query(W, G):
    dt, q, _, _ = _tw_fns(np.asarray(W).dtype)
    W = _host(W, dt, 2)
    K, N = W.shape
    sz = TwSizes()
    _check(getattr(load(), q)(_np_ptr(W), K, N, G, ct.byref(sz)))
    return dict(T=sz.T, sum_kt=sz.sum_kt, sum_nt=sz.sum_nt, vals_elems=sz.vals_elems)


def _tw_pack(W, G, dt, q, pk):
    W = _host(W, dt, 2)
    K, N = W.shape
    sz = TwSizes()
    _check(getattr(load(), q)(_np_ptr(W), K, N, G, ct.byref(sz)))
    vals = np.empty(sz.vals_elems, dt)
    ok = np.empty(sz.sum_kt, np.int32)
    on = np.empty(sz.sum_nt, np.int32)
    vp = np.empty(sz.T + 1, np.int32)
    kp = np.empty(sz.T + 1, np.int32)
    np_ = np.empty(sz.T + 1, np.int32)
    order = np.empty(sz.T, np.int32)
    _check(getattr(load(), pk)(_np_ptr(W), K, N, G, ct.byref(sz), _np_ptr(vals), _np_ptr(ok), _np_ptr(on),
                               _np_ptr(vp), _np_ptr(kp), _np_ptr(np_), _np_ptr(order)))
    return TwPacked(K, N, G, int(sz.T), vals, ok, on, vp, kp, np_, order,
                    max_nt=int(np.diff(np_).max()) if sz.T > 0 else 0)


def tw_pack_f16(W, G):
    """W [K, N] float16 -> TwPacked (host arrays)."""
    return _tw_pack(W, G, np.float16, "tw_pack_query", "tw_pack_f16")


def tw_pack_i8(W, G):
    """W [K, N] int8 -> TwPacked (host arrays, int8 values, rows padded to 16)."""
    return _tw_pack(W, G, np.int8, "tw_pack_query_i8", "tw_pack_i8")


def _tw_unpack(p: TwPacked, dt, fn):
    W = np.empty((p.K, p.N), dt)
    arrs = [_host(p.vals, dt), _host(p.offset_k, np.int32), _host(p.offset_n, np.int32),
            _host(p.v_ptr, np.int32), _host(p.k_ptr, np.int32), _host(p.n_ptr, np.int32)]
    # the library reads T+1 prefix sums and as many values / offsets as they
    # claim: check the lengths here, where they are known
    T = -(-p.N // p.G)
    vals, offk, offn, vp, kp, np_ = arrs
    if vp.size != T + 1 or kp.size != T + 1 or np_.size != T + 1:
        raise ValueError(f"prefix-sum arrays must hold T+1 = {T + 1} entries")
    if vals.size < vp[-1] or offk.size < kp[-1] or offn.size < np_[-1]:
        raise ValueError("vals / offset_k / offset_n shorter than their prefix sums claim")
    _check(getattr(load(), fn)(*[_np_ptr(a) for a in arrs], p.K, p.N, p.G, _np_ptr(W)))
    return W


def tw_unpack_f16(p: TwPacked):
    return _tw_unpack(p, np.float16, "tw_unpack_f16")


def tw_unpack_i8(p: TwPacked):
    return _tw_unpack(p, np.int8, "tw_unpack_i8")


# ---------------------------------------------------------------- device side
def _torch():
    import torch
    return torch


def _dev(t, dtype, shape=None, name="tensor"):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a torch tensor on a HIP device")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return ct.c_void_p(t.data_ptr()) if t is not None else None


def _on(first, *others):
    """Every tensor of a call on first's device; returns the context that
    makes that device current for the launch (the library checks and launches
    on the current device, on that device's current torch stream)."""
    torch = _torch()
    for t in others:
        if t is not None and t.device != first.device:
            raise ValueError(f"all tensors must be on {first.device}, found one on {t.device}")
    return torch.cuda.device(first.device)


def _stream(t):
    torch = _torch()
    return ct.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _out(out, shape, dtype, like):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    return _dev(out, dtype, shape, "out")


def ssg_device_arch():
    buf = ct.create_string_buffer(256)
    _check(load().ssg_device_arch(buf, 256))
    return buf.value.decode()


# GEMM kinds of the split-K calls (SSG_KIND_* in ssg.h).
SSG_KIND_DENSE_F16, SSG_KIND_W24_F16, SSG_KIND_DENSE_I8, SSG_KIND_W24_I8 = 0, 1, 2, 3


def splitk_suggest(kind, M, N, K):
    """The library's K-split count for a GEMM kind and shape (1 = unsplit)."""
    return int(load().ssg_splitk_suggest(kind, M, N, K))


def tile_choice(kind, M, N, K):
    """(rows, columns) of the output tile the library's GEMMs use for a kind and shape."""
    v = int(load().ssg_tile_choice(kind, M, N, K))
    return v // 1024, v % 1024


def splitk_workspace_bytes(M, N, splits):
    return int(load().ssg_splitk_workspace_bytes(M, N, splits))


def _splits(kind, M, N, K, splits):
    """splits=None: the library's suggestion; otherwise the caller's count (1 = the
    unsplit entry point)."""
    return splitk_suggest(kind, M, N, K) if splits is None else int(splits)


def _workspace(M, N, p, like, ws=None):
    """Device workspace of a split call: the caller's (a uint8 tensor of at least
    splitk_workspace_bytes(M, N, p) bytes), else one from torch's caching allocator
    (stream-ordered reuse, so it may be released as soon as the launches are queued)."""
    torch = _torch()
    if ws is not None:
        _dev(ws, torch.uint8, None, "workspace")
        return ws
    return torch.empty(max(16, splitk_workspace_bytes(M, N, p)), dtype=torch.uint8, device=like.device)


def dense_gemm_f16(A, Wt, out=None, splits=None, workspace=None):
    """C = A . Wt^T; A [M, K] fp16, Wt [N, K] fp16 -> C [M, N] fp16.  splits: K splits
    (None: the library's choice for the shape; see dense_gemm_f16_splitk in ssg.h)."""
    torch = _torch()
    M, K = A.shape
    N = Wt.shape[0]
    _dev(A, torch.float16, (M, K), "A")
    _dev(Wt, torch.float16, (N, K), "Wt")
    C = _out(out, (M, N), torch.float16, A)
    p = _splits(SSG_KIND_DENSE_F16, M, N, K, splits)
    with _on(A, Wt, C):
        if p == 1:
            _check(load().dense_gemm_f16(_ptr(A), _ptr(Wt), _ptr(C), M, N, K, _stream(A)))
        else:
            ws = _workspace(M, N, p, A, workspace)
            _check(load().dense_gemm_f16_splitk(_ptr(A), _ptr(Wt), _ptr(C), M, N, K, p, _ptr(ws), ws.numel(),
                                                _stream(A)))
    return C


def dense_gemm_i8(A, Wt, scale=None, out=None, splits=None, workspace=None):
    """int8 dense GEMM; scale None -> int32 C, else fp32 C = float(acc) * scale[n]."""
    torch = _torch()
    M, K = A.shape
    N = Wt.shape[0]
    _dev(A, torch.int8, (M, K), "A")
    _dev(Wt, torch.int8, (N, K), "Wt")
    if scale is not None:
        _dev(scale, torch.float32, (N,), "scale")
    C = _out(out, (M, N), torch.int32 if scale is None else torch.float32, A)
    p = _splits(SSG_KIND_DENSE_I8, M, N, K, splits)
    with _on(A, Wt, scale, C):
        if p == 1:
            _check(load().dense_gemm_i8(_ptr(A), _ptr(Wt), _ptr(scale), _ptr(C), M, N, K, _stream(A)))
        else:
            ws = _workspace(M, N, p, A, workspace)
            code = SSG_OUT_I32 if scale is None else SSG_OUT_F32
            _check(load().dense_gemm_i8_splitk(_ptr(A), _ptr(Wt), _ptr(scale), None, _ptr(C), code, M, N, K, p,
                                               _ptr(ws), ws.numel(), _stream(A)))
    return C


# Output kinds of the int8 GEMMs' selectable epilogue (SSG_OUT_* in ssg.h).
SSG_OUT_I32, SSG_OUT_F32, SSG_OUT_F16, SSG_OUT_I8 = 0, 1, 2, 3
_OUT_KINDS = {"i32": SSG_OUT_I32, "f32": SSG_OUT_F32, "f16": SSG_OUT_F16, "i8": SSG_OUT_I8}


def _out_kind(out_type):
    torch = _torch()
    if out_type not in _OUT_KINDS:
        raise ValueError(f"out_type must be one of {sorted(_OUT_KINDS)}, got {out_type!r}")
    dt = {"i32": torch.int32, "f32": torch.float32, "f16": torch.float16, "i8": torch.int8}[out_type]
    return _OUT_KINDS[out_type], dt


def _epilogue_args(N, scale, bias):
    torch = _torch()
    if scale is not None:
        _dev(scale, torch.float32, (N,), "scale")
    if bias is not None:
        _dev(bias, torch.float32, (N,), "bias")


def dense_gemm_i8_out(A, Wt, scale, bias=None, out_type="f16", out=None, splits=None, workspace=None):
    """int8 dense GEMM with the selectable epilogue: y = float(acc) * scale[n] (+ bias[n]),
    stored as out_type ("f32", "f16", "i8"; "i32" = raw accumulators, no scale or bias)."""
    torch = _torch()
    M, K = A.shape
    N = Wt.shape[0]
    _dev(A, torch.int8, (M, K), "A")
    _dev(Wt, torch.int8, (N, K), "Wt")
    code, dt = _out_kind(out_type)
    _epilogue_args(N, scale, bias)
    C = _out(out, (M, N), dt, A)
    p = _splits(SSG_KIND_DENSE_I8, M, N, K, splits)
    with _on(A, Wt, scale, bias, C):
        if p == 1:
            _check(load().dense_gemm_i8_out(_ptr(A), _ptr(Wt), _ptr(scale), _ptr(bias), _ptr(C), code, M, N, K,
                                            _stream(A)))
        else:
            ws = _workspace(M, N, p, A, workspace)
            _check(load().dense_gemm_i8_splitk(_ptr(A), _ptr(Wt), _ptr(scale), _ptr(bias), _ptr(C), code, M, N, K,
                                               p, _ptr(ws), ws.numel(), _stream(A)))
    return C


def w24_gemm_i8_out(A, vals, meta, scale, bias=None, out_type="f16", out=None, splits=None, workspace=None):
    """2:4 int8 GEMM with the selectable epilogue (see dense_gemm_i8_out)."""
    torch = _torch()
    M, K = A.shape
    N = vals.shape[0]
    _dev(A, torch.int8, (M, K), "A")
    _dev(vals, torch.int8, (N, K // 2), "vals")
    _dev(meta, torch.int32, (N, -(-K // 32)), "meta")
    code, dt = _out_kind(out_type)
    _epilogue_args(N, scale, bias)
    C = _out(out, (M, N), dt, A)
    p = _splits(SSG_KIND_W24_I8, M, N, K, splits)
    with _on(A, vals, meta, scale, bias, C):
        if p == 1:
            _check(load().w24_gemm_i8_out(_ptr(A), _ptr(vals), _ptr(meta), _ptr(scale), _ptr(bias), _ptr(C), code,
                                          M, N, K, _stream(A)))
        else:
            ws = _workspace(M, N, p, A, workspace)
            _check(load().w24_gemm_i8_splitk(_ptr(A), _ptr(vals), _ptr(meta), _ptr(scale), _ptr(bias), _ptr(C),
                                             code, M, N, K, p, _ptr(ws), ws.numel(), _stream(A)))
    return C


def w24_gemm_f16(A, vals, meta, out=None, splits=None, workspace=None):
    """2:4 GEMM; A [M, K] fp16, vals [N, K/2] fp16, meta [N, K/32] int32 (uint32 bits).
    splits: K splits (None: the library's choice for the shape)."""
    torch = _torch()
    M, K = A.shape
    N = vals.shape[0]
    _dev(A, torch.float16, (M, K), "A")
    _dev(vals, torch.float16, (N, K // 2), "vals")
    _dev(meta, torch.int32, (N, -(-K // 32)), "meta")
    C = _out(out, (M, N), torch.float16, A)
    p = _splits(SSG_KIND_W24_F16, M, N, K, splits)
    with _on(A, vals, meta, C):
        if p == 1:
            _check(load().w24_gemm_f16(_ptr(A), _ptr(vals), _ptr(meta), _ptr(C), M, N, K, _stream(A)))
        else:
            ws = _workspace(M, N, p, A, workspace)
            _check(load().w24_gemm_f16_splitk(_ptr(A), _ptr(vals), _ptr(meta), _ptr(C), M, N, K, p, _ptr(ws),
                                              ws.numel(), _stream(A)))
    return C


def w24_gemm_i8(A, vals, meta, scale=None, out=None, splits=None, workspace=None):
    """2:4 int8 GEMM; scale None -> int32 C, else fp32 C = float(acc) * scale[n]."""
    torch = _torch()
    M, K = A.shape
    N = vals.shape[0]
    _dev(A, torch.int8, (M, K), "A")
    _dev(vals, torch.int8, (N, K // 2), "vals")
    _dev(meta, torch.int32, (N, -(-K // 32)), "meta")
    if scale is not None:
        _dev(scale, torch.float32, (N,), "scale")
    C = _out(out, (M, N), torch.int32 if scale is None else torch.float32, A)
    p = _splits(SSG_KIND_W24_I8, M, N, K, splits)
    with _on(A, vals, meta, scale, C):
        if p == 1:
            _check(load().w24_gemm_i8(_ptr(A), _ptr(vals), _ptr(meta), _ptr(scale), _ptr(C), M, N, K, _stream(A)))
        else:
            ws = _workspace(M, N, p, A, workspace)
            code = SSG_OUT_I32 if scale is None else SSG_OUT_F32
            _check(load().w24_gemm_i8_splitk(_ptr(A), _ptr(vals), _ptr(meta), _ptr(scale), None, _ptr(C), code,
                                             M, N, K, p, _ptr(ws), ws.numel(), _stream(A)))
    return C


def dense_gemm_f16_splitk(A, Wt, splits, workspace=None, out=None):
    """dense_gemm_f16 with K split `splits` ways (1 = unsplit); workspace: optional uint8
    device tensor of at least splitk_workspace_bytes(M, N, splits) bytes."""
    return dense_gemm_f16(A, Wt, out=out, splits=splits, workspace=workspace)


def w24_gemm_f16_splitk(A, vals, meta, splits, workspace=None, out=None):
    """w24_gemm_f16 with K split `splits` ways (see dense_gemm_f16_splitk)."""
    return w24_gemm_f16(A, vals, meta, out=out, splits=splits, workspace=workspace)


SSG_STATIC_SCRATCH_BYTES = 32 << 20


def w24_gemm_f16_splitk_static(A, vals, meta, splits, out=None):
    """w24_gemm_f16_splitk without a workspace: the partials go to the library's
    static per-GPU scratch (splits * M * N * 4 <= SSG_STATIC_SCRATCH_BYTES).
    Calls that may overlap on one GPU race on that scratch."""
    torch = _torch()
    M, K = A.shape
    N = vals.shape[0]
    _dev(A, torch.float16, (M, K), "A")
    _dev(vals, torch.float16, (N, K // 2), "vals")
    _dev(meta, torch.int32, (N, -(-K // 32)), "meta")
    C = _out(out, (M, N), torch.float16, A)
    with _on(A, vals, meta, C):
        _check(load().w24_gemm_f16_splitk_static(_ptr(A), _ptr(vals), _ptr(meta), _ptr(C), M, N, K, int(splits),
                                                 _stream(A)))
    return C


def dense_gemm_i8_splitk(A, Wt, scale, bias=None, out_type="f16", splits=1, workspace=None, out=None):
    """dense_gemm_i8_out with K split `splits` ways (int8 results equal the unsplit call's)."""
    return dense_gemm_i8_out(A, Wt, scale, bias, out_type=out_type, out=out, splits=splits, workspace=workspace)


def w24_gemm_i8_splitk(A, vals, meta, scale, bias=None, out_type="f16", splits=1, workspace=None, out=None):
    """w24_gemm_i8_out with K split `splits` ways (int8 results equal the unsplit call's)."""
    return w24_gemm_i8_out(A, vals, meta, scale, bias, out_type=out_type, out=out, splits=splits,
                           workspace=workspace)


def tw_gemm_f16(At, packed: TwPacked, out=None):
    """Tile-wise GEMM; At [K, M] fp16 (K-major A), packed arrays on the device.  When
    the packer found every tile at most 64 columns wide, the call goes through
    tw_gemm_f16_ex with SSG_TW_NARROW (the same result from the narrow-tile kernels)."""
    if packed.narrow():
        return tw_gemm_f16_ex(At, packed, out=out)
    torch = _torch()
    K, M = At.shape
    if K != packed.K:
        raise ValueError(f"At has K={K}, packed weight has K={packed.K}")
    _dev(At, torch.float16, (K, M), "At")
    arrs = packed.arrays()
    _dev(arrs["vals"], torch.float16, None, "vals")
    for key in ("offset_k", "offset_n", "v_ptr", "k_ptr", "n_ptr", "tile_order"):
        _dev(arrs[key], torch.int32, None, key)
    C = _out(out, (M, packed.N), torch.float16, At)
    with _on(At, C, *arrs.values()):
        _check(load().tw_gemm_f16(_ptr(At), _ptr(arrs["vals"]), _ptr(arrs["offset_k"]), _ptr(arrs["offset_n"]),
                                  _ptr(arrs["v_ptr"]), _ptr(arrs["k_ptr"]), _ptr(arrs["n_ptr"]),
                                  _ptr(arrs["tile_order"]), packed.T, packed.G, _ptr(C), M, packed.N, K, _stream(At)))
    return C


def tw_gemm_i8(At, packed: TwPacked, scale, bias=None, out_type="f16", out=None):
    """int8 tile-wise GEMM; At [K, M] int8 (K-major A), packed int8 tiles on the device;
    y = float(acc) * scale[n] (+ bias[n]) stored as out_type ("f32", "f16", "i8"; "i32"
    writes the raw accumulators and takes no scale or bias)."""
    torch = _torch()
    K, M = At.shape
    if K != packed.K:
        raise ValueError(f"At has K={K}, packed weight has K={packed.K}")
    _dev(At, torch.int8, (K, M), "At")
    arrs = packed.arrays()
    _dev(arrs["vals"], torch.int8, None, "vals")
    for key in ("offset_k", "offset_n", "v_ptr", "k_ptr", "n_ptr", "tile_order"):
        _dev(arrs[key], torch.int32, None, key)
    code, dt = _out_kind(out_type)
    _epilogue_args(packed.N, scale, bias)
    C = _out(out, (M, packed.N), dt, At)
    with _on(At, C, scale, bias, *arrs.values()):
        _check(load().tw_gemm_i8(_ptr(At), _ptr(arrs["vals"]), _ptr(arrs["offset_k"]), _ptr(arrs["offset_n"]),
                                 _ptr(arrs["v_ptr"]), _ptr(arrs["k_ptr"]), _ptr(arrs["n_ptr"]),
                                 _ptr(arrs["tile_order"]), packed.T, packed.G, _ptr(scale), _ptr(bias), _ptr(C),
                                 code, M, packed.N, K, _stream(At)))
    return C


SSG_TW_OUT_T = 1


SSG_TW_A_ROWMAJOR = 2


SSG_TW_NARROW = 4


def tw_gemm_f16_ex(At, packed: TwPacked, t_first=0, t_count=None, out_t=False, a_rowmajor=False, out=None,
                   narrow=None):
    """Tile-wise GEMM over tiles tile_order[t_first : t_first + t_count]; with out_t the
    result is written transposed, Ct [N, M] (the K-major input of a next tile-wise layer).
    With a_rowmajor the first argument is row-major A [M, K] (the slides' "without
    transpose" case).  Only the selected tiles' column windows of the output are written.
    narrow: pass SSG_TW_NARROW (None: when the packer found every tile <= 64 columns)."""
    torch = _torch()
    if a_rowmajor:
        M, K = At.shape
    else:
        K, M = At.shape
    if K != packed.K:
        raise ValueError(f"At has K={K}, packed weight has K={packed.K}")
    if t_count is None:
        t_count = packed.T - t_first
    _dev(At, torch.float16, (M, K) if a_rowmajor else (K, M), "A" if a_rowmajor else "At")
    arrs = packed.arrays()
    _dev(arrs["vals"], torch.float16, None, "vals")
    for key in ("offset_k", "offset_n", "v_ptr", "k_ptr", "n_ptr", "tile_order"):
        _dev(arrs[key], torch.int32, None, key)
    C = _out(out, (packed.N, M) if out_t else (M, packed.N), torch.float16, At)
    if narrow is None:
        narrow = packed.narrow()
    flags = ((SSG_TW_OUT_T if out_t else 0) | (SSG_TW_A_ROWMAJOR if a_rowmajor else 0)
             | (SSG_TW_NARROW if narrow else 0))
    with _on(At, C, *arrs.values()):
        _check(load().tw_gemm_f16_ex(_ptr(At), _ptr(arrs["vals"]), _ptr(arrs["offset_k"]), _ptr(arrs["offset_n"]),
                                     _ptr(arrs["v_ptr"]), _ptr(arrs["k_ptr"]), _ptr(arrs["n_ptr"]),
                                     _ptr(arrs["tile_order"]), packed.T, packed.G, int(t_first), int(t_count),
                                     flags, _ptr(C), M, packed.N, K, _stream(At)))
    return C


def tw_gemm_f16_streams(At, packed: TwPacked, streams, out=None):
    """The slides' multi-stream schedule: one launch per condensed tile, tiles taken
    in tile_order and dealt round-robin over `streams` (default-priority torch
    streams); the current stream waits for all of them before returning."""
    torch = _torch()
    K, M = At.shape
    C = _out(out, (M, packed.N), torch.float16, At)
    cur = torch.cuda.current_stream()
    for st in streams:
        st.wait_stream(cur)
    for i in range(packed.T):
        with torch.cuda.stream(streams[i % len(streams)]):
            tw_gemm_f16_ex(At, packed, t_first=i, t_count=1, out=C)
    for st in streams:
        cur.wait_stream(st)
    return C


def ssg_transpose_f16(A, out=None):
    """At [K, M] = A^T for A [M, K] fp16."""
    torch = _torch()
    M, K = A.shape
    _dev(A, torch.float16, (M, K), "A")
    At = _out(out, (K, M), torch.float16, A)
    with _on(A, At):
        _check(load().ssg_transpose_f16(_ptr(A), _ptr(At), M, K, _stream(A)))
    return At
