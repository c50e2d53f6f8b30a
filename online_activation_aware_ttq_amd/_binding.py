"""ctypes binding of ``libttq.so`` (the C ABI in ``include/ttq.h``).

Argument marshalling only: every step of the projection runs in the gfx950
kernels of the library.  Torch is used for device memory and streams.  If the
library has not been built, importing the compute functions raises -- there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# TTQ_LIBRARY selects another build of the same library (the CPU tests use
# it for a host build with address and undefined-behaviour sanitizers)
LIB_PATH = os.environ.get("TTQ_LIBRARY") or os.path.join(PKG_DIR, "libttq.so")

TTQ_OK = 0
TTQ_EINVAL = -1
TTQ_ENULL = -2
TTQ_EALIGN = -3
TTQ_EWORKSPACE = -4
TTQ_EUNSUPPORTED = -5
TTQ_EHIP = -100

TTQ_FLAG_FORCE_FUSED = 1
TTQ_FLAG_FORCE_TWO_PHASE = 2

# Every entry point include/ttq.h declares, with its ctypes signature.
_c = ctypes
_vp = _c.c_void_p
EXPORTS = {
    "ttq_workspace_bytes": (_c.c_int, [_vp, _c.c_int64, _c.POINTER(_c.c_size_t)]),
    "ttq_linear": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _vp, _vp, _c.c_size_t, _vp]),
    "ttq_linear_batched": (_c.c_int, [_vp, _c.c_int64, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _c.c_size_t,
                                      _vp]),
    "ttq_linear_noalloc": (_c.c_int, [_vp, _c.c_int64, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp]),
    "ttq_path": (_c.c_int, [_vp, _c.c_int64]),
    "ttq_segmented_workspace_bytes": (_c.c_int, [_vp, _c.c_int64, _vp,
                                                 _c.POINTER(_c.c_size_t)]),
    "ttq_linear_segmented": (_c.c_int, [_vp, _c.c_int64, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _c.c_size_t, _vp]),
    "ttq_packed_row_bytes": (_c.c_int, [_vp, _c.POINTER(_c.c_int64)]),
    "ttq_quantize_workspace_bytes": (_c.c_int, [_vp, _c.POINTER(_c.c_size_t)]),
    "ttq_qmatmul_workspace_bytes": (_c.c_int, [_vp, _c.POINTER(_c.c_size_t)]),
    "ttq_quantize": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _c.c_size_t, _vp]),
    "ttq_qmatmul": (_c.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _c.c_size_t, _vp]),
    "ttq_lowrank_pca_workspace_bytes": (_c.c_int, [_vp, _c.c_int32,
                                                   _c.POINTER(_c.c_size_t)]),
    "ttq_lowrank_pca": (_c.c_int, [_vp, _c.c_int32, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _vp, _c.c_size_t, _vp]),
    "ttq_status_string": (_c.c_char_p, [_c.c_int]),
    "ttq_last_hip_error": (_c.c_int, []),
    "ttq_stream_read": (_c.c_int, [_vp, _c.c_int64, _vp, _vp]),
    "ttq_version": (_c.c_char_p, []),
    "ttq_timing_enable": (_c.c_int, [_c.c_int]),
    "ttq_timing_reset": (_c.c_int, []),
    "ttq_kernel_count": (_c.c_int, []),
    "ttq_kernel_name": (_c.c_char_p, [_c.c_int]),
    "ttq_timing_query": (_c.c_int, [_c.c_int, _c.POINTER(_c.c_double),
                                    _c.POINTER(_c.c_int64)]),
}


class ttq_params(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int64),
        ("d_out", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("rank", ctypes.c_int64),
        ("bits", ctypes.c_int32),
        ("group", ctypes.c_int32),
        ("p", ctypes.c_double),
        ("lambda_", ctypes.c_double),
        ("alpha", ctypes.c_double),
        ("flags", ctypes.c_uint32),
        ("qformat", ctypes.c_uint32),
    ]


# quantizer formats (TTQ_QF_* of include/ttq.h)
QFORMATS = {"asym": 0, "sym": 1, "intzp": 2, "fp8": 3}


def qformat_code(qformat) -> int:
    """TTQ_QF_* value of a format name ("asym", "sym", "intzp", "fp8") or int."""
    if isinstance(qformat, str):
        if qformat not in QFORMATS:
            raise ValueError(f"unknown quantizer format {qformat!r}")
        return QFORMATS[qformat]
    return int(qformat)


class TTQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = ttq_status_string(status)
        if status == TTQ_EHIP:
            msg += f" (hipError {load_library().ttq_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


_lib = None


def load_library() -> ctypes.CDLL:
    """Load the in-tree ``libttq.so``; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m online_activation_aware_ttq_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def make_params(*, d: int, d_out: int, T: int, rank: int = 0, bits: int,
                group: int, p: float, lam: float, alpha: float,
                flags: int = 0, qformat="asym") -> ttq_params:
    return ttq_params(int(d), int(d_out), int(T), int(rank), int(bits),
                      int(group), float(p), float(lam), float(alpha),
                      int(flags), qformat_code(qformat))


# The calls below build the same parameter block for every call of one shape;
# the library only reads it, so one block per shape is kept (bounded).
_PARAMS = {}


def _params(d, d_out, T, rank, bits, group, p, lam, alpha, flags, qformat):
    key = (d, d_out, T, rank, bits, group, p, lam, alpha, flags, qformat)
    prm = _PARAMS.get(key)
    if prm is None:
        if len(_PARAMS) > 4096:
            _PARAMS.clear()
            _NEED.clear()
        prm = _PARAMS[key] = make_params(d=d, d_out=d_out, T=T, rank=rank,
                                         bits=bits, group=group, p=p, lam=lam,
                                         alpha=alpha, flags=flags,
                                         qformat=qformat)
    return prm, key


def _current_stream(dev) -> int:
    """Raw handle of torch's current stream on `dev` (the cheap accessor when
    this torch build has it)."""
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(dev.index if dev.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(dev).cuda_stream


# Workspace for calls that bring none: one buffer per (device, stream), kept
# between calls.  Calls on one stream run in order, so they can share it;
# calls on different streams get different buffers.  When a buffer has to
# grow, the stream is drained before the old one is released.
_NEED = {}
_SCRATCH = {}


def _workspace(dev, stream, need_key, query):
    import torch
    need = _NEED.get(need_key) if need_key is not None else None
    if need is None:
        need = max(int(query()), 256)
        if need_key is not None:
            _NEED[need_key] = need
    key = (dev.index, stream)
    buf = _SCRATCH.get(key)
    if buf is None or buf.numel() < need:
        if buf is not None:
            torch.cuda.synchronize(dev)
        buf = _SCRATCH[key] = torch.empty(need, dtype=torch.uint8, device=dev)
    return buf


def ttq_status_string(status: int) -> str:
    return load_library().ttq_status_string(int(status)).decode()


def ttq_version() -> str:
    return load_library().ttq_version().decode()


def ttq_workspace_bytes(prm: ttq_params, n_requests: int = 1) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().ttq_workspace_bytes(ctypes.byref(prm), int(n_requests),
                                            ctypes.byref(out))
    if st != TTQ_OK:
        raise TTQError(st, "ttq_workspace_bytes")
    return int(out.value)


def ttq_path(prm: ttq_params, n_requests: int = 1) -> int:
    st = load_library().ttq_path(ctypes.byref(prm), int(n_requests))
    if st < 0:
        raise TTQError(st, "ttq_path")
    return st


# ------------------------------------------------------------------ torch side
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check(t, name, dtype, shape, device):
    if t is None:
        return
    if getattr(t, "dtype", None) is not dtype:
        raise TypeError(f"{name} must be a torch.Tensor of {dtype}, got "
                        f"{getattr(t, 'dtype', type(t))}")
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _call(batched: bool, W, X, B, A, *, p, lam, alpha, bits, group, Y,
          codes_out, scales_out, mins_out, dhalf_out, workspace, stream,
          flags, qformat, noalloc=False):
    import torch
    lib = load_library()
    if batched:
        R, T, d = X.shape
    else:
        (T, d), R = X.shape, 1
    d_out = W.shape[0]
    rank = 0 if A is None else A.shape[0]
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("W must be a GPU tensor")
    lead = (R,) if batched else ()
    G = d // group if group > 0 and d % group == 0 else 0
    _check(W, "W", torch.bfloat16, (d_out, d), dev)
    _check(X, "X", torch.bfloat16, lead + (T, d), dev)
    _check(B, "B", torch.bfloat16, (d_out, rank), dev)
    _check(A, "A", torch.bfloat16, (rank, d), dev)
    if (A is None) != (B is None):
        raise ValueError("pass both B and A or neither")
    prm, key = _params(d, d_out, T, rank, bits, group, p, lam, alpha, flags,
                       qformat)
    if Y is None:
        Y = torch.empty(lead + (T, d_out), dtype=torch.float32, device=dev)
    _check(Y, "Y", torch.float32, lead + (T, d_out), dev)
    _check(codes_out, "codes_out", torch.uint8, lead + (d_out, d), dev)
    _check(scales_out, "scales_out", torch.float32, lead + (d_out, G), dev)
    _check(mins_out, "mins_out", torch.float32, lead + (d_out, G), dev)
    _check(dhalf_out, "dhalf_out", torch.float32, lead + (d,), dev)
    if stream is None:
        stream = _current_stream(dev)
    if noalloc:
        args = [_ptr(W), _ptr(X), _ptr(B), _ptr(A), _ptr(Y), _ptr(codes_out),
                _ptr(scales_out), _ptr(mins_out), _ptr(dhalf_out), stream]
        st = lib.ttq_linear_noalloc(ctypes.byref(prm), R, *args)
        if st != TTQ_OK:
            raise TTQError(st, "ttq_linear_noalloc")
        return Y
    if workspace is None:  # (a given workspace is checked by the library)
        workspace = _workspace(dev, stream, ("linear", key, R),
                               lambda: ttq_workspace_bytes(prm, R))
    args = [_ptr(W), _ptr(X), _ptr(B), _ptr(A), _ptr(Y), _ptr(codes_out),
            _ptr(scales_out), _ptr(mins_out), _ptr(dhalf_out),
            _ptr(workspace), workspace.numel(), stream]
    if batched:
        st = lib.ttq_linear_batched(ctypes.byref(prm), R, *args)
    else:
        st = lib.ttq_linear(ctypes.byref(prm), *args)
    if st != TTQ_OK:
        raise TTQError(st, "ttq_linear_batched" if batched else "ttq_linear")
    return Y


def ttq_linear(W, X, B=None, A=None, *, p: float, lam: float, alpha: float,
               bits: int, group: int, Y=None, codes_out=None, scales_out=None,
               mins_out=None, dhalf_out=None, workspace=None, stream=None,
               flags: int = 0, qformat="asym"):
    """Y[T, d_out] = Q_D[W] X + B (A X) for one request (see include/ttq.h).

    W [d_out, d], X [T, d], B [d_out, r], A [r, d] are bfloat16 GPU tensors;
    Y is float32.  Enqueued on ``stream`` (default: torch's current stream).
    """
    return _call(False, W, X, B, A, p=p, lam=lam, alpha=alpha, bits=bits,
                 group=group, Y=Y, codes_out=codes_out, scales_out=scales_out,
                 mins_out=mins_out, dhalf_out=dhalf_out, workspace=workspace,
                 stream=stream, flags=flags, qformat=qformat)


def ttq_linear_batched(W, X, B=None, A=None, *, p: float, lam: float,
                       alpha: float, bits: int, group: int, Y=None,
                       codes_out=None, scales_out=None, mins_out=None,
                       dhalf_out=None, workspace=None, stream=None,
                       flags: int = 0, qformat="asym"):
    """R requests with their own statistics on a shared W: X [R, T, d]."""
    return _call(True, W, X, B, A, p=p, lam=lam, alpha=alpha, bits=bits,
                 group=group, Y=Y, codes_out=codes_out, scales_out=scales_out,
                 mins_out=mins_out, dhalf_out=dhalf_out, workspace=workspace,
                 stream=stream, flags=flags, qformat=qformat)


def ttq_linear_noalloc(W, X, B=None, A=None, *, p: float, lam: float,
                       alpha: float, bits: int, group: int, Y,
                       codes_out=None, scales_out=None, mins_out=None,
                       dhalf_out=None, stream=None, flags: int = 0,
                       qformat="asym"):
    """ttq_linear_batched (X [R, T, d]) on the library's static scratch: no
    workspace and no allocation; Y must be given (see include/ttq.h)."""
    if Y is None:
        raise ValueError("ttq_linear_noalloc needs a preallocated Y")
    return _call(True, W, X, B, A, p=p, lam=lam, alpha=alpha, bits=bits,
                 group=group, Y=Y, codes_out=codes_out, scales_out=scales_out,
                 mins_out=mins_out, dhalf_out=dhalf_out, workspace=None,
                 stream=stream, flags=flags, qformat=qformat, noalloc=True)


TTQ_NOALLOC_SCRATCH_BYTES = 64 << 20


def _offsets(seg_offsets):
    arr = (ctypes.c_int64 * len(seg_offsets))(*[int(v) for v in seg_offsets])
    return arr, len(seg_offsets) - 1


def ttq_segmented_workspace_bytes(prm: ttq_params, seg_offsets) -> int:
    arr, n = _offsets(seg_offsets)
    out = ctypes.c_size_t(0)
    st = load_library().ttq_segmented_workspace_bytes(
        ctypes.byref(prm), n, ctypes.cast(arr, ctypes.c_void_p), ctypes.byref(out))
    if st != TTQ_OK:
        raise TTQError(st, "ttq_segmented_workspace_bytes")
    return int(out.value)


def ttq_linear_segmented(W, X, B=None, A=None, *, seg_offsets, p: float,
                         lam: float, alpha: float, bits: int, group: int,
                         Y=None, codes_out=None, scales_out=None, mins_out=None,
                         dhalf_out=None, workspace=None, stream=None,
                         flags: int = 0, qformat="asym"):
    """Requests of different lengths packed in X [T, d]: request i owns rows
    seg_offsets[i] .. seg_offsets[i+1]-1 and has its own statistics."""
    import torch
    T, d = X.shape
    d_out = W.shape[0]
    rank = 0 if A is None else A.shape[0]
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("W must be a GPU tensor")
    n = len(seg_offsets) - 1
    G = d // group if group > 0 and d % group == 0 else 0
    _check(W, "W", torch.bfloat16, (d_out, d), dev)
    _check(X, "X", torch.bfloat16, (T, d), dev)
    _check(B, "B", torch.bfloat16, (d_out, rank), dev)
    _check(A, "A", torch.bfloat16, (rank, d), dev)
    if (A is None) != (B is None):
        raise ValueError("pass both B and A or neither")
    prm = make_params(d=d, d_out=d_out, T=T, rank=rank, bits=bits,
                      group=group, p=p, lam=lam, alpha=alpha, flags=flags,
                      qformat=qformat)
    if Y is None:
        Y = torch.empty((T, d_out), dtype=torch.float32, device=dev)
    _check(Y, "Y", torch.float32, (T, d_out), dev)
    _check(codes_out, "codes_out", torch.uint8, (n, d_out, d), dev)
    _check(scales_out, "scales_out", torch.float32, (n, d_out, G), dev)
    _check(mins_out, "mins_out", torch.float32, (n, d_out, G), dev)
    _check(dhalf_out, "dhalf_out", torch.float32, (n, d), dev)
    if stream is None:
        stream = _current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, stream, None,
                               lambda: ttq_segmented_workspace_bytes(prm, seg_offsets))
    arr, _ = _offsets(seg_offsets)
    st = load_library().ttq_linear_segmented(
        ctypes.byref(prm), n, ctypes.cast(arr, ctypes.c_void_p), _ptr(W),
        _ptr(X), _ptr(B), _ptr(A), _ptr(Y), _ptr(codes_out), _ptr(scales_out),
        _ptr(mins_out), _ptr(dhalf_out), _ptr(workspace), workspace.numel(),
        stream)
    if st != TTQ_OK:
        raise TTQError(st, "ttq_linear_segmented")
    return Y


# ------------------------------------------- quantize once, decode from codes
def container_bits(bits: int) -> int:
    """Bits each stored code takes (1, 2, 4 or 8)."""
    return 1 if bits <= 1 else 2 if bits <= 2 else 4 if bits <= 4 else 8


def ttq_packed_row_bytes(prm: ttq_params) -> int:
    out = ctypes.c_int64(0)
    st = load_library().ttq_packed_row_bytes(ctypes.byref(prm), ctypes.byref(out))
    if st != TTQ_OK:
        raise TTQError(st, "ttq_packed_row_bytes")
    return int(out.value)


_ROW_BYTES = {}


def _row_bytes(d: int, bits: int, group: int) -> int:
    """Packed row bytes for the shape checks of the calls below (the calls
    themselves validate every parameter)."""
    key = (d, bits, group)
    if key not in _ROW_BYTES:
        _ROW_BYTES[key] = ttq_packed_row_bytes(
            make_params(d=d, d_out=1, T=0, bits=bits, group=group, p=1.0,
                        lam=0.0, alpha=0.0))
    return _ROW_BYTES[key]


def ttq_quantize_workspace_bytes(prm: ttq_params) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().ttq_quantize_workspace_bytes(ctypes.byref(prm),
                                                     ctypes.byref(out))
    if st != TTQ_OK:
        raise TTQError(st, "ttq_quantize_workspace_bytes")
    return int(out.value)


def ttq_qmatmul_workspace_bytes(prm: ttq_params) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().ttq_qmatmul_workspace_bytes(ctypes.byref(prm),
                                                    ctypes.byref(out))
    if st != TTQ_OK:
        raise TTQError(st, "ttq_qmatmul_workspace_bytes")
    return int(out.value)


def ttq_quantize(W, X, *, p: float, lam: float, alpha: float, bits: int,
                 group: int, codes=None, scales=None, mins=None,
                 dhalf_inv=None, dhalf_out=None, workspace=None, stream=None,
                 qformat="asym"):
    """Quantize W once for the prompt X (see include/ttq.h).

    Returns (codes [d_out, row_bytes] uint8, scales [d_out, G] float32,
    mins [d_out, G] float32, dhalf_inv [d] float32).
    """
    import torch
    lib = load_library()
    T, d = X.shape
    d_out = W.shape[0]
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("W must be a GPU tensor")
    prm = make_params(d=d, d_out=d_out, T=T, bits=bits, group=group, p=p,
                      lam=lam, alpha=alpha, qformat=qformat)
    rb = ttq_packed_row_bytes(prm)
    G = d // group
    _check(W, "W", torch.bfloat16, (d_out, d), dev)
    _check(X, "X", torch.bfloat16, (T, d), dev)
    if codes is None:
        codes = torch.empty((d_out, rb), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((d_out, G), dtype=torch.float32, device=dev)
    if mins is None:
        mins = torch.empty((d_out, G), dtype=torch.float32, device=dev)
    if dhalf_inv is None:
        dhalf_inv = torch.empty((d,), dtype=torch.float32, device=dev)
    _check(codes, "codes", torch.uint8, (d_out, rb), dev)
    _check(scales, "scales", torch.float32, (d_out, G), dev)
    _check(mins, "mins", torch.float32, (d_out, G), dev)
    _check(dhalf_inv, "dhalf_inv", torch.float32, (d,), dev)
    _check(dhalf_out, "dhalf_out", torch.float32, (d,), dev)
    if stream is None:
        stream = _current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, stream, None,
                               lambda: ttq_quantize_workspace_bytes(prm))
    st = lib.ttq_quantize(ctypes.byref(prm), _ptr(W), _ptr(X), _ptr(codes),
                          _ptr(scales), _ptr(mins), _ptr(dhalf_inv),
                          _ptr(dhalf_out), _ptr(workspace), workspace.numel(),
                          stream)
    if st != TTQ_OK:
        raise TTQError(st, "ttq_quantize")
    return codes, scales, mins, dhalf_inv


def ttq_qmatmul(codes, scales, mins, dhalf_inv, X, B=None, A=None, *,
                bits: int, group: int, Y=None, workspace=None, stream=None,
                flags: int = 0, qformat="asym"):
    """Y[T, d_out] = X ((min + s q) D^{-1/2})^T + (X A^T) B^T from the codes
    stored by ttq_quantize (see include/ttq.h; ``qformat`` as given to it:
    E4M3 codes decode as FP8 values)."""
    import torch
    lib = load_library()
    T, d = X.shape
    d_out = codes.shape[0]
    rank = 0 if A is None else A.shape[0]
    dev = X.device
    if dev.type != "cuda":
        raise ValueError("X must be a GPU tensor")
    if (A is None) != (B is None):
        raise ValueError("pass both B and A or neither")
    prm, key = _params(d, d_out, T, rank, bits, group, 1.0, 0.0, 0.0, flags,
                       qformat)
    rb = _row_bytes(d, bits, group)
    G = d // group
    _check(codes, "codes", torch.uint8, (d_out, rb), dev)
    _check(scales, "scales", torch.float32, (d_out, G), dev)
    _check(mins, "mins", torch.float32, (d_out, G), dev)
    _check(dhalf_inv, "dhalf_inv", torch.float32, (d,), dev)
    _check(X, "X", torch.bfloat16, (T, d), dev)
    _check(B, "B", torch.bfloat16, (d_out, rank), dev)
    _check(A, "A", torch.bfloat16, (rank, d), dev)
    if Y is None:
        Y = torch.empty((T, d_out), dtype=torch.float32, device=dev)
    _check(Y, "Y", torch.float32, (T, d_out), dev)
    if stream is None:
        stream = _current_stream(dev)
    if workspace is None:  # (a given workspace is checked by the library)
        workspace = _workspace(dev, stream, ("qmatmul", key),
                               lambda: ttq_qmatmul_workspace_bytes(prm))
    st = lib.ttq_qmatmul(ctypes.byref(prm), _ptr(codes), _ptr(scales),
                         _ptr(mins), _ptr(dhalf_inv), _ptr(X), _ptr(B), _ptr(A),
                         _ptr(Y), _ptr(workspace), workspace.numel(), stream)
    if st != TTQ_OK:
        raise TTQError(st, "ttq_qmatmul")
    return Y


# ------------------------------------------------- low-rank factors by PCA
def ttq_lowrank_pca_workspace_bytes(prm: ttq_params, iters: int) -> int:
    out = ctypes.c_size_t(0)
    st = load_library().ttq_lowrank_pca_workspace_bytes(
        ctypes.byref(prm), int(iters), ctypes.byref(out))
    if st != TTQ_OK:
        raise TTQError(st, "ttq_lowrank_pca_workspace_bytes")
    return int(out.value)


def ttq_lowrank_pca(W, Omega, *, iters: int, X=None, p: float = 2.0,
                    lam: float = 0.0, alpha: float = 0.0, want_residual=True,
                    workspace=None, stream=None):
    """Low-rank factors by PCA (see include/ttq.h): returns (B [d_out, r],
    A [r, d], Wres [d_out, d] or None), bf16 GPU tensors.  ``Omega`` is the
    float32 [d, r] Gaussian test matrix; with ``X`` ([T, d] bf16) the
    principal subspace is that of W D^{1/2}."""
    import torch
    d_out, d = W.shape
    r = Omega.shape[1]
    T = 0 if X is None else X.shape[0]
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("W must be a GPU tensor")
    _check(W, "W", torch.bfloat16, (d_out, d), dev)
    _check(Omega, "Omega", torch.float32, (d, r), dev)
    if X is not None:
        _check(X, "X", torch.bfloat16, (T, d), dev)
    prm = make_params(d=d, d_out=d_out, T=T, rank=r, bits=4, group=32, p=p,
                      lam=lam, alpha=alpha)
    B = torch.empty((d_out, r), dtype=torch.bfloat16, device=dev)
    A = torch.empty((r, d), dtype=torch.bfloat16, device=dev)
    Wres = torch.empty((d_out, d), dtype=torch.bfloat16, device=dev) \
        if want_residual else None
    if stream is None:
        stream = _current_stream(dev)
    if workspace is None:
        workspace = _workspace(dev, stream, None,
                               lambda: ttq_lowrank_pca_workspace_bytes(prm, iters))
    st = load_library().ttq_lowrank_pca(
        ctypes.byref(prm), int(iters), _ptr(W), _ptr(X), _ptr(Omega), _ptr(B),
        _ptr(A), _ptr(Wres), _ptr(workspace), workspace.numel(), stream)
    if st != TTQ_OK:
        raise TTQError(st, "ttq_lowrank_pca")
    return B, A, Wres


# ------------------------------------------------------------------ timing
def stream_read(src, sink=None, stream=None):
    """Plain read of a device tensor's bytes (the ceiling of a one-pass
    kernel over W; see ttq_stream_read).  Returns the per-workgroup XOR
    words (uint32 stored in an int32 tensor)."""
    import torch
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("stream_read: src must be a contiguous device tensor")
    nbytes = src.numel() * src.element_size()
    nblk = -(-nbytes // (128 * 1024))
    if sink is None:
        sink = torch.empty(max(1, nblk), dtype=torch.int32, device=src.device)
    if stream is None:
        stream = _current_stream(src.device)
    st = load_library().ttq_stream_read(_ptr(src), nbytes, _ptr(sink), stream)
    if st != TTQ_OK:
        raise TTQError(st, "ttq_stream_read")
    return sink


def timing_enable(on: bool = True) -> None:
    load_library().ttq_timing_enable(1 if on else 0)


def timing_reset() -> None:
    load_library().ttq_timing_reset()


def timing_query() -> dict:
    """{kernel name: (total milliseconds, launches)} for recorded launches."""
    lib = load_library()
    out = {}
    for k in range(lib.ttq_kernel_count()):
        ms = ctypes.c_double(0.0)
        n = ctypes.c_int64(0)
        st = lib.ttq_timing_query(k, ctypes.byref(ms), ctypes.byref(n))
        if st != TTQ_OK:
            raise TTQError(st, "ttq_timing_query")
        out[lib.ttq_kernel_name(k).decode()] = (ms.value, n.value)
    return out
