"""ctypes binding of libssd.so (include/ssd.h) for torch tensors.

Argument marshalling only: shapes and dtypes are checked, outputs allocated
with torch on the input's device, and the C entry point is called on torch's
current stream.  Every step of the forward, backward and decode passes runs
in the library's HIP kernels; there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssd.so")
_lib = None

SSD_OK = 0
SSD_DTYPE_F32 = 0
SSD_DTYPE_BF16 = 1
_STATUS = {0: "SSD_OK", 1: "SSD_ERR_INVALID_ARGUMENT", 2: "SSD_ERR_UNSUPPORTED",
           3: "SSD_ERR_HIP", 4: "SSD_ERR_OUT_OF_MEMORY", 5: "SSD_ERR_SCRATCH_LIMIT"}

# Every function include/ssd.h declares, with its ctypes signature.
_vp, _fp, _i32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
_i64, _i32 = ctypes.c_int64, ctypes.c_int32
SIGNATURES = {
    "ssd_chunked_fwd": ([_vp, _fp, _fp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                         _i32, _vp, _fp, _vp], ctypes.c_int),
    "ssd_chunked_fwd_noalloc": ([_vp, _fp, _fp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _vp, _fp, _vp], ctypes.c_int),
    "ssd_chunked_fwd_varlen": ([_vp, _fp, _fp, _vp, _vp, _i32p, _i64, _i64, _i32, _i32, _i32,
                                _i32, _i32, _i32, _vp, _fp, _vp], ctypes.c_int),
    "ssd_chunked_fwd_ex": ([_vp, _fp, _fp, _vp, _vp, _i32p, _i64, _i64, _i32, _i32, _i32, _i32,
                            _i32, _i32, _fp, _fp, _i32, _vp, _fp, _vp], ctypes.c_int),
    "ssd_chunked_bwd": ([_vp, _fp, _fp, _vp, _vp, _i32p, _i64, _i64, _i32, _i32, _i32, _i32, _i32,
                         _i32, _fp, _fp, _i32, _vp, _fp, _vp, _fp, _fp, _vp, _vp, _fp, _fp, _vp],
                        ctypes.c_int),
    "ssd_decode_step": ([_vp, _fp, _fp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _fp, _i32, _fp,
                         _vp, _vp], ctypes.c_int),
    "ssd_chunked_fwd_normalized": ([_vp, _fp, _fp, _vp, _vp, _i32p, _i64, _i64, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _fp, _i32, _vp, _fp, _fp, _vp], ctypes.c_int),
    "ssd_selective_scan": ([_vp, _fp, _fp, _vp, _vp, _i64, _i64, _i32, _i32, _i32, _vp, _fp, _vp],
                           ctypes.c_int),
    "ssd_chunked_fwd_intermediates": ([_vp, _fp, _fp, _vp, _vp, _i32p, _i64, _i64, _i32, _i32,
                                       _i32, _i32, _i32, _i32, _vp, _fp, _fp, _fp, _fp, _vp],
                                      ctypes.c_int),
    "ssd_chunk_slots": ([_i64, _i64, _i32, _i32], ctypes.c_int64),
    "ssd_config_supported": ([_i32, _i32, _i32], ctypes.c_int32),
    "ssd_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "ssd_workspace_selfcheck": ([], ctypes.c_int32),
    "ssd_kernel_timing_enable": ([_i32], ctypes.c_int),
    "ssd_kernel_timing_read": ([_i32, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_int64), _i32], ctypes.c_int),
}

KERNEL_NAMES = ["seq_table", "chunk_state", "state_pass", "chunk_output", "chunk_cb", "decode_step",
                "backward_glue", "selective_scan"]


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}")


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise SSDError(-1, f"libssd.so not built at {_LIB_PATH} "
                               "(run python -m mamba_ssd_layer_amd.build)")
        l = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            f = getattr(l, name)
            f.argtypes = args
            f.restype = res
        _lib = l
    return _lib


def _check(rc: int, where: str):
    if rc != SSD_OK:
        raise SSDError(rc, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_DTYPE_BF16
    if t.dtype == torch.float32:
        return SSD_DTYPE_F32
    raise TypeError("x/B/C must be bfloat16 or float32")


def _need(t: torch.Tensor, name: str, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def ssd_chunked_fwd(x, dt, A_head, B, C, chunk_len: int, y=None, final_state=None,
                    return_final_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Batched SSD forward. x (b,T,H,P), dt (b,T,H) fp32, A_head (H,) fp32,
    B/C (b,T,G,N) in x's dtype.  Returns (y (b,T,H,P), final_state (b,H,P,N) fp32 or None)."""
    if x.dim() != 4:
        raise ValueError("x must be (batch, seqlen, nheads, headdim)")
    b, T, H, P = x.shape
    G, N = B.shape[-2:]
    dev = x.device
    _need(x, "x", x.dtype, dev)
    _need(dt, "dt", torch.float32, dev)
    _need(A_head, "A_head", torch.float32, dev)
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev)
    if tuple(dt.shape) != (b, T, H) or tuple(A_head.shape) != (H,) or \
            tuple(B.shape) != (b, T, G, N) or tuple(C.shape) != (b, T, G, N):
        raise ValueError("inconsistent shapes")
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, dev)
        if y.shape != x.shape:
            raise ValueError("y must have x's shape")
    if final_state is None and return_final_state:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, dev)
        if tuple(final_state.shape) != (b, H, P, N):
            raise ValueError("final_state must be (b,H,P,N)")
    rc = lib().ssd_chunked_fwd(_ptr(x), _ptr(dt), _ptr(A_head), _ptr(B), _ptr(C), b, T, H, P, N,
                               G, int(chunk_len), _dtype_code(x), _ptr(y), _ptr(final_state),
                               ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_chunked_fwd")
    return y, final_state


def ssd_chunked_fwd_noalloc(x, dt, A_head, B, C, chunk_len: int, y, final_state=None):
    """ssd_chunked_fwd through the entry point that allocates nothing (its
    workspace is the library's static device scratch): the caller passes y and
    optionally final_state, and nothing is allocated here either."""
    if x.dim() != 4:
        raise ValueError("x must be (batch, seqlen, nheads, headdim)")
    b, T, H, P = x.shape
    G, N = B.shape[-2:]
    dev = x.device
    for t, n, d in ((x, "x", x.dtype), (dt, "dt", torch.float32), (A_head, "A_head", torch.float32),
                    (B, "B", x.dtype), (C, "C", x.dtype), (y, "y", x.dtype)):
        _need(t, n, d, dev)
    if tuple(dt.shape) != (b, T, H) or tuple(A_head.shape) != (H,) or \
            tuple(B.shape) != (b, T, G, N) or tuple(C.shape) != (b, T, G, N) or y.shape != x.shape:
        raise ValueError("inconsistent shapes")
    if final_state is not None:
        _need(final_state, "final_state", torch.float32, dev)
        if tuple(final_state.shape) != (b, H, P, N):
            raise ValueError("final_state must be (b,H,P,N)")
    rc = lib().ssd_chunked_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(A_head), _ptr(B), _ptr(C), b, T, H, P, N,
                                       G, int(chunk_len), _dtype_code(x), _ptr(y), _ptr(final_state),
                                       ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_chunked_fwd_noalloc")
    return y, final_state


def ssd_chunked_fwd_varlen(x, dt, A_head, B, C, cu_seqlens, chunk_len: int, y=None,
                           final_state=None, return_final_state: bool = True):
    """Packed variable-length SSD forward. x (Ttot,H,P), dt (Ttot,H), B/C (Ttot,G,N),
    cu_seqlens (S+1,) int32 on the device.  Returns (y, final_state (S,H,P,N) or None)."""
    if x.dim() != 3:
        raise ValueError("x must be (total_len, nheads, headdim)")
    Tt, H, P = x.shape
    G, N = B.shape[-2:]
    dev = x.device
    _need(x, "x", x.dtype, dev)
    _need(dt, "dt", torch.float32, dev)
    _need(A_head, "A_head", torch.float32, dev)
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
    S = cu_seqlens.shape[0] - 1
    if tuple(dt.shape) != (Tt, H) or tuple(B.shape) != (Tt, G, N) or tuple(C.shape) != (Tt, G, N):
        raise ValueError("inconsistent shapes")
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
    rc = lib().ssd_chunked_fwd_varlen(_ptr(x), _ptr(dt), _ptr(A_head), _ptr(B), _ptr(C),
                                      _ptr(cu_seqlens), S, Tt, H, P, N, G, int(chunk_len),
                                      _dtype_code(x), _ptr(y), _ptr(final_state),
                                      ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_chunked_fwd_varlen")
    return y, final_state


def ssd_chunked_fwd_ex(x, dt, A_head, B, C, chunk_len: int, cu_seqlens=None, initial_state=None,
                       D=None, x_times_dt: bool = False, y=None, final_state=None,
                       return_final_state: bool = True):
    """SSD forward with the options of ssd_chunked_fwd_ex.  Batched (4-D x
    (b,T,H,P), cu_seqlens None) or packed (3-D x (Ttot,H,P) with cu_seqlens (S+1,)
    int32 on the device).  initial_state (S,H,P,N) fp32 or None (zero); D (H,) fp32
    or None (skip term y += D_h x); x_times_dt: the input enters as dt x.
    Returns (y, final_state (S,H,P,N) or None)."""
    dev = x.device
    if x.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens goes with packed 3-D inputs")
        b, T, H, P = x.shape
        S, Tt = b, b * T
        lead = (b, T)
    elif x.dim() == 3:
        if cu_seqlens is None:
            raise ValueError("packed 3-D inputs need cu_seqlens")
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        Tt, H, P = x.shape
        S = cu_seqlens.shape[0] - 1
        lead = (Tt,)
    else:
        raise ValueError("x must be (b,T,H,P) or (Ttot,H,P)")
    G, N = B.shape[-2:]
    _need(x, "x", x.dtype, dev)
    _need(dt, "dt", torch.float32, dev)
    _need(A_head, "A_head", torch.float32, dev)
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev)
    if tuple(dt.shape) != lead + (H,) or tuple(A_head.shape) != (H,) or \
            tuple(B.shape) != lead + (G, N) or tuple(C.shape) != lead + (G, N):
        raise ValueError("inconsistent shapes")
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, dev)
        if tuple(initial_state.shape) != (S, H, P, N):
            raise ValueError("initial_state must be (S,H,P,N)")
    if D is not None:
        _need(D, "D", torch.float32, dev)
        if tuple(D.shape) != (H,):
            raise ValueError("D must be (H,)")
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, dev)
        if y.shape != x.shape:
            raise ValueError("y must have x's shape")
    if final_state is None and return_final_state:
        final_state = torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _need(final_state, "final_state", torch.float32, dev)
        if tuple(final_state.shape) != (S, H, P, N):
            raise ValueError("final_state must be (S,H,P,N)")
    rc = lib().ssd_chunked_fwd_ex(_ptr(x), _ptr(dt), _ptr(A_head), _ptr(B), _ptr(C), _ptr(cu_seqlens),
                                  S, Tt, H, P, N, G, int(chunk_len), _dtype_code(x),
                                  _ptr(initial_state), _ptr(D), 1 if x_times_dt else 0,
                                  _ptr(y), _ptr(final_state),
                                  ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_chunked_fwd_ex")
    return y, final_state


def ssd_chunked_fwd_normalized(x, dt, A_head, B, C, chunk_len: int, cu_seqlens=None, D=None,
                               x_times_dt: bool = False, return_final_state: bool = True, y=None,
                               denom=None):
    """SSD forward with the output divided by its denominator term M 1
    (ssd_chunked_fwd_normalized).  Inputs as ssd_chunked_fwd_ex without an
    initial state; B and C should come from a positive feature map.  y (x's
    shape and dtype) and denom ((Ttot,H) fp32) may be given to be written in
    place.  Returns (y, final_state (S,H,P,N) or None, denom (Ttot,H) fp32)."""
    dev = x.device
    if x.dim() == 4:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens goes with packed 3-D inputs")
        b, T, H, P = x.shape
        S, Tt = b, b * T
        lead = (b, T)
    elif x.dim() == 3:
        if cu_seqlens is None:
            raise ValueError("packed 3-D inputs need cu_seqlens")
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        Tt, H, P = x.shape
        S = cu_seqlens.shape[0] - 1
        lead = (Tt,)
    else:
        raise ValueError("x must be (b,T,H,P) or (Ttot,H,P)")
    G, N = B.shape[-2:]
    _need(x, "x", x.dtype, dev)
    _need(dt, "dt", torch.float32, dev)
    _need(A_head, "A_head", torch.float32, dev)
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev)
    if tuple(dt.shape) != lead + (H,) or tuple(A_head.shape) != (H,) or \
            tuple(B.shape) != lead + (G, N) or tuple(C.shape) != lead + (G, N):
        raise ValueError("inconsistent shapes")
    if D is not None:
        _need(D, "D", torch.float32, dev)
        if tuple(D.shape) != (H,):
            raise ValueError("D must be (H,)")
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, dev)
        if y.shape != x.shape:
            raise ValueError("y must have x's shape")
    final_state = torch.empty((S, H, P, N), dtype=torch.float32, device=dev) if return_final_state else None
    if denom is None:
        denom = torch.empty((Tt, H), dtype=torch.float32, device=dev)
    else:
        _need(denom, "denom", torch.float32, dev)
        if tuple(denom.shape) != (Tt, H):
            raise ValueError("denom must be (Ttot, H)")
    rc = lib().ssd_chunked_fwd_normalized(_ptr(x), _ptr(dt), _ptr(A_head), _ptr(B), _ptr(C), _ptr(cu_seqlens),
                                          S, Tt, H, P, N, G, int(chunk_len), _dtype_code(x), _ptr(D),
                                          1 if x_times_dt else 0, _ptr(y), _ptr(final_state), _ptr(denom),
                                          ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_chunked_fwd_normalized")
    return y, final_state, denom


def ssd_chunked_bwd(x, dt, A_head, B, C, dy, chunk_len: int, cu_seqlens=None, initial_state=None,
                    D=None, x_times_dt: bool = False, dfinal_state=None, want_dD: bool = False,
                    want_dinitial: bool = False):
    """Gradients of the SSD forward (ssd_chunked_fwd_ex's arguments) given dy (x's
    shape and dtype) and optionally dfinal_state (S,H,P,N) fp32.  Returns a dict
    dx, ddt, dA, dB, dC, and dD / dinitial_state when asked for (None otherwise)."""
    dev = x.device
    if x.dim() == 4:
        b, T, H, P = x.shape
        S, Tt = b, b * T
    elif x.dim() == 3:
        if cu_seqlens is None:
            raise ValueError("packed 3-D inputs need cu_seqlens")
        _need(cu_seqlens, "cu_seqlens", torch.int32, dev)
        Tt, H, P = x.shape
        S = cu_seqlens.shape[0] - 1
    else:
        raise ValueError("x must be (b,T,H,P) or (Ttot,H,P)")
    G, N = B.shape[-2:]
    for t, name, dtp in ((x, "x", x.dtype), (dt, "dt", torch.float32), (A_head, "A_head", torch.float32),
                         (B, "B", x.dtype), (C, "C", x.dtype), (dy, "dy", x.dtype)):
        _need(t, name, dtp, dev)
    if dy.shape != x.shape or B.shape != C.shape or tuple(A_head.shape) != (H,):
        raise ValueError("inconsistent shapes")
    for t, name, shp in ((initial_state, "initial_state", (S, H, P, N)), (dfinal_state, "dfinal_state", (S, H, P, N)),
                         (D, "D", (H,))):
        if t is not None:
            _need(t, name, torch.float32, dev)
            if tuple(t.shape) != shp:
                raise ValueError(f"{name} must be {shp}")
    out = dict(dx=torch.empty_like(x), ddt=torch.empty_like(dt), dA=torch.empty((H,), dtype=torch.float32, device=dev),
               dB=torch.empty_like(B), dC=torch.empty_like(C),
               dD=torch.empty((H,), dtype=torch.float32, device=dev) if want_dD else None,
               dinitial_state=torch.empty((S, H, P, N), dtype=torch.float32, device=dev) if want_dinitial else None)
    rc = lib().ssd_chunked_bwd(_ptr(x), _ptr(dt), _ptr(A_head), _ptr(B), _ptr(C), _ptr(cu_seqlens), S, Tt, H, P,
                               N, G, int(chunk_len), _dtype_code(x), _ptr(initial_state), _ptr(D),
                               1 if x_times_dt else 0, _ptr(dy), _ptr(dfinal_state), _ptr(out["dx"]),
                               _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]),
                               _ptr(out["dD"]), _ptr(out["dinitial_state"]), ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_chunked_bwd")
    return out


def ssd_decode_step(x, dt, A_head, B, C, state, y=None, D=None, x_times_dt: bool = False):
    """One recurrent (decode) step.  x (b,H,P), dt (b,H) fp32, A_head (H,) fp32,
    B/C (b,G,N) in x's dtype, state (b,H,P,N) fp32, updated in place; D and
    x_times_dt as for ssd_chunked_fwd_ex.  Returns y (b,H,P) in x's dtype."""
    if x.dim() != 3:
        raise ValueError("x must be (batch, nheads, headdim)")
    b, H, P = x.shape
    G, N = B.shape[-2:]
    dev = x.device
    _need(x, "x", x.dtype, dev)
    _need(dt, "dt", torch.float32, dev)
    _need(A_head, "A_head", torch.float32, dev)
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev)
    _need(state, "state", torch.float32, dev)
    if tuple(dt.shape) != (b, H) or tuple(A_head.shape) != (H,) or tuple(B.shape) != (b, G, N) or \
            tuple(C.shape) != (b, G, N) or tuple(state.shape) != (b, H, P, N):
        raise ValueError("inconsistent shapes")
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, dev)
        if y.shape != x.shape:
            raise ValueError("y must have x's shape")
    if D is not None:
        _need(D, "D", torch.float32, dev)
        if tuple(D.shape) != (H,):
            raise ValueError("D must be (H,)")
    rc = lib().ssd_decode_step(_ptr(x), _ptr(dt), _ptr(A_head), _ptr(B), _ptr(C), b, H, P, N, G,
                               _dtype_code(x), _ptr(D), 1 if x_times_dt else 0, _ptr(state), _ptr(y),
                               ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_decode_step")
    return y


def ssd_selective_scan(x, delta, A, B, C, y=None, want_final_state: bool = True):
    """The comparator: selective scan with a diagonal transition.  x (b,D,T)
    and delta (b,D,T) channel-major (delta fp32), A (D,N) fp32, B/C (b,T,N) in
    x's dtype.  Returns y (b,D,T) in x's dtype and the final state (b,D,N) fp32
    (None unless want_final_state)."""
    if x.dim() != 3:
        raise ValueError("x must be (batch, channels, seqlen)")
    b, D, T = x.shape
    N = A.shape[-1]
    dev = x.device
    _need(x, "x", x.dtype, dev)
    _need(delta, "delta", torch.float32, dev)
    _need(A, "A", torch.float32, dev)
    _need(B, "B", x.dtype, dev)
    _need(C, "C", x.dtype, dev)
    if tuple(delta.shape) != (b, D, T) or tuple(A.shape) != (D, N) or tuple(B.shape) != (b, T, N) or \
            tuple(C.shape) != (b, T, N):
        raise ValueError("inconsistent shapes")
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", x.dtype, dev)
        if y.shape != x.shape:
            raise ValueError("y must have x's shape")
    fs = torch.empty((b, D, N), dtype=torch.float32, device=dev) if want_final_state else None
    rc = lib().ssd_selective_scan(_ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), b, T, D, N,
                                  _dtype_code(x), _ptr(y), _ptr(fs), ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_selective_scan")
    return y, fs


def ssd_chunked_fwd_intermediates(x, dt, A_head, B, C, chunk_len: int, cu_seqlens=None):
    """Forward pass that also returns the per-chunk intermediates (fp32):
    acs (K,H,Q), states (K,H,P,N), hin (K,H,P,N), with K = chunk slots.
    Batched inputs (4-D x) or packed inputs with cu_seqlens."""
    dev = x.device
    if x.dim() == 4:
        b, T = x.shape[:2]
        S, Tt = b, b * T
        varlen = 0
    else:
        Tt = x.shape[0]
        S = cu_seqlens.shape[0] - 1
        varlen = 1
    H, P = x.shape[-2:]
    G, N = B.shape[-2:]
    Q = int(chunk_len)
    K = int(lib().ssd_chunk_slots(S, Tt, Q, varlen))
    y = torch.empty_like(x)
    fs = torch.empty((S, H, P, N), dtype=torch.float32, device=dev)
    acs = torch.full((K, H, Q), float("nan"), dtype=torch.float32, device=dev)
    states = torch.full((K, H, P, N), float("nan"), dtype=torch.float32, device=dev)
    hin = torch.full((K, H, P, N), float("nan"), dtype=torch.float32, device=dev)
    rc = lib().ssd_chunked_fwd_intermediates(
        _ptr(x), _ptr(dt), _ptr(A_head), _ptr(B), _ptr(C), _ptr(cu_seqlens) if varlen else None,
        S, Tt, H, P, N, G, Q, _dtype_code(x), _ptr(y), _ptr(fs), _ptr(acs), _ptr(states),
        _ptr(hin), ctypes.c_void_p(_stream_ptr(dev)))
    _check(rc, "ssd_chunked_fwd_intermediates")
    return dict(y=y, final_state=fs, acs=acs, states=states, hin=hin)


def config_supported(dtype: torch.dtype, dstate: int, chunk_len: int) -> bool:
    code = SSD_DTYPE_BF16 if dtype == torch.bfloat16 else SSD_DTYPE_F32
    return bool(lib().ssd_config_supported(code, int(dstate), int(chunk_len)))


def kernel_timing_enable(on: bool):
    _check(lib().ssd_kernel_timing_enable(1 if on else 0), "ssd_kernel_timing_enable")


def kernel_timing_read(reset: bool = True) -> dict:
    """{kernel name: (total ms, launches)} of the timed launches since the last reset."""
    out = {}
    for k, name in enumerate(KERNEL_NAMES):
        ms = ctypes.c_double(0.0)
        n = ctypes.c_int64(0)
        _check(lib().ssd_kernel_timing_read(k, ctypes.byref(ms), ctypes.byref(n), 1 if reset else 0),
               "ssd_kernel_timing_read")
        out[name] = (ms.value, n.value)
    return out
