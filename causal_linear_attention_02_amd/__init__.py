"""Kernelized (linear) attention on AMD Instinct MI355X.

Thin Python binding over the C ABI of ``liblinattn.so`` (declared in
include/linattn.h). Functions carry the same names as the C entry points and
only marshal arguments: shapes and dtypes are read from torch tensors, raw
device pointers and the current HIP stream are passed through ctypes, and
outputs / workspace are allocated with torch (device memory plumbing). Every
step of the computation runs in the library's HIP kernels; importing this
package fails when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "LA_OK", "LA_ERR_INVALID_ARG", "LA_ERR_UNSUPPORTED", "LA_ERR_WORKSPACE", "LA_ERR_HIP",
    "LA_F32", "LA_BF16", "LA_ELU1", "LA_PERFORMER", "LA_IDENTITY", "LA_POLY2",
    "la_feature_map", "lib", "library_path", "LinAttnError",
    "la_version", "la_status_string", "la_forward_workspace_size", "la_forward", "la_forward_ex",
    "la_decode_step", "la_feature_map_apply", "feature_dim", "la_forward_decay", "la_decode_step_decay",
    "la_backward_workspace_size", "la_backward", "la_backward_decay", "la_forward_gated_workspace_size", "la_forward_gated",
    "la_decode_step_gated", "la_device_status", "la_forward_static", "LA_STATIC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# LINATTN_LIBRARY names another build of this same library (for example a
# host-side sanitizer build of the ABI layer used by the CPU tests)
library_path = os.environ.get("LINATTN_LIBRARY") or os.path.join(_HERE, "liblinattn.so")
header_path = os.path.join(os.path.dirname(_HERE), "include", "linattn.h")

LA_OK = 0
LA_ERR_INVALID_ARG = -1
LA_ERR_UNSUPPORTED = -2
LA_ERR_WORKSPACE = -3
LA_ERR_HIP = -4
LA_F32 = 0
LA_BF16 = 1
LA_ELU1 = 0
LA_PERFORMER = 1
LA_IDENTITY = 2
LA_POLY2 = 3
LA_STATIC_SCRATCH_BYTES = 32 << 20   # the fixed device workspace of la_forward_static, per GPU


class la_feature_map(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("m", ctypes.c_int), ("W", ctypes.c_void_p)]


def _load():
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build the HIP library first "
            "(python causal_linear_attention_02_amd/build.py)")
    L = ctypes.CDLL(library_path)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    fmp = ctypes.POINTER(la_feature_map)
    L.la_version.argtypes, L.la_version.restype = [], i
    L.la_status_string.argtypes, L.la_status_string.restype = [i], ctypes.c_char_p
    L.la_device_status.argtypes, L.la_device_status.restype = [vp], i
    L.la_forward_workspace_size.argtypes = [i, i, i, i, fmp, i]
    L.la_forward_workspace_size.restype = sz
    L.la_forward_workspace_size_dt.argtypes = [i, i, i, i, fmp, i, i]
    L.la_forward_workspace_size_dt.restype = sz
    fwd = [vp, vp, vp, vp, i, i, i, i, fmp, i, i, i, vp, vp, vp, vp, vp, sz, vp]
    L.la_forward.argtypes, L.la_forward.restype = fwd, i
    L.la_forward_ex.argtypes, L.la_forward_ex.restype = fwd + [vp], i
    L.la_forward_static.argtypes, L.la_forward_static.restype = fwd[:16] + [vp], i
    L.la_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, fmp, i, i, vp]
    L.la_decode_step.restype = i
    L.la_forward_decay.argtypes = [vp, vp, vp, vp, i, i, i, i, fmp, vp, i, i, vp, vp, vp, vp, vp, sz, vp]
    L.la_forward_decay.restype = i
    L.la_decode_step_decay.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, fmp, vp, i, i, vp]
    L.la_decode_step_decay.restype = i
    L.la_feature_map_apply.argtypes = [vp, vp, ctypes.c_longlong, i, fmp, i, i, vp]
    L.la_feature_map_apply.restype = i
    L.la_backward_workspace_size.argtypes = [i, i, i, i, fmp]
    L.la_backward_workspace_size.restype = sz
    L.la_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, fmp, i, i, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.la_backward.restype = i
    L.la_backward_decay.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, fmp, vp, i, i, vp, vp, vp, vp, vp, vp, vp,
                                    sz, vp]
    L.la_backward_decay.restype = i
    L.la_forward_gated_workspace_size.argtypes = [i, i, i, i, fmp]
    L.la_forward_gated_workspace_size.restype = sz
    L.la_forward_gated.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, fmp, i, i, vp, vp, vp, vp, vp, sz, vp]
    L.la_forward_gated.restype = i
    L.la_decode_step_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, fmp, i, i, vp]
    L.la_decode_step_gated.restype = i
    return L


lib = _load()


class LinAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {lib.la_status_string(status).decode()} ({status})")


def _check(status: int, what: str):
    if status == LA_OK:
        return
    if status in (LA_ERR_INVALID_ARG, LA_ERR_WORKSPACE):
        raise ValueError(f"{what}: {lib.la_status_string(status).decode()} ({status})")
    if status == LA_ERR_UNSUPPORTED:
        raise NotImplementedError(f"{what}: {lib.la_status_string(status).decode()} ({status})")
    raise LinAttnError(status, what)


def declared_functions():
    """Names of the functions declared in include/linattn.h."""
    with open(header_path) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(la_\w+)\s*\(", text, re.M)))


def _dtype_code(t: torch.Tensor) -> int:
    return _dtype_code_of(t.dtype)


def _dtype_code_of(dtype) -> int:
    if dtype == torch.bfloat16:
        return LA_BF16
    if dtype == torch.float32:
        return LA_F32
    raise TypeError(f"unsupported dtype {dtype}; use bfloat16 or float32")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live in GPU memory")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _fmap(feature_map: str, W):
    if feature_map in ("elu1", LA_ELU1):
        return la_feature_map(LA_ELU1, 0, None)
    if feature_map in ("identity", LA_IDENTITY):
        return la_feature_map(LA_IDENTITY, 0, None)
    if feature_map in ("poly2", LA_POLY2):
        return la_feature_map(LA_POLY2, 0, None)
    if feature_map in ("performer", LA_PERFORMER):
        if W is None:
            raise ValueError("the performer map needs W (m x d, float32, on the device)")
        if W.dtype != torch.float32:
            raise TypeError("W must be float32")
        return la_feature_map(LA_PERFORMER, int(W.shape[0]), _ptr(W))
    raise ValueError(f"unknown feature map {feature_map!r}")


def feature_dim(d: int, feature_map: str = "elu1", W=None) -> int:
    if feature_map in ("poly2", LA_POLY2):
        return 1 + d + d * d
    return int(W.shape[0]) if feature_map in ("performer", LA_PERFORMER) else d


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def la_version() -> int:
    return lib.la_version()


def la_status_string(status: int) -> str:
    return lib.la_status_string(status).decode()


def la_device_status(stream=None) -> int:
    """Synchronize the stream, then read and clear the device flag raised by
    decay factors or gates outside [1/4, 1]: LA_OK or LA_ERR_INVALID_ARG."""
    st = lib.la_device_status(_stream(stream))
    if st not in (LA_OK, LA_ERR_INVALID_ARG):
        raise LinAttnError(st, "la_device_status")
    return st


def la_forward_workspace_size(B, H, N, d, feature_map="elu1", W=None, causal=True, dtype=None) -> int:
    """Workspace bytes of la_forward; exact for `dtype` (torch.float32 or
    torch.bfloat16) when given, else enough for either."""
    fm = _fmap(feature_map, W)
    if dtype is None:
        return int(lib.la_forward_workspace_size(B, H, N, d, ctypes.byref(fm), int(causal)))
    return int(lib.la_forward_workspace_size_dt(B, H, N, d, ctypes.byref(fm), int(causal), _dtype_code_of(dtype)))


def la_forward_ex(q, k, v, *, feature_map="elu1", W=None, causal=True, normalize=True, S_in=None, z_in=None,
                  return_state=False, out=None, workspace=None, stream=None, events=None):
    """Linear attention over [B, H, N, d] tensors. Returns out, or (out, S, z)."""
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    fm = _fmap(feature_map, W)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if out is None:
        out = torch.empty_like(q)
    S_out = z_out = None
    if return_state:
        df = feature_dim(d, feature_map, W)
        S_out = torch.empty((B, H, df, d), device=q.device, dtype=torch.float32)
        z_out = torch.empty((B, H, df), device=q.device, dtype=torch.float32)
    need = int(lib.la_forward_workspace_size_dt(B, H, N, d, ctypes.byref(fm), int(causal), dt))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ev = None
    if events is not None:
        if len(events) != 4:
            raise ValueError("events: exactly 4 timing events are recorded")
        for e in events:
            if e.cuda_event == 0:   # torch creates the HIP event on first use
                e.record()
        arr = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
        ev = ctypes.cast(arr, ctypes.c_void_p)
    st = lib.la_forward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, ctypes.byref(fm), int(causal),
                           int(normalize), dt, _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                           _ptr(workspace), ws_bytes, _stream(stream), ev)
    _check(st, "la_forward")
    return (out, S_out, z_out) if return_state else out


def la_forward(q, k, v, **kw):
    """Same as la_forward_ex without timing events."""
    kw.pop("events", None)
    return la_forward_ex(q, k, v, **kw)


def la_forward_static(q, k, v, *, feature_map="elu1", W=None, causal=True, normalize=True, S_in=None, z_in=None,
                      return_state=False, out=None, stream=None):
    """la_forward with the library's fixed device workspace (no workspace
    argument; the C call allocates nothing). Pass `out` (and call with
    return_state=False) to allocate nothing here either."""
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    fm = _fmap(feature_map, W)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if out is None:
        out = torch.empty_like(q)
    S_out = z_out = None
    if return_state:
        df = feature_dim(d, feature_map, W)
        S_out = torch.empty((B, H, df, d), device=q.device, dtype=torch.float32)
        z_out = torch.empty((B, H, df), device=q.device, dtype=torch.float32)
    st = lib.la_forward_static(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, ctypes.byref(fm), int(causal),
                               int(normalize), dt, _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                               _stream(stream))
    _check(st, "la_forward_static")
    return (out, S_out, z_out) if return_state else out


def la_decode_step(S, z, q, k, v, *, feature_map="elu1", W=None, normalize=True, out=None, stream=None):
    """One decode step on [B, H, d] tokens; S [B, H, d', d] and z [B, H, d'] are updated in place."""
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, d] shape")
    B, H, d = q.shape
    fm = _fmap(feature_map, W)
    df = feature_dim(d, feature_map, W)
    if tuple(S.shape) != (B, H, df, d) or tuple(z.shape) != (B, H, df):
        raise ValueError("state shapes must be S [B, H, d', d] and z [B, H, d']")
    if S.dtype != torch.float32 or z.dtype != torch.float32:
        raise TypeError("state must be float32")
    if out is None:
        out = torch.empty_like(q)
    st = lib.la_decode_step(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, d, ctypes.byref(fm),
                            int(normalize), _dtype_code(q), _stream(stream))
    _check(st, "la_decode_step")
    return out


def _gamma(gamma, H, device):
    if not torch.is_tensor(gamma) or gamma.dtype != torch.float32 or gamma.numel() != H:
        raise ValueError("gamma: a float32 tensor with one value per head")
    if gamma.device != device:
        raise ValueError("gamma must live on the same device as the inputs")
    return gamma.contiguous()


def la_forward_decay(q, k, v, gamma, *, feature_map="elu1", W=None, normalize=True, S_in=None, z_in=None,
                     return_state=False, out=None, workspace=None, stream=None):
    """Causal linear attention with a per-head decay gamma [H] on [B, H, N, d] tensors."""
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    g = _gamma(gamma, H, q.device)
    fm = _fmap(feature_map, W)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if out is None:
        out = torch.empty_like(q)
    S_out = z_out = None
    if return_state:
        df = feature_dim(d, feature_map, W)
        S_out = torch.empty((B, H, df, d), device=q.device, dtype=torch.float32)
        z_out = torch.empty((B, H, df), device=q.device, dtype=torch.float32)
    need = int(lib.la_forward_workspace_size(B, H, N, d, ctypes.byref(fm), 1))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.la_forward_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, ctypes.byref(fm), _ptr(g),
                              int(normalize), _dtype_code(q), _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                              _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "la_forward_decay")
    return (out, S_out, z_out) if return_state else out


def la_decode_step_decay(S, z, q, k, v, gamma, *, feature_map="elu1", W=None, normalize=True, out=None,
                         stream=None):
    """Decode step with a per-head decay gamma [H]; S, z updated in place."""
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, d] shape")
    B, H, d = q.shape
    g = _gamma(gamma, H, q.device)
    fm = _fmap(feature_map, W)
    df = feature_dim(d, feature_map, W)
    if tuple(S.shape) != (B, H, df, d) or tuple(z.shape) != (B, H, df):
        raise ValueError("state shapes must be S [B, H, d', d] and z [B, H, d']")
    if out is None:
        out = torch.empty_like(q)
    st = lib.la_decode_step_decay(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, d, ctypes.byref(fm),
                                  _ptr(g), int(normalize), _dtype_code(q), _stream(stream))
    _check(st, "la_decode_step_decay")
    return out


def la_feature_map_apply(x, *, feature_map="elu1", W=None, out_dtype=None, out=None, stream=None):
    """phi applied to each row of x [..., d]; returns [..., d']."""
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    fm = _fmap(feature_map, W)
    df = feature_dim(d, feature_map, W)
    odt = x.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(tuple(x.shape[:-1]) + (df,), device=x.device, dtype=odt)
    st = lib.la_feature_map_apply(_ptr(x), _ptr(out), rows, d, ctypes.byref(fm), _dtype_code(x), _dtype_code(out),
                                  _stream(stream))
    _check(st, "la_feature_map_apply")
    return out


def la_backward_workspace_size(B, H, N, d, feature_map="elu1") -> int:
    fm = _fmap(feature_map, None)
    return int(lib.la_backward_workspace_size(B, H, N, d, ctypes.byref(fm)))


def la_backward(q, k, v, dout, *, feature_map="elu1", normalize=True, S_in=None, z_in=None, dS_out=None,
                dz_out=None, return_state_grad=False, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Gradients of causal la_forward: returns (dq, dk, dv), or (dq, dk, dv, dS_in, dz_in)."""
    return _backward(q, k, v, dout, None, feature_map, normalize, S_in, z_in, dS_out, dz_out, return_state_grad,
                     dq, dk, dv, workspace, stream)


def la_backward_decay(q, k, v, dout, gamma, *, feature_map="elu1", normalize=True, S_in=None, z_in=None,
                      dS_out=None, dz_out=None, return_state_grad=False, dq=None, dk=None, dv=None, workspace=None,
                      stream=None):
    """Gradients of la_forward_decay (per-head decay gamma [H]): (dq, dk, dv[, dS_in, dz_in])."""
    if q.dim() != 4:
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    g = _gamma(gamma, q.shape[1], q.device)
    return _backward(q, k, v, dout, g, feature_map, normalize, S_in, z_in, dS_out, dz_out, return_state_grad,
                     dq, dk, dv, workspace, stream)


def _backward(q, k, v, dout, gamma, feature_map, normalize, S_in, z_in, dS_out, dz_out, return_state_grad, dq, dk,
              dv, workspace, stream):
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    fm = _fmap(feature_map, None)
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype or dout.dtype != q.dtype:
        raise TypeError("q, k, v, dout must share one dtype")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    dS_in = dz_in = None
    if return_state_grad:
        dS_in = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
        dz_in = torch.empty((B, H, d), device=q.device, dtype=torch.float32)
    need = int(lib.la_backward_workspace_size(B, H, N, d, ctypes.byref(fm)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if gamma is None:
        st = lib.la_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
                             ctypes.byref(fm), int(normalize), dt, _ptr(S_in), _ptr(z_in), _ptr(dS_out),
                             _ptr(dz_out), _ptr(dS_in), _ptr(dz_in), _ptr(workspace), ws_bytes, _stream(stream))
        _check(st, "la_backward")
    else:
        st = lib.la_backward_decay(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d,
                                   ctypes.byref(fm), _ptr(gamma), int(normalize), dt, _ptr(S_in), _ptr(z_in),
                                   _ptr(dS_out), _ptr(dz_out), _ptr(dS_in), _ptr(dz_in), _ptr(workspace), ws_bytes,
                                   _stream(stream))
        _check(st, "la_backward_decay")
    return (dq, dk, dv, dS_in, dz_in) if return_state_grad else (dq, dk, dv)


def la_forward_gated_workspace_size(B, H, N, d, feature_map="elu1") -> int:
    fm = _fmap(feature_map, None)
    return int(lib.la_forward_gated_workspace_size(B, H, N, d, ctypes.byref(fm)))


def _gates(g, shape, device):
    if not torch.is_tensor(g) or g.dtype != torch.float32 or tuple(g.shape) != tuple(shape):
        raise ValueError(f"log-gates: a float32 tensor of shape {tuple(shape)}")
    if g.device != device:
        raise ValueError("log-gates must live on the same device as the inputs")
    return g


def la_forward_gated(q, k, v, log_gates, *, feature_map="elu1", normalize=True, S_in=None, z_in=None,
                     return_state=False, out=None, workspace=None, stream=None):
    """Causal gated linear attention on [B, H, N, d] tensors; log_gates [B, H, N, d] float32."""
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    B, H, N, d = q.shape
    g = _gates(log_gates, q.shape, q.device)
    fm = _fmap(feature_map, None)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if out is None:
        out = torch.empty_like(q)
    S_out = z_out = None
    if return_state:
        S_out = torch.empty((B, H, d, d), device=q.device, dtype=torch.float32)
        z_out = torch.empty((B, H, d), device=q.device, dtype=torch.float32)
    need = int(lib.la_forward_gated_workspace_size(B, H, N, d, ctypes.byref(fm)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.la_forward_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, N, d, ctypes.byref(fm),
                              int(normalize), _dtype_code(q), _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                              _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "la_forward_gated")
    return (out, S_out, z_out) if return_state else out


def la_decode_step_gated(S, z, q, k, v, log_gate, *, feature_map="elu1", W=None, normalize=True, out=None,
                         stream=None):
    """Decode step with a per-feature gate: S, z updated in place; log_gate [B, H, d'] float32."""
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, d] shape")
    B, H, d = q.shape
    fm = _fmap(feature_map, W)
    df = feature_dim(d, feature_map, W)
    g = _gates(log_gate, (B, H, df), q.device)
    if tuple(S.shape) != (B, H, df, d) or tuple(z.shape) != (B, H, df):
        raise ValueError("state shapes must be S [B, H, d', d] and z [B, H, d']")
    if out is None:
        out = torch.empty_like(q)
    st = lib.la_decode_step_gated(_ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out), B, H, d,
                                  ctypes.byref(fm), int(normalize), _dtype_code(q), _stream(stream))
    _check(st, "la_decode_step_gated")
    return out
