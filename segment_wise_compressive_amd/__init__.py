"""MI355X-native linear attention with phi(x) = elu(x) + 1.

Thin Python binding over the C ABI of ``liblinattn.so`` (declared in
``include/linattn.h``).  The functions named ``la_*`` mirror the C entry
points one to one: they only check and marshal arguments (device pointers,
strides, the current HIP stream) and raise ``LinAttnError`` on a non-OK status.
Every step of the computation runs in the library's HIP kernels; there is no
fallback of any kind, and a missing library is an error.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import functools
import os
import re
from typing import Optional, Tuple

import torch

__all__ = [
    "LinAttnError", "LA_F32", "LA_BF16", "STATUS",
    "library_path", "load_library",
    "la_status_str", "la_version",
    "la_causal_fwd_workspace", "la_causal_fwd", "la_causal_fwd_unnormalized",
    "la_causal_fwd_noalloc", "la_noalloc_scratch_bytes",
    "la_causal_bwd_workspace", "la_causal_bwd", "prepare_causal_bwd", "causal_bwd",
    "la_decode_step",
    "la_noncausal_workspace", "la_noncausal_fwd",
    "la_memory_workspace", "la_memory_fwd",
    "causal_fwd", "noncausal_fwd", "decode_step", "memory_fwd",
    "Prepared", "prepare_causal_fwd", "prepare_noncausal_fwd", "prepare_decode_step", "prepare_memory_fwd",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIBPATH = os.path.join(_HERE, "liblinattn.so")
_lib = None

LA_F32, LA_BF16 = 0, 1
# la_status values of linattn.h
STATUS = {"LA_OK": 0, "LA_ERR_NULL": -1, "LA_ERR_SHAPE": -2, "LA_ERR_DTYPE": -3, "LA_ERR_ALIGN": -4,
          "LA_ERR_UNSUPPORTED": -5, "LA_ERR_WORKSPACE": -6, "LA_ERR_LAUNCH": -7, "LA_ERR_VALUE": -8,
          "LA_ERR_ALIAS": -9}


class LinAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {la_status_str(status)} (status {status})")
        self.status = status


class la_strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("n", ctypes.c_int64)]


def library_path() -> str:
    return _LIBPATH


def load_library():
    """Load liblinattn.so (built in-tree).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIBPATH):
        raise RuntimeError(f"{_LIBPATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIBPATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    S = la_strides
    lib.la_status_str.argtypes = [i32]
    lib.la_status_str.restype = ctypes.c_char_p
    lib.la_version.argtypes = []
    lib.la_version.restype = i32
    lib.la_causal_fwd_workspace.argtypes = [i32, i32, i32, i32, i32]
    lib.la_causal_fwd_workspace.restype = sz
    lib.la_causal_fwd.argtypes = [vp, S, vp, S, vp, S, i32, vp, S, i32, i32, i32, i32, i32, f32,
                                  vp, vp, vp, vp, vp, sz, vp]
    lib.la_causal_fwd.restype = i32
    lib.la_causal_fwd_unnormalized.argtypes = lib.la_causal_fwd.argtypes
    lib.la_causal_fwd_unnormalized.restype = i32
    lib.la_causal_fwd_noalloc.argtypes = [vp, S, vp, S, vp, S, i32, vp, S, i32, i32, i32, i32, i32, f32,
                                          vp, vp, vp, vp, vp]
    lib.la_causal_fwd_noalloc.restype = i32
    lib.la_causal_bwd_workspace.argtypes = [i32, i32, i32, i32]
    lib.la_causal_bwd_workspace.restype = sz
    lib.la_causal_bwd.argtypes = [vp, S, vp, S, vp, S, i32, vp, S, vp, S, i32, i32, i32, i32, f32,
                                  vp, vp, vp, vp, vp, S, vp, S, vp, S, vp, vp, vp, sz, vp]
    lib.la_causal_bwd.restype = i32
    lib.la_noalloc_scratch_bytes.argtypes = []
    lib.la_noalloc_scratch_bytes.restype = sz
    lib.la_decode_step.argtypes = [vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, f32, vp]
    lib.la_decode_step.restype = i32
    lib.la_noncausal_workspace.argtypes = [i32, i32, i32, i32]
    lib.la_noncausal_workspace.restype = sz
    lib.la_noncausal_fwd.argtypes = [vp, S, vp, S, vp, S, i32, vp, S, i32, i32, i32, i32, f32, vp, sz, vp]
    lib.la_noncausal_fwd.restype = i32
    lib.la_memory_workspace.argtypes = [i32, i32, i32, i32]
    lib.la_memory_workspace.restype = sz
    lib.la_memory_fwd.argtypes = [vp, S, vp, S, vp, S, i32, vp, S, i32, i32, i32, i32, f32,
                                  vp, vp, vp, vp, vp, sz, vp]
    lib.la_memory_fwd.restype = i32
    _lib = lib
    return lib


# ---------------------------------------------------------------- marshalling
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return LA_F32
    if t.dtype == torch.bfloat16:
        return LA_BF16
    raise TypeError(f"q, k, v must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides(t: torch.Tensor) -> la_strides:
    if t.dim() != 4 or (t.shape[-1] > 1 and t.stride(-1) != 1):
        raise ValueError("expected a [B, H, N, d] tensor with unit stride along d")
    return la_strides(t.stride(0), t.stride(1), t.stride(2))


def _stream(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _state_check(t, shape, name):
    if t is None:
        return
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}")


# ---------------------------------------------------------------- C ABI mirrors
def la_status_str(status: int) -> str:
    return load_library().la_status_str(int(status)).decode()


def la_version() -> int:
    return int(load_library().la_version())


@functools.lru_cache(maxsize=4096)
def la_causal_fwd_workspace(B: int, H: int, N: int, d: int, chunk: int = 0) -> int:
    """Workspace bytes of la_causal_fwd / la_causal_fwd_unnormalized (0 for
    arguments the call would reject)."""
    return int(load_library().la_causal_fwd_workspace(B, H, N, d, chunk))


@functools.lru_cache(maxsize=4096)
def la_noncausal_workspace(B: int, H: int, N: int, d: int) -> int:
    """Workspace bytes of la_noncausal_fwd."""
    return int(load_library().la_noncausal_workspace(B, H, N, d))


@functools.lru_cache(maxsize=4096)
def la_memory_workspace(B: int, H: int, N: int, d: int) -> int:
    """Workspace bytes of la_memory_fwd."""
    return int(load_library().la_memory_workspace(B, H, N, d))


class Prepared:
    """A C-ABI call with every argument checked and marshalled once.

    Calling the object issues the C call with those arguments, on the stream
    given at construction or else on the stream current at call time, and
    raises LinAttnError on a non-OK status.  For loops that call the library
    repeatedly on the same buffers (serving loops, benchmarks).  The object
    keeps the tensors alive; their storage must not be reallocated.
    """

    def __init__(self, fn, args, device, where, keep):
        self._fn, self._args, self._dev, self._where, self._keep = fn, list(args), device, where, keep
        self._fixed_stream = args[-1] is not None

    def __call__(self) -> None:
        if not self._fixed_stream:
            self._args[-1] = ctypes.c_void_p(torch.cuda.current_stream(self._dev).cuda_stream)
        st = self._fn(*self._args)
        if st != 0:
            raise LinAttnError(st, self._where)


def _opt_stream(stream, device):
    return None if stream is None else _stream(stream, device)


def prepare_causal_fwd(q, k, v, out=None, *, chunk: int = 0, eps: float = 1e-6,
                       z_in=None, s_in=None, z_out=None, s_out=None,
                       workspace: Optional[torch.Tensor] = None, stream=None,
                       normalize: bool = True) -> Prepared:
    """Check and marshal a la_causal_fwd call (nothing runs until it is called).
    normalize=False marshals la_causal_fwd_unnormalized instead (same arguments).

    q, k, v: [B, H, N, d] bf16 or fp32 CUDA tensors (any strides with unit d stride).
    out: float32 [B, H, N, d] or None (state only; then q may be None).  States:
    float32 contiguous [B, H, d, d] / [B, H, d]; z_out/s_out may be the z_in/s_in
    tensors themselves.  A workspace of la_causal_fwd_workspace() bytes is
    allocated if none is given.
    """
    B, H, N, d = k.shape
    if (q is not None and tuple(q.shape) != (B, H, N, d)) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    if (q is not None and q.dtype != k.dtype) or v.dtype != k.dtype:
        raise TypeError("q, k, v must have the same dtype")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (B, H, N, d)):
        raise ValueError("out must be float32 [B, H, N, d]")
    for t, shp, nm in ((z_in, (B, H, d, d), "z_in"), (z_out, (B, H, d, d), "z_out"),
                       (s_in, (B, H, d), "s_in"), (s_out, (B, H, d), "s_out")):
        _state_check(t, shp, nm)
    ws_bytes = la_causal_fwd_workspace(B, H, N, d, chunk)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=k.device)
    have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    so = _strides(out) if out is not None else la_strides(0, 0, 0)
    sq = _strides(q) if q is not None else la_strides(0, 0, 0)
    args = [_ptr(q), sq, _ptr(k), _strides(k), _ptr(v), _strides(v), _dtype_code(k),
            _ptr(out), so, B, H, N, d, int(chunk), ctypes.c_float(eps),
            _ptr(z_in), _ptr(s_in), _ptr(z_out), _ptr(s_out), _ptr(workspace), ctypes.c_size_t(have),
            _opt_stream(stream, k.device)]
    lib = load_library()
    fn, name = (lib.la_causal_fwd, "la_causal_fwd") if normalize else \
        (lib.la_causal_fwd_unnormalized, "la_causal_fwd_unnormalized")
    return Prepared(fn, args, k.device, name, (q, k, v, out, z_in, s_in, z_out, s_out, workspace))


def la_causal_fwd(q, k, v, out=None, *, chunk: int = 0, eps: float = 1e-6,
                  z_in=None, s_in=None, z_out=None, s_out=None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Causal linear attention forward (la_causal_fwd in linattn.h); arguments
    as for prepare_causal_fwd."""
    prepare_causal_fwd(q, k, v, out, chunk=chunk, eps=eps, z_in=z_in, s_in=s_in, z_out=z_out, s_out=s_out,
                       workspace=workspace, stream=stream)()


def la_causal_fwd_unnormalized(q, k, v, out=None, *, chunk: int = 0, eps: float = 1e-6,
                               z_in=None, s_in=None, z_out=None, s_out=None,
                               workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Causal linear attention without the normaliser (la_causal_fwd_unnormalized
    in linattn.h); arguments as for prepare_causal_fwd."""
    prepare_causal_fwd(q, k, v, out, chunk=chunk, eps=eps, z_in=z_in, s_in=s_in, z_out=z_out, s_out=s_out,
                       workspace=workspace, stream=stream, normalize=False)()


def la_noalloc_scratch_bytes() -> int:
    """Bytes of the per-GPU scratch array behind la_causal_fwd_noalloc."""
    return int(load_library().la_noalloc_scratch_bytes())


def la_causal_fwd_noalloc(q, k, v, out=None, *, chunk: int = 0, eps: float = 1e-6,
                          z_in=None, s_in=None, z_out=None, s_out=None, stream=None) -> None:
    """la_causal_fwd_noalloc in linattn.h: la_causal_fwd with the library's
    fixed per-GPU scratch array instead of a workspace (allocates nothing;
    calls that overlap on one GPU race).  Arguments as for prepare_causal_fwd."""
    B, H, N, d = k.shape
    if (q is not None and tuple(q.shape) != (B, H, N, d)) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    if (q is not None and q.dtype != k.dtype) or v.dtype != k.dtype:
        raise TypeError("q, k, v must have the same dtype")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (B, H, N, d)):
        raise ValueError("out must be float32 [B, H, N, d]")
    for t, shp, nm in ((z_in, (B, H, d, d), "z_in"), (z_out, (B, H, d, d), "z_out"),
                       (s_in, (B, H, d), "s_in"), (s_out, (B, H, d), "s_out")):
        _state_check(t, shp, nm)
    so = _strides(out) if out is not None else la_strides(0, 0, 0)
    sq = _strides(q) if q is not None else la_strides(0, 0, 0)
    st = load_library().la_causal_fwd_noalloc(
        _ptr(q), sq, _ptr(k), _strides(k), _ptr(v), _strides(v), _dtype_code(k),
        _ptr(out), so, B, H, N, d, int(chunk), ctypes.c_float(eps),
        _ptr(z_in), _ptr(s_in), _ptr(z_out), _ptr(s_out), _stream(stream, k.device))
    if st != 0:
        raise LinAttnError(st, "la_causal_fwd_noalloc")


@functools.lru_cache(maxsize=4096)
def la_causal_bwd_workspace(B: int, H: int, N: int, d: int) -> int:
    """Workspace bytes of la_causal_bwd."""
    return int(load_library().la_causal_bwd_workspace(B, H, N, d))


def prepare_causal_bwd(q, k, v, out, dout, dq, dk, dv, *, eps: float = 1e-6,
                       z_in=None, s_in=None, dz_out=None, ds_out=None, dz_in=None, ds_in=None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> Prepared:
    """Check and marshal a la_causal_bwd call (nothing runs until it is called).

    q, k, v: the forward call's inputs; out: its float32 output; dout: float32
    gradient of out; dq, dk, dv: float32 [B, H, N, d] results (any strides with
    unit d stride).  States and their gradients: float32 contiguous.
    """
    B, H, N, d = q.shape
    for t, nm in ((k, "k"), (v, "v")):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{nm} must match q in shape and dtype")
    for t, nm in ((out, "out"), (dout, "dout"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{nm} must be float32 [B, H, N, d]")
    for t, shp, nm in ((z_in, (B, H, d, d), "z_in"), (dz_out, (B, H, d, d), "dz_out"), (dz_in, (B, H, d, d), "dz_in"),
                       (s_in, (B, H, d), "s_in"), (ds_out, (B, H, d), "ds_out"), (ds_in, (B, H, d), "ds_in")):
        _state_check(t, shp, nm)
    ws_bytes = la_causal_bwd_workspace(B, H, N, d)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), _dtype_code(q),
            _ptr(out), _strides(out), _ptr(dout), _strides(dout), B, H, N, d, ctypes.c_float(eps),
            _ptr(z_in), _ptr(s_in), _ptr(dz_out), _ptr(ds_out),
            _ptr(dq), _strides(dq), _ptr(dk), _strides(dk), _ptr(dv), _strides(dv), _ptr(dz_in), _ptr(ds_in),
            _ptr(workspace), ctypes.c_size_t(have), _opt_stream(stream, q.device)]
    return Prepared(load_library().la_causal_bwd, args, q.device, "la_causal_bwd",
                    (q, k, v, out, dout, dq, dk, dv, z_in, s_in, dz_out, ds_out, dz_in, ds_in, workspace))


def la_causal_bwd(q, k, v, out, dout, dq, dk, dv, **kw) -> None:
    """Backward pass of the causal form (la_causal_bwd in linattn.h); arguments
    as for prepare_causal_bwd."""
    prepare_causal_bwd(q, k, v, out, dout, dq, dk, dv, **kw)()


def causal_bwd(q, k, v, out, dout, *, eps: float = 1e-6, state=None, dstate=None, want_dstate: bool = False):
    """(dq, dk, dv) of causal linear attention, plus (dz_in, ds_in) when
    want_dstate.  state: the forward call's (z_in, s_in); dstate: the
    gradient (dz_out, ds_out) reaching its final state."""
    B, H, N, d = q.shape
    dq, dk, dv = (torch.empty(B, H, N, d, dtype=torch.float32, device=q.device) for _ in range(3))
    z_in, s_in = state if state is not None else (None, None)
    dz_out, ds_out = dstate if dstate is not None else (None, None)
    dz_in = ds_in = None
    if want_dstate:
        dz_in = torch.empty(B, H, d, d, dtype=torch.float32, device=q.device)
        ds_in = torch.empty(B, H, d, dtype=torch.float32, device=q.device)
    la_causal_bwd(q, k, v, out, dout, dq, dk, dv, eps=eps, z_in=z_in, s_in=s_in, dz_out=dz_out, ds_out=ds_out,
                  dz_in=dz_in, ds_in=ds_in)
    return (dq, dk, dv, dz_in, ds_in) if want_dstate else (dq, dk, dv)


def prepare_decode_step(q, k, v, z, s, out, *, eps: float = 1e-6, stream=None) -> Prepared:
    """Check and marshal a la_decode_step call (nothing runs until it is called).

    q, k, v: contiguous [B, H, d]; z float32 [B, H, d, d]; s float32 [B, H, d];
    out float32 [B, H, d].  Each call updates z and s in place.
    """
    B, H, d = q.shape
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        if tuple(t.shape) != (B, H, d) or not t.is_contiguous() or t.dtype != q.dtype:
            raise ValueError(f"{nm} must be a contiguous [B, H, d] tensor of q's dtype")
    _state_check(z, (B, H, d, d), "z")
    _state_check(s, (B, H, d), "s")
    _state_check(out, (B, H, d), "out")
    args = [_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(z), _ptr(s), _ptr(out), B, H, d,
            ctypes.c_float(eps), _opt_stream(stream, q.device)]
    return Prepared(load_library().la_decode_step, args, q.device, "la_decode_step", (q, k, v, z, s, out))


def la_decode_step(q, k, v, z, s, out, *, eps: float = 1e-6, stream=None) -> None:
    """One recurrent step per head; z, s updated in place (la_decode_step in linattn.h)."""
    prepare_decode_step(q, k, v, z, s, out, eps=eps, stream=stream)()


def prepare_noncausal_fwd(q, k, v, out, *, eps: float = 1e-6,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> Prepared:
    """Check and marshal a la_noncausal_fwd call (nothing runs until it is called)."""
    B, H, N, d = q.shape
    if tuple(k.shape) != (B, H, N, d) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must have the same dtype")
    if out.dtype != torch.float32 or tuple(out.shape) != (B, H, N, d):
        raise ValueError("out must be float32 [B, H, N, d]")
    ws_bytes = la_noncausal_workspace(B, H, N, d)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), _dtype_code(q),
            _ptr(out), _strides(out), B, H, N, d, ctypes.c_float(eps), _ptr(workspace), ctypes.c_size_t(have),
            _opt_stream(stream, q.device)]
    return Prepared(load_library().la_noncausal_fwd, args, q.device, "la_noncausal_fwd", (q, k, v, out, workspace))


def la_noncausal_fwd(q, k, v, out, *, eps: float = 1e-6,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Non-causal linear attention forward (la_noncausal_fwd in linattn.h)."""
    prepare_noncausal_fwd(q, k, v, out, eps=eps, workspace=workspace, stream=stream)()


def prepare_memory_fwd(q, k, v, out=None, *, eps: float = 1e-6,
                       z_in=None, s_in=None, z_out=None, s_out=None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> Prepared:
    """Check and marshal a la_memory_fwd call (nothing runs until it is called).

    q, k, v: [B, H, N, d] bf16 or fp32 CUDA tensors (unit d stride); out:
    float32 [B, H, N, d] or None (update only).  Memory: float32 contiguous
    [B, H, d, d] / [B, H, d]; z_out/s_out may be the z_in/s_in tensors themselves.
    """
    B, H, N, d = q.shape
    if tuple(k.shape) != (B, H, N, d) or tuple(v.shape) != (B, H, N, d):
        raise ValueError("q, k, v must have the same shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must have the same dtype")
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != (B, H, N, d)):
        raise ValueError("out must be float32 [B, H, N, d]")
    for t, shp, nm in ((z_in, (B, H, d, d), "z_in"), (z_out, (B, H, d, d), "z_out"),
                       (s_in, (B, H, d), "s_in"), (s_out, (B, H, d), "s_out")):
        _state_check(t, shp, nm)
    ws_bytes = la_memory_workspace(B, H, N, d)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    so = _strides(out) if out is not None else la_strides(0, 0, 0)
    args = [_ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v), _dtype_code(q),
            _ptr(out), so, B, H, N, d, ctypes.c_float(eps),
            _ptr(z_in), _ptr(s_in), _ptr(z_out), _ptr(s_out), _ptr(workspace), ctypes.c_size_t(have),
            _opt_stream(stream, q.device)]
    return Prepared(load_library().la_memory_fwd, args, q.device, "la_memory_fwd",
                    (q, k, v, out, z_in, s_in, z_out, s_out, workspace))


def la_memory_fwd(q, k, v, out=None, *, eps: float = 1e-6,
                  z_in=None, s_in=None, z_out=None, s_out=None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> None:
    """Compressive memory of one segment (la_memory_fwd in linattn.h); arguments
    as for prepare_memory_fwd."""
    prepare_memory_fwd(q, k, v, out, eps=eps, z_in=z_in, s_in=s_in, z_out=z_out, s_out=s_out,
                       workspace=workspace, stream=stream)()


# ---------------------------------------------------------------- conveniences
def causal_fwd(q, k, v, *, eps: float = 1e-6, chunk: int = 0,
               state: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
               return_state: bool = False):
    """out = causal linear attention of (q, k, v), optionally carrying (Z, S)."""
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=q.device)
    z_in, s_in = state if state is not None else (None, None)
    z_out = s_out = None
    if return_state:
        z_out = torch.empty(B, H, d, d, dtype=torch.float32, device=q.device)
        s_out = torch.empty(B, H, d, dtype=torch.float32, device=q.device)
    la_causal_fwd(q, k, v, out, chunk=chunk, eps=eps, z_in=z_in, s_in=s_in, z_out=z_out, s_out=s_out)
    return (out, (z_out, s_out)) if return_state else out


def noncausal_fwd(q, k, v, *, eps: float = 1e-6):
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=q.device)
    la_noncausal_fwd(q, k, v, out, eps=eps)
    return out


def decode_step(q, k, v, z, s, *, eps: float = 1e-6):
    """One generation step; z and s are updated in place.  Returns out [B, H, d]."""
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    la_decode_step(q, k, v, z, s, out, eps=eps)
    return out


def memory_fwd(q, k, v, memory: Optional[Tuple[torch.Tensor, torch.Tensor]] = None, *, eps: float = 1e-6):
    """Reads of one segment from the memory of earlier segments, and the
    memory after the segment: returns (out, (z, s))."""
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=q.device)
    z_in, s_in = memory if memory is not None else (None, None)
    z_out = torch.empty(B, H, d, d, dtype=torch.float32, device=q.device)
    s_out = torch.empty(B, H, d, dtype=torch.float32, device=q.device)
    la_memory_fwd(q, k, v, out, eps=eps, z_in=z_in, s_in=s_in, z_out=z_out, s_out=s_out)
    return out, (z_out, s_out)


def declared_entry_points(header: Optional[str] = None):
    """Names of the functions declared in include/linattn.h."""
    header = header or os.path.join(os.path.dirname(_HERE), "include", "linattn.h")
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(la_\w+)\s*\(", text, re.M)))
