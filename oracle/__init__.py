"""fp64 CPU oracle for linear attention with phi(x) = elu(x) + 1.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this package.  It shares no
code with the HIP library: the arithmetic lives in ``linattn_oracle.c`` (plain
C, double precision, OpenMP over heads), which this module builds with gcc and
calls through ctypes.

Every function takes NumPy/torch CPU arrays laid out [BH, N, d] (or [BH, d]
for the decode step), converts them to contiguous float32 (exact for bf16 and
fp32 inputs) and returns float64 results.  Citations of the defining passages
are in the C source, next to each function.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# The mutation tests point this at deliberately broken builds of the oracle.
_LIB = os.environ.get("LINATTN_ORACLE_LIB_OVERRIDE", _LIB)
_lib = None


def build(force: bool = True) -> str:
    """Compile linattn_oracle.c into liboracle.so with gcc (-O2, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        fp = ctypes.POINTER(ctypes.c_float)
        L, D = ctypes.c_long, ctypes.c_double
        lib.oracle_causal.argtypes = [L, L, L, D, fp, fp, fp, dp, dp, dp, dp, dp]
        lib.oracle_causal.restype = None
        lib.oracle_decode_step.argtypes = [L, L, D, fp, fp, fp, dp, dp, dp]
        lib.oracle_decode_step.restype = None
        lib.oracle_noncausal.argtypes = [L, L, L, D, fp, fp, fp, dp, dp, dp]
        lib.oracle_noncausal.restype = None
        lib.oracle_memory.argtypes = [L, L, L, D, fp, fp, fp, dp, dp, dp, dp, dp]
        lib.oracle_memory.restype = None
        lib.oracle_causal_unnormalized.argtypes = [L, L, L, fp, fp, fp, dp, dp]
        lib.oracle_causal_unnormalized.restype = None
        lib.oracle_causal_bwd.argtypes = [L, L, L, D, fp, fp, fp, fp, dp, dp, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_causal_bwd.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor (CPU); bf16 -> float32 is exact
        x = x.detach().float().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().double().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _fptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _dptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def causal(q, k, v, eps: float, z_in=None, s_in=None, want_out: bool = True):
    """Causal linear attention, recurrent form.

    q, k, v: [..., N, d] (leading dims flattened to heads).
    z_in: [..., d, d] or None; s_in: [..., d] or None.
    Returns (out [..., N, d] or None, z_out [..., d, d], s_out [..., d]) in float64.
    """
    qa, ka, va = _f32(q), _f32(k), _f32(v)
    lead, (N, d) = qa.shape[:-2], qa.shape[-2:]
    BH = int(np.prod(lead)) if lead else 1
    zi = None if z_in is None else _f64(z_in).reshape(BH, d, d)
    si = None if s_in is None else _f64(s_in).reshape(BH, d)
    out = np.empty((BH, N, d), np.float64) if want_out else None
    zo = np.empty((BH, d, d), np.float64)
    so = np.empty((BH, d), np.float64)
    _load().oracle_causal(BH, N, d, float(eps), _fptr(qa), _fptr(ka), _fptr(va),
                          _dptr(zi), _dptr(si), _dptr(out), _dptr(zo), _dptr(so))
    return (None if out is None else out.reshape(*lead, N, d),
            zo.reshape(*lead, d, d), so.reshape(*lead, d))


def decode_step(q, k, v, z, s, eps: float):
    """One recurrent step per head.  q, k, v: [..., d]; z: [..., d, d]; s: [..., d].

    Returns (out [..., d], z_new, s_new) in float64; the inputs are not modified.
    """
    qa, ka, va = _f32(q), _f32(k), _f32(v)
    lead, d = qa.shape[:-1], qa.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    zz = _f64(z).reshape(BH, d, d).copy()
    ss = _f64(s).reshape(BH, d).copy()
    out = np.empty((BH, d), np.float64)
    _load().oracle_decode_step(BH, d, float(eps), _fptr(qa), _fptr(ka), _fptr(va),
                               _dptr(zz), _dptr(ss), _dptr(out))
    return out.reshape(*lead, d), zz.reshape(*lead, d, d), ss.reshape(*lead, d)


def noncausal(q, k, v, eps: float, want_out: bool = True):
    """Non-causal linear attention.  Returns (out or None, z, s) in float64."""
    qa, ka, va = _f32(q), _f32(k), _f32(v)
    lead, (N, d) = qa.shape[:-2], qa.shape[-2:]
    BH = int(np.prod(lead)) if lead else 1
    out = np.empty((BH, N, d), np.float64) if want_out else None
    zo = np.empty((BH, d, d), np.float64)
    so = np.empty((BH, d), np.float64)
    _load().oracle_noncausal(BH, N, d, float(eps), _fptr(qa), _fptr(ka), _fptr(va),
                             _dptr(out), _dptr(zo), _dptr(so))
    return (None if out is None else out.reshape(*lead, N, d),
            zo.reshape(*lead, d, d), so.reshape(*lead, d))


def memory(q, k, v, eps: float, z_in=None, s_in=None, want_out: bool = True):
    """Compressive memory of one segment: every query reads (z_in, s_in), the
    memory left by earlier segments; then the segment's keys and values are
    added.  Returns (out [..., N, d] or None, z_out [..., d, d], s_out [..., d])
    in float64."""
    qa, ka, va = _f32(q), _f32(k), _f32(v)
    lead, (N, d) = qa.shape[:-2], qa.shape[-2:]
    BH = int(np.prod(lead)) if lead else 1
    zi = None if z_in is None else _f64(z_in).reshape(BH, d, d)
    si = None if s_in is None else _f64(s_in).reshape(BH, d)
    out = np.empty((BH, N, d), np.float64) if want_out else None
    zo = np.empty((BH, d, d), np.float64)
    so = np.empty((BH, d), np.float64)
    _load().oracle_memory(BH, N, d, float(eps), _fptr(qa), _fptr(ka), _fptr(va),
                          _dptr(zi), _dptr(si), _dptr(out), _dptr(zo), _dptr(so))
    return (None if out is None else out.reshape(*lead, N, d),
            zo.reshape(*lead, d, d), so.reshape(*lead, d))


def causal_unnormalized(q, k, v, z_in=None):
    """Causal linear attention without the normaliser: out_t = phi(q_t)^T Z_t
    with Z_t = z_in + sum_{i<=t} phi(k_i) v_i^T.  Returns out [..., N, d] in
    float64 (the carried state is the same as oracle.causal's)."""
    qa, ka, va = _f32(q), _f32(k), _f32(v)
    lead, (N, d) = qa.shape[:-2], qa.shape[-2:]
    BH = int(np.prod(lead)) if lead else 1
    zi = None if z_in is None else _f64(z_in).reshape(BH, d, d)
    out = np.empty((BH, N, d), np.float64)
    _load().oracle_causal_unnormalized(BH, N, d, _fptr(qa), _fptr(ka), _fptr(va), _dptr(zi), _dptr(out))
    return out.reshape(*lead, N, d)


def causal_bwd(q, k, v, dout, eps: float, z_in=None, s_in=None, dz_out=None, ds_out=None):
    """Gradients of oracle.causal: for the upstream gradient dout [..., N, d]
    (and dz_out [..., d, d], ds_out [..., d] reaching the final state; None =
    zeros), returns (dq, dk, dv [..., N, d], dz_in [..., d, d], ds_in [..., d])
    in float64.  dout is read as float32 (the values a GPU call sees)."""
    qa, ka, va, da = _f32(q), _f32(k), _f32(v), _f32(dout)
    lead, (N, d) = qa.shape[:-2], qa.shape[-2:]
    BH = int(np.prod(lead)) if lead else 1
    zi = None if z_in is None else _f64(z_in).reshape(BH, d, d)
    si = None if s_in is None else _f64(s_in).reshape(BH, d)
    dzo = None if dz_out is None else _f64(dz_out).reshape(BH, d, d)
    dso = None if ds_out is None else _f64(ds_out).reshape(BH, d)
    dq = np.empty((BH, N, d), np.float64)
    dk = np.empty((BH, N, d), np.float64)
    dv = np.empty((BH, N, d), np.float64)
    dzi = np.empty((BH, d, d), np.float64)
    dsi = np.empty((BH, d), np.float64)
    _load().oracle_causal_bwd(BH, N, d, float(eps), _fptr(qa), _fptr(ka), _fptr(va), _fptr(da),
                              _dptr(zi), _dptr(si), _dptr(dzo), _dptr(dso),
                              _dptr(dq), _dptr(dk), _dptr(dv), _dptr(dzi), _dptr(dsi))
    sh = lambda a: a.reshape(*lead, N, d)
    return sh(dq), sh(dk), sh(dv), dzi.reshape(*lead, d, d), dsi.reshape(*lead, d)
