"""The C-ABI library: loads without a GPU, exports every declared entry point,
and rejects bad arguments synchronously, before any device work.

No compute call is made here: every call below fails validation, which the
library does before its first HIP call (fake, never dereferenced pointers).
"""
import ctypes
import os

import pytest
import torch

import segment_wise_compressive_amd as la
from segment_wise_compressive_amd import la_strides

FAKE = 0x10000000  # 16-byte aligned, never dereferenced
# la_status values (linattn.h)
NULL_, SHAPE, DTYPE, ALIGN, UNSUP, WS, LAUNCH, VALUE, ALIAS = (la.STATUS[n] for n in (
    "LA_ERR_NULL", "LA_ERR_SHAPE", "LA_ERR_DTYPE", "LA_ERR_ALIGN", "LA_ERR_UNSUPPORTED", "LA_ERR_WORKSPACE",
    "LA_ERR_LAUNCH", "LA_ERR_VALUE", "LA_ERR_ALIAS"))

# Calls with fake pointers must never reach a device: these tests only run
# where there is none.
no_device = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer validation tests run without a GPU")


@pytest.fixture(scope="module")
def lib():
    return la.load_library()


def test_exports_every_declared_symbol(lib):
    names = la.declared_entry_points()
    assert set(names) == {"la_status_str", "la_version", "la_causal_fwd_workspace", "la_causal_fwd",
                          "la_decode_step", "la_noncausal_workspace", "la_noncausal_fwd",
                          "la_memory_workspace", "la_memory_fwd", "la_causal_fwd_unnormalized",
                          "la_causal_fwd_noalloc", "la_noalloc_scratch_bytes",
                          "la_causal_bwd_workspace", "la_causal_bwd"}
    raw = ctypes.CDLL(la.library_path())
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(lib):
    # the values of the header's enum, each with its own text
    header = open(os.path.join(os.path.dirname(os.path.dirname(la.__file__)), "include", "linattn.h")).read()
    for name, code in la.STATUS.items():
        assert f"{name} = {code}" in header, name
        s = la.la_status_str(code)
        assert s.startswith(name), (name, s)
    assert sorted(la.STATUS.values()) == list(range(-9, 1))
    assert "unknown" in la.la_status_str(99)
    assert la.la_version() >= 100


def test_workspace_queries(lib):
    assert la.la_causal_fwd_workspace(4, 8, 4096, 64, 64) > 0
    assert la.la_causal_fwd_workspace(4, 8, 4096, 48, 64) == 0   # bad d
    assert la.la_causal_fwd_workspace(4, 8, 4096, 64, 24) == 0   # bad chunk
    assert la.la_causal_fwd_workspace(4, 8, 0, 64) == 0          # N = 0 needs none
    # the status block (give-up counter) comes first in every causal workspace
    assert la.la_causal_fwd_workspace(1, 1, 1, 32) >= 256
    assert la.la_noncausal_workspace(8, 16, 16384, 64) > 0
    assert la.la_noncausal_workspace(8, 16, 0, 64) == 0


def _causal(lib, **kw):
    B, H, N, d = kw.get("B", 1), kw.get("H", 2), kw.get("N", 128), kw.get("d", 64)
    st = la_strides(H * N * d, N * d, d)
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, dt=la.LA_BF16, out=FAKE + 0x300000,
                so=st, chunk=0, eps=1e-6, z_in=None, s_in=None, z_out=None, s_out=None,
                ws=FAKE + 0x400000, ws_bytes=1 << 30, sq=st, sk=st, sv=st)
    args.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.la_causal_fwd(vp(args["q"]), args["sq"], vp(args["k"]), args["sk"], vp(args["v"]), args["sv"],
                             args["dt"], vp(args["out"]), args["so"], B, H, N, d, args["chunk"], args["eps"],
                             vp(args["z_in"]), vp(args["s_in"]), vp(args["z_out"]), vp(args["s_out"]),
                             vp(args["ws"]), args["ws_bytes"], None)


@no_device
@pytest.mark.parametrize("kw, status", [
    (dict(d=48), UNSUP), (dict(d=16), UNSUP), (dict(chunk=24), UNSUP), (dict(chunk=256), UNSUP),
    (dict(dt=7), DTYPE),
    (dict(eps=-1.0), VALUE), (dict(eps=float("inf")), VALUE), (dict(eps=float("nan")), VALUE),
    (dict(N=-1), SHAPE), (dict(B=-1), SHAPE),
    (dict(q=None), NULL_), (dict(k=None), NULL_), (dict(v=None), NULL_),
    (dict(out=None), NULL_),                             # state only needs z_out or s_out
    (dict(out=None, q=None, k=None, z_out=FAKE + 0x500000), NULL_),  # state only still needs k
    (dict(out=None, q=None, k=FAKE + 0x100002, z_out=FAKE + 0x500000), ALIGN),
    (dict(q=FAKE + 2), ALIGN), (dict(out=FAKE + 0x300004), ALIGN),
    (dict(sq=la_strides(2 * 128 * 64, 128 * 64, 60)), ALIGN),  # 120-byte row stride
    (dict(sk=la_strides(-64, 0, 64)), SHAPE),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS),
    (dict(z_in=FAKE + 0x500000, z_out=FAKE + 0x500000 + 64), ALIAS),   # partial overlap
    (dict(s_in=FAKE + 0x500000, z_out=FAKE + 0x500000 - 256), ALIAS),  # z_out runs into s_in
    (dict(z_in=FAKE + 0x500008), ALIGN),
])
def test_causal_validation(lib, kw, status):
    assert _causal(lib, **kw) == status


@no_device
def test_decode_validation(lib):
    vp = ctypes.c_void_p
    f = lambda *a: lib.la_decode_step(*a)
    ok = [vp(FAKE), vp(FAKE + 0x1000), vp(FAKE + 0x2000), 1, vp(FAKE + 0x3000), vp(FAKE + 0x100000),
          vp(FAKE + 0x200000), 2, 3, 64, 1e-6, None]
    bad = list(ok); bad[9] = 100
    assert f(*bad) == UNSUP
    bad = list(ok); bad[0] = None
    assert f(*bad) == NULL_
    bad = list(ok); bad[4] = vp(FAKE + 0x3004)
    assert f(*bad) == ALIGN
    bad = list(ok); bad[3] = 2
    assert f(*bad) == DTYPE
    bad = list(ok); bad[10] = -1.0
    assert f(*bad) == VALUE


@no_device
def test_noncausal_validation(lib):
    vp = ctypes.c_void_p
    st = la_strides(2 * 64 * 64, 64 * 64, 64)
    base = [vp(FAKE), st, vp(FAKE + 0x100000), st, vp(FAKE + 0x200000), st, 1, vp(FAKE + 0x300000), st,
            1, 2, 64, 64, 1e-6, vp(FAKE + 0x400000), 1 << 30, None]
    bad = list(base); bad[12] = 96
    assert lib.la_noncausal_fwd(*bad) == UNSUP
    bad = list(base); bad[7] = None
    assert lib.la_noncausal_fwd(*bad) == NULL_
    bad = list(base); bad[15] = 0
    assert lib.la_noncausal_fwd(*bad) == WS
    bad = list(base); bad[2] = vp(FAKE + 0x100002)
    assert lib.la_noncausal_fwd(*bad) == ALIGN


@no_device
def test_unnormalized_validation(lib):
    # the unnormalised entry point shares la_causal_fwd's checks
    st = la_strides(2 * 128 * 64, 128 * 64, 64)
    vp = ctypes.c_void_p
    base = [vp(FAKE), st, vp(FAKE + 0x100000), st, vp(FAKE + 0x200000), st, 1, vp(FAKE + 0x300000), st,
            1, 2, 128, 64, 0, 1e-6, None, None, None, None, vp(FAKE + 0x400000), 1 << 30, None]
    bad = list(base); bad[12] = 48
    assert lib.la_causal_fwd_unnormalized(*bad) == UNSUP
    bad = list(base); bad[13] = 24
    assert lib.la_causal_fwd_unnormalized(*bad) == UNSUP
    bad = list(base); bad[7] = None
    assert lib.la_causal_fwd_unnormalized(*bad) == NULL_
    bad = list(base); bad[20] = 16
    assert lib.la_causal_fwd_unnormalized(*bad) == WS


def _memory(lib, **kw):
    B, H, N, d = kw.get("B", 1), kw.get("H", 2), kw.get("N", 128), kw.get("d", 64)
    st = la_strides(H * N * d, N * d, d)
    args = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, dt=la.LA_BF16, out=FAKE + 0x300000,
                so=st, eps=1e-6, z_in=None, s_in=None, z_out=None, s_out=None,
                ws=FAKE + 0x400000, ws_bytes=1 << 30, sq=st, sk=st, sv=st)
    args.update(kw)
    vp = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.la_memory_fwd(vp(args["q"]), args["sq"], vp(args["k"]), args["sk"], vp(args["v"]), args["sv"],
                             args["dt"], vp(args["out"]), args["so"], B, H, N, d, args["eps"],
                             vp(args["z_in"]), vp(args["s_in"]), vp(args["z_out"]), vp(args["s_out"]),
                             vp(args["ws"]), args["ws_bytes"], None)


@no_device
@pytest.mark.parametrize("kw, status", [
    (dict(d=48), UNSUP), (dict(dt=7), DTYPE), (dict(eps=-1.0), VALUE), (dict(eps=float("nan")), VALUE),
    (dict(N=-1), SHAPE), (dict(q=None), NULL_), (dict(v=None), NULL_),
    (dict(out=None), NULL_),                             # update only needs z_out or s_out
    (dict(k=FAKE + 0x100002), ALIGN), (dict(out=FAKE + 0x300004), ALIGN),
    (dict(ws=None), WS), (dict(ws_bytes=16), WS),
    (dict(z_in=FAKE + 0x500000, z_out=FAKE + 0x500000 + 64), ALIAS),
    (dict(s_in=FAKE + 0x500000, z_out=FAKE + 0x500000 - 256), ALIAS),
    (dict(s_out=FAKE + 0x500008), ALIGN),
])
def test_memory_validation(lib, kw, status):
    assert _memory(lib, **kw) == status


def test_memory_workspace_query(lib):
    assert la.la_memory_workspace(1, 16, 2048, 128) > 0
    assert la.la_memory_workspace(1, 16, 0, 128) == 0
    assert la.la_memory_workspace(1, 16, 2048, 96) == 0


def test_binding_rejects_bad_tensors():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(TypeError):
        la.la_causal_fwd(q, q, q, torch.zeros(1, 2, 8, 64))
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        la.la_causal_fwd(q, q, q[:, :, :4], torch.zeros(1, 2, 8, 64))
    with pytest.raises(ValueError):
        la.la_causal_fwd(q, q, q, torch.zeros(1, 2, 8, 64), z_in=torch.zeros(1, 2, 64, 63))


def test_noalloc_scratch_size(lib):
    assert la.la_noalloc_scratch_bytes() == 32 << 20


@no_device
def test_noalloc_validation(lib):
    # the allocation-free entry point checks as la_causal_fwd does, and
    # rejects a call whose workspace would not fit in the scratch array
    vp = ctypes.c_void_p

    def call(B=1, H=2, N=128, d=64, out=FAKE + 0x300000, q=FAKE, eps=1e-6):
        st = la_strides(H * N * d, N * d, d)
        return lib.la_causal_fwd_noalloc(None if q is None else vp(q), st, vp(FAKE + 0x100000), st,
                                         vp(FAKE + 0x200000), st, la.LA_BF16, None if out is None else vp(out),
                                         st, B, H, N, d, 0, eps, None, None, None, None, None)
    assert call(d=48) == UNSUP
    assert call(q=None) == NULL_
    assert call(eps=-1.0) == VALUE
    big = (1, 1024, 4096, 128)
    assert la.la_causal_fwd_workspace(*big) > la.la_noalloc_scratch_bytes()
    assert call(*big) == WS


@no_device
def test_backward_validation(lib):
    vp = ctypes.c_void_p
    B, H, N, d = 1, 2, 128, 64
    st = la_strides(H * N * d, N * d, d)

    def call(**kw):
        p = dict(q=FAKE, k=FAKE + 0x100000, v=FAKE + 0x200000, out=FAKE + 0x300000, dout=FAKE + 0x400000,
                 dq=FAKE + 0x500000, dk=FAKE + 0x600000, dv=FAKE + 0x700000, dz_in=None, ds_in=None,
                 ws=FAKE + 0x800000, ws_bytes=1 << 30, d=d, eps=1e-6, dt=la.LA_BF16)
        p.update(kw)
        x = lambda a: None if a is None else vp(a)
        return lib.la_causal_bwd(x(p["q"]), st, x(p["k"]), st, x(p["v"]), st, p["dt"], x(p["out"]), st,
                                 x(p["dout"]), st, B, H, N, p["d"], p["eps"], None, None, None, None,
                                 x(p["dq"]), st, x(p["dk"]), st, x(p["dv"]), st, x(p["dz_in"]), x(p["ds_in"]),
                                 x(p["ws"]), p["ws_bytes"], None)
    assert call(d=48) == UNSUP
    assert call(dt=5) == DTYPE
    assert call(eps=-1.0) == VALUE
    assert call(dout=None) == NULL_
    assert call(dv=None) == NULL_
    assert call(dk=FAKE + 0x600004) == ALIGN
    assert call(dq=FAKE + 0x100000) == ALIAS          # dq over k
    assert call(dk=FAKE + 0x500000 + 64) == ALIAS     # dk over dq
    assert call(ws=None) == WS
    assert call(ws_bytes=64) == WS
    assert la.la_causal_bwd_workspace(B, H, N, d) > 0
    assert la.la_causal_bwd_workspace(B, H, 0, d) == 0
