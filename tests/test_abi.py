"""The C-ABI library: loads without a GPU, exports every declared entry point,
and rejects bad arguments synchronously, before any device work.

No compute call is made here: every call below fails validation, which the
library does before its first HIP call (fake, never dereferenced pointers).
"""
import ctypes

import pytest
import torch

import segment_wise_compressive_amd as la
from segment_wise_compressive_amd import la_strides

FAKE = 0x10000000  # 16-byte aligned, never dereferenced

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
                          "la_memory_workspace", "la_memory_fwd", "la_causal_fwd_unnormalized"}
    raw = ctypes.CDLL(la.library_path())
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(lib):
    for code in range(0, 10):
        s = la.la_status_str(code)
        assert s.startswith("LA_")
    assert "unknown" in la.la_status_str(99)
    assert la.la_version() >= 100


def test_workspace_queries(lib):
    assert la.la_causal_fwd_workspace(4, 8, 4096, 64, torch.bfloat16, 64) > 0
    assert la.la_causal_fwd_workspace(4, 8, 4096, 48, torch.bfloat16, 64) == 0   # bad d
    assert la.la_causal_fwd_workspace(4, 8, 4096, 64, torch.bfloat16, 24) == 0   # bad chunk
    inplace = la.la_causal_fwd_workspace(1, 16, 2048, 128, torch.bfloat16, 0, True)
    plain = la.la_causal_fwd_workspace(1, 16, 2048, 128, torch.bfloat16, 0, False)
    assert inplace >= plain
    assert la.la_noncausal_workspace(8, 16, 16384, 64, torch.bfloat16) > 0
    assert la.la_noncausal_workspace(8, 16, 0, 64, torch.bfloat16) == 0


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
    (dict(d=48), 5), (dict(d=16), 5), (dict(chunk=24), 5), (dict(chunk=256), 5),
    (dict(dt=7), 3),
    (dict(eps=-1.0), 6), (dict(eps=float("inf")), 6), (dict(eps=float("nan")), 6),
    (dict(N=-1), 2), (dict(B=-1), 2),
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1),
    (dict(out=None), 1),                                 # state only needs z_out or s_out
    (dict(q=FAKE + 2), 4), (dict(out=FAKE + 0x300004), 4),
    (dict(sq=la_strides(2 * 128 * 64, 128 * 64, 60)), 4),  # 120-byte row stride
    (dict(sk=la_strides(-64, 0, 64)), 2),
    (dict(ws=None), 7), (dict(ws_bytes=16), 7),
    (dict(z_in=FAKE + 0x500000, z_out=FAKE + 0x500000 + 64), 8),   # partial overlap
    (dict(s_in=FAKE + 0x500000, z_out=FAKE + 0x500000 - 256), 8),  # z_out runs into s_in
    (dict(z_in=FAKE + 0x500008), 4),
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
    assert f(*bad) == 5
    bad = list(ok); bad[0] = None
    assert f(*bad) == 1
    bad = list(ok); bad[4] = vp(FAKE + 0x3004)
    assert f(*bad) == 4
    bad = list(ok); bad[3] = 2
    assert f(*bad) == 3
    bad = list(ok); bad[10] = -1.0
    assert f(*bad) == 6


@no_device
def test_noncausal_validation(lib):
    vp = ctypes.c_void_p
    st = la_strides(2 * 64 * 64, 64 * 64, 64)
    base = [vp(FAKE), st, vp(FAKE + 0x100000), st, vp(FAKE + 0x200000), st, 1, vp(FAKE + 0x300000), st,
            1, 2, 64, 64, 1e-6, vp(FAKE + 0x400000), 1 << 30, None]
    bad = list(base); bad[12] = 96
    assert lib.la_noncausal_fwd(*bad) == 5
    bad = list(base); bad[7] = None
    assert lib.la_noncausal_fwd(*bad) == 1
    bad = list(base); bad[15] = 0
    assert lib.la_noncausal_fwd(*bad) == 7
    bad = list(base); bad[2] = vp(FAKE + 0x100002)
    assert lib.la_noncausal_fwd(*bad) == 4


@no_device
def test_unnormalized_validation(lib):
    # the unnormalised entry point shares la_causal_fwd's checks
    st = la_strides(2 * 128 * 64, 128 * 64, 64)
    vp = ctypes.c_void_p
    base = [vp(FAKE), st, vp(FAKE + 0x100000), st, vp(FAKE + 0x200000), st, 1, vp(FAKE + 0x300000), st,
            1, 2, 128, 64, 0, 1e-6, None, None, None, None, vp(FAKE + 0x400000), 1 << 30, None]
    bad = list(base); bad[12] = 48
    assert lib.la_causal_fwd_unnormalized(*bad) == 5
    bad = list(base); bad[13] = 24
    assert lib.la_causal_fwd_unnormalized(*bad) == 5
    bad = list(base); bad[7] = None
    assert lib.la_causal_fwd_unnormalized(*bad) == 1
    bad = list(base); bad[20] = 16
    assert lib.la_causal_fwd_unnormalized(*bad) == 7


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
    (dict(d=48), 5), (dict(dt=7), 3), (dict(eps=-1.0), 6), (dict(eps=float("nan")), 6),
    (dict(N=-1), 2), (dict(q=None), 1), (dict(v=None), 1),
    (dict(out=None), 1),                                 # update only needs z_out or s_out
    (dict(k=FAKE + 0x100002), 4), (dict(out=FAKE + 0x300004), 4),
    (dict(ws=None), 7), (dict(ws_bytes=16), 7),
    (dict(z_in=FAKE + 0x500000, z_out=FAKE + 0x500000 + 64), 8),
    (dict(s_in=FAKE + 0x500000, z_out=FAKE + 0x500000 - 256), 8),
    (dict(s_out=FAKE + 0x500008), 4),
])
def test_memory_validation(lib, kw, status):
    assert _memory(lib, **kw) == status


def test_memory_workspace_query(lib):
    assert la.la_memory_workspace(1, 16, 2048, 128, torch.bfloat16) > 0
    assert la.la_memory_workspace(1, 16, 0, 128, torch.bfloat16) == 0
    assert la.la_memory_workspace(1, 16, 2048, 96, torch.bfloat16) == 0


def test_binding_rejects_bad_tensors():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    with pytest.raises(TypeError):
        la.la_causal_fwd(q, q, q, torch.zeros(1, 2, 8, 64))
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        la.la_causal_fwd(q, q, q[:, :, :4], torch.zeros(1, 2, 8, 64))
    with pytest.raises(ValueError):
        la.la_causal_fwd(q, q, q, torch.zeros(1, 2, 8, 64), z_in=torch.zeros(1, 2, 64, 63))
