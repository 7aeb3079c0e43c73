"""GPU parity of la_memory_fwd (compressive memory of one segment: every
query reads the memory left by earlier segments, then the segment is added)
against the fp64 oracle, through the C ABI.

Tolerances as for the other entry points: row-wise relative error of 2e-3
for bf16 inputs and 1e-5 for fp32 inputs, on the reads and on every head's
memory (Z block, S vector).
"""
import numpy as np
import pytest
import torch

import oracle
import segment_wise_compressive_amd as la
from segment_wise_compressive_amd import inputs as inp
from reference_forms import rowwise_rel_err

pytestmark = pytest.mark.gpu
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-3}
DEV = "cuda:0"


def _log(msg):
    print(msg, flush=True)


def heads_err(gpu, ref, d):
    return rowwise_rel_err(np.asarray(gpu).reshape(-1, d), np.asarray(ref).reshape(-1, d))


def block_err(gpu, ref, n):
    """one row per head: its whole Z block (n = d * d) or S vector (n = d)."""
    return rowwise_rel_err(np.asarray(gpu).reshape(-1, n), np.asarray(ref).reshape(-1, n))


def earlier_memory(B, H, d, seed, dtype):
    """A memory as earlier segments leave it: the state of 300 random tokens
    (fp32 values, the same ones for the GPU and the oracle)."""
    scale = 1.0 if dtype == torch.float32 else d ** -0.5
    q, k, v = inp.qkv((B, H, 300, d), seed, dtype, scale)
    _, z, s = oracle.causal(q, k, v, 1e-6, want_out=False)
    return torch.from_numpy(z).float(), torch.from_numpy(s).float()


def run_memory(q, k, v, z_in=None, s_in=None, want_out=True, eps=1e-6):
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=DEV) if want_out else None
    z = torch.empty(B, H, d, d, device=DEV)
    s = torch.empty(B, H, d, device=DEV)
    la.la_memory_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, eps=eps,
                     z_in=None if z_in is None else z_in.to(DEV), s_in=None if s_in is None else s_in.to(DEV),
                     z_out=z, s_out=s)
    torch.cuda.synchronize()
    return (None if out is None else out.cpu()), z.cpu(), s.cpu()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N", [1, 100, 1500])
def test_memory_small(dtype, d, N):
    B, H = 2, 3
    _log(f"memory dtype={dtype} d={d} N={N}")
    scale = 1.0 if dtype == torch.float32 else d ** -0.5
    q, k, v = inp.qkv((B, H, N, d), 1200 + d + N, dtype, scale)
    z0, s0 = earlier_memory(B, H, d, 1300 + d, dtype)
    ro, rz, rs = oracle.memory(q, k, v, 1e-6, z0, s0)
    out, z, s = run_memory(q, k, v, z0, s0)
    assert heads_err(out, ro, d) < TOL[dtype]
    assert block_err(z, rz, d * d) < TOL[dtype]
    assert block_err(s, rs, d) < TOL[dtype]


@pytest.mark.parametrize("d", [64, 128])
def test_memory_segment_chain_ping_pong_and_in_place(d):
    B, H, N, seg = 1, 4, 4 * 700, 700
    _log(f"memory chain d={d}")
    q, k, v = inp.qkv((B, H, N, d), 1400 + d, torch.bfloat16, d ** -0.5)
    zr = sr = None
    zs = [torch.zeros(B, H, d, d, device=DEV) for _ in range(2)]
    ss = [torch.zeros(B, H, d, device=DEV) for _ in range(2)]
    zi = torch.zeros(B, H, d, d, device=DEV)
    si = torch.zeros(B, H, d, device=DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for i in range(N // seg):
        sl = slice(i * seg, (i + 1) * seg)
        ro, zr, sr = oracle.memory(q[:, :, sl], k[:, :, sl], v[:, :, sl], 1e-6, zr, sr)
        o1 = torch.empty(B, H, seg, d, device=DEV)
        la.la_memory_fwd(qd[:, :, sl], kd[:, :, sl], vd[:, :, sl], o1,
                         z_in=zs[i & 1] if i else None, s_in=ss[i & 1] if i else None,
                         z_out=zs[(i + 1) & 1], s_out=ss[(i + 1) & 1])
        o2 = torch.empty_like(o1)
        la.la_memory_fwd(qd[:, :, sl], kd[:, :, sl], vd[:, :, sl], o2, z_in=zi, s_in=si, z_out=zi, s_out=si)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(zi, zs[(i + 1) & 1]) and torch.equal(si, ss[(i + 1) & 1])
        if i == 0:
            assert not o1.cpu().any()   # an empty memory reads 0 / eps
        else:
            assert heads_err(o1.cpu(), ro, d) < 2e-3, i
    assert block_err(zi.cpu(), zr, d * d) < 2e-3
    assert block_err(si.cpu(), sr, d) < 2e-3


def test_memory_update_only_and_zero_length():
    B, H, N, d = 2, 3, 500, 128
    q, k, v = inp.qkv((B, H, N, d), 1500, torch.bfloat16, d ** -0.5)
    z0, s0 = earlier_memory(B, H, d, 1501, torch.bfloat16)
    _, z1, s1 = run_memory(q, k, v, z0, s0)
    none, z2, s2 = run_memory(q, k, v, z0, s0, want_out=False)
    assert none is None and torch.equal(z1, z2) and torch.equal(s1, s2)
    e = torch.empty(B, H, 0, d, dtype=torch.bfloat16)
    _, z3, s3 = run_memory(e, e, e, z0, s0)
    assert torch.equal(z3, z0) and torch.equal(s3, s0)
    _, z4, s4 = run_memory(e, e, e)
    assert not z4.any() and not s4.any()


def test_memory_bitwise_deterministic():
    B, H, N, d = 1, 16, 2048, 128
    q, k, v = inp.qkv((B, H, N, d), 1600, torch.bfloat16, d ** -0.5)
    z0, s0 = earlier_memory(B, H, d, 1601, torch.bfloat16)
    a = run_memory(q, k, v, z0, s0)
    b = run_memory(q, k, v, z0, s0)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_memory_strided_inputs_and_wide_output():
    # [B, N, H, d] storage viewed as [B, H, N, d]; reads into a wider buffer
    B, H, N, d = 2, 4, 777, 128
    g = torch.Generator().manual_seed(1700)
    base = [(torch.randn(B, N, H, d, generator=g) * d ** -0.5).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.permute(0, 2, 1, 3) for t in base)
    z0, s0 = earlier_memory(B, H, d, 1701, torch.bfloat16)
    ro, rz, rs = oracle.memory(q.contiguous(), k.contiguous(), v.contiguous(), 1e-6, z0, s0)
    qd, kd, vd = (t.to(DEV).permute(0, 2, 1, 3) for t in base)
    wide = torch.full((B, H, N, 2 * d), 7.0, device=DEV)
    z = torch.empty(B, H, d, d, device=DEV)
    s = torch.empty(B, H, d, device=DEV)
    la.la_memory_fwd(qd, kd, vd, wide[..., :d], z_in=z0.to(DEV), s_in=s0.to(DEV), z_out=z, s_out=s)
    torch.cuda.synchronize()
    assert heads_err(wide[..., :d].cpu(), ro, d) < 2e-3
    assert (wide[..., d:] == 7.0).all()
    assert block_err(z.cpu(), rz, d * d) < 2e-3 and block_err(s.cpu(), rs, d) < 2e-3
