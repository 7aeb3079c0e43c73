"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerance: max row-wise relative error (max_j |x_j - y_j| / max_j |y_j| over
each output row, each head's Z block and each head's S) of 2e-3 for bf16
inputs with fp32 accumulation and 1e-5 for fp32 inputs.

Small cases compare every element; the full-size workloads compare every
output of a sample of heads (the oracle computes a head independently of the
others) plus properties of the whole output.
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
    """row-wise error with one row per (b, h, t) output vector."""
    return rowwise_rel_err(gpu.reshape(-1, d), ref.reshape(-1, d))


def state_err(gpu, ref):
    """one row per head: the whole Z block (or S vector) of that head."""
    g = gpu.reshape(gpu.shape[0] * gpu.shape[1], -1) if gpu.dim() > 2 else gpu.reshape(-1, gpu.shape[-1])
    r = ref.reshape(g.shape)
    return rowwise_rel_err(g, r)


def run_causal(q, k, v, chunk=0, eps=1e-6, z_in=None, s_in=None, want_state=True):
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=q.device)
    z_out = torch.empty(B, H, d, d, dtype=torch.float32, device=q.device) if want_state else None
    s_out = torch.empty(B, H, d, dtype=torch.float32, device=q.device) if want_state else None
    la.la_causal_fwd(q, k, v, out, chunk=chunk, eps=eps, z_in=z_in, s_in=s_in, z_out=z_out, s_out=s_out)
    torch.cuda.synchronize()
    return out, z_out, s_out


def rand_state(B, H, d, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    z = torch.randn(B, H, d, d, generator=g) * scale
    s = torch.rand(B, H, d, generator=g) * 10 + 1
    return z, s


# ---------------------------------------------------------------- small cases, every element
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N", [1, 17, 300])
def test_causal_small_all_elements(dtype, d, N):
    B, H = 2, 3
    _log(f"causal small dtype={dtype} d={d} N={N}")
    scale = 1.0 if dtype == torch.float32 else d ** -0.5
    q, k, v = inp.qkv((B, H, N, d), 10 + d + N, dtype, scale)
    z0, s0 = rand_state(B, H, d, 7, 0.5)
    ro, rz, rs = oracle.causal(q, k, v, 1e-6, z0, s0)
    out, z, s = run_causal(*(t.to(DEV) for t in (q, k, v)), z_in=z0.to(DEV), s_in=s0.to(DEV))
    tol = TOL[dtype]
    assert heads_err(out.cpu(), ro, d) < tol
    assert state_err(z.cpu(), torch.from_numpy(rz)) < tol
    assert state_err(s.cpu(), torch.from_numpy(rs)) < tol


@pytest.mark.parametrize("B,H,N,d", [(1, 8, 300, 64), (1, 8, 448, 64), (1, 4, 300, 128), (2, 8, 1000, 64)])
def test_causal_group_orders(B, H, N, d):
    # shapes whose workgroups fill whole XCDs with whole heads (the grid
    # order that pairs early and late groups on a CU, odd group counts
    # included) and one that does not; every element against the oracle
    _log(f"causal group orders B={B} H={H} N={N} d={d}")
    q, k, v = inp.qkv((B, H, N, d), 600 + N + d, torch.bfloat16, d ** -0.5)
    z0, s0 = rand_state(B, H, d, 11, 0.5)
    ro, rz, rs = oracle.causal(q, k, v, 1e-6, z0, s0)
    out, z, s = run_causal(*(t.to(DEV) for t in (q, k, v)), z_in=z0.to(DEV), s_in=s0.to(DEV))
    assert heads_err(out.cpu(), ro, d) < 2e-3
    assert state_err(z.cpu(), torch.from_numpy(rz)) < 2e-3
    assert state_err(s.cpu(), torch.from_numpy(rs)) < 2e-3


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_chunk_sizes_and_groups(chunk, d):
    # one head and a long sequence: many token groups (mode-4 scan) and a
    # ragged tail; every chunk size must agree with the oracle
    B, H, N = 1, 2, 3000 + 37
    _log(f"causal chunk={chunk} d={d} N={N}")
    q, k, v = inp.qkv((B, H, N, d), 500 + chunk, torch.bfloat16, d ** -0.5)
    ro, rz, rs = oracle.causal(q, k, v, 1e-6)
    out, z, s = run_causal(*(t.to(DEV) for t in (q, k, v)), chunk=chunk)
    assert heads_err(out.cpu(), ro, d) < 2e-3
    assert state_err(z.cpu(), torch.from_numpy(rz)) < 2e-3
    assert state_err(s.cpu(), torch.from_numpy(rs)) < 2e-3


def test_small_fp32_workload():
    w = inp.WORKLOADS[inp.SMALL]
    _log(f"workload {w.name}")
    q, k, v = inp.workload_inputs(w)
    ro, rz, rs = oracle.causal(q, k, v, w.eps)
    out, z, s = run_causal(*(t.to(DEV) for t in (q, k, v)), chunk=w.chunk, eps=w.eps)
    assert heads_err(out.cpu(), ro, w.d) < 1e-5
    assert state_err(z.cpu(), torch.from_numpy(rz)) < 1e-5


def test_constant_v_gpu():
    B, H, N, d = 1, 4, 700, 64
    q, k, _ = inp.qkv((B, H, N, d), 31, torch.bfloat16, 0.125)
    c = (torch.randn(B, H, 1, d, generator=torch.Generator().manual_seed(3)) * 0.1).to(torch.bfloat16)
    v = c.expand(B, H, N, d).contiguous()
    out, _, _ = run_causal(q.to(DEV), k.to(DEV), v.to(DEV), eps=0.0)
    err = rowwise_rel_err(out.cpu().reshape(-1, d), c.float().expand(B, H, N, d).reshape(-1, d))
    assert err < 1e-5


# ---------------------------------------------------------------- full-size workloads (sampled heads)
def test_headline_workload_sampled_heads():
    w = inp.WORKLOADS[inp.HEADLINE]
    _log(f"workload {w.name}")
    q, k, v = inp.workload_inputs(w)
    out, z, s = run_causal(*(t.to(DEV) for t in (q, k, v)), chunk=w.chunk, eps=w.eps)
    out, z, s = out.cpu(), z.cpu(), s.cpu()
    assert torch.isfinite(out).all()
    for b, h in [(0, 0), (1, 3), (2, 5), (3, 7)]:
        ro, rz, rs = oracle.causal(q[b, h], k[b, h], v[b, h], w.eps)
        assert heads_err(out[b, h], ro, w.d) < 2e-3, (b, h)
        assert rowwise_rel_err(z[b, h].reshape(1, -1), rz.reshape(1, -1)) < 2e-3
        assert rowwise_rel_err(s[b, h].reshape(1, -1), rs.reshape(1, -1)) < 2e-3


def test_segmented_workload_sampled_heads():
    w = inp.WORKLOADS[inp.SEGMENTED]
    _log(f"workload {w.name}")
    q, k, v = inp.workload_inputs(w)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=DEV)
    zs = [torch.zeros(B, H, d, d, device=DEV), torch.empty(B, H, d, d, device=DEV)]
    ss = [torch.zeros(B, H, d, device=DEV), torch.empty(B, H, d, device=DEV)]
    nseg = N // w.segment
    for i in range(nseg):
        sl = slice(i * w.segment, (i + 1) * w.segment)
        la.la_causal_fwd(qd[:, :, sl], kd[:, :, sl], vd[:, :, sl], out[:, :, sl], eps=w.eps,
                         z_in=zs[i & 1] if i else None, s_in=ss[i & 1] if i else None,
                         z_out=zs[(i + 1) & 1], s_out=ss[(i + 1) & 1])
    torch.cuda.synchronize()
    zf, sf = zs[nseg & 1].cpu(), ss[nseg & 1].cpu()
    oc = out.cpu()
    assert torch.isfinite(oc).all()
    for h in (0, 11):
        ro, rz, rs = oracle.causal(q[0, h], k[0, h], v[0, h], w.eps)
        assert heads_err(oc[0, h], ro, d) < 2e-3, h
        assert rowwise_rel_err(zf[0, h].reshape(1, -1), rz.reshape(1, -1)) < 2e-3
        assert rowwise_rel_err(sf[0, h].reshape(1, -1), rs.reshape(1, -1)) < 2e-3
    # the carried segments agree with one call over the whole sequence
    full, zfull, _ = run_causal(qd, kd, vd, eps=w.eps)
    assert heads_err(oc, full.cpu(), d) < 2e-3
    assert state_err(zf, zfull.cpu()) < 2e-3


def test_decode_workload_sampled_heads():
    w = inp.WORKLOADS[inp.DECODE]
    _log(f"workload {w.name}")
    (pq, pk, pv), (sq, sk, sv) = inp.workload_inputs(w)
    B, H, d, T = w.B, w.H, w.d, w.N
    z = torch.empty(B, H, d, d, device=DEV)
    s = torch.empty(B, H, d, device=DEV)
    la.la_causal_fwd(pq.to(DEV), pk.to(DEV), pv.to(DEV), None, eps=w.eps, z_out=z, s_out=s)
    sqd, skd, svd = (t.to(DEV) for t in (sq, sk, sv))
    outs = torch.empty(T, B, H, d, device=DEV)
    for t in range(T):
        la.la_decode_step(sqd[t], skd[t], svd[t], z, s, outs[t], eps=w.eps)
    torch.cuda.synchronize()
    oc, zc, sc = outs.cpu(), z.cpu(), s.cpu()
    assert torch.isfinite(oc).all()
    for b, h in [(0, 0), (37, 19), (63, 31)]:
        qq = torch.cat([pq[b, h], sq[:, b, h]], 0)
        kk = torch.cat([pk[b, h], sk[:, b, h]], 0)
        vv = torch.cat([pv[b, h], sv[:, b, h]], 0)
        ro, rz, rs = oracle.causal(qq, kk, vv, w.eps)
        assert heads_err(oc[:, b, h], ro[w.prefix:], d) < 2e-3, (b, h)
        assert rowwise_rel_err(zc[b, h].reshape(1, -1), rz.reshape(1, -1)) < 2e-3
        assert rowwise_rel_err(sc[b, h].reshape(1, -1), rs.reshape(1, -1)) < 2e-3


def test_noncausal_workload_sampled_heads():
    w = inp.WORKLOADS[inp.NONCAUSAL]
    _log(f"workload {w.name}")
    q, k, v = inp.workload_inputs(w)
    out = la.noncausal_fwd(q.to(DEV), k.to(DEV), v.to(DEV), eps=w.eps)
    torch.cuda.synchronize()
    oc = out.cpu()
    assert torch.isfinite(oc).all()
    for b, h in [(0, 0), (3, 9), (7, 15)]:
        ro, _, _ = oracle.noncausal(q[b, h], k[b, h], v[b, h], w.eps)
        assert heads_err(oc[b, h], ro, w.d) < 2e-3, (b, h)


# ---------------------------------------------------------------- other entry points, small
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N", [1, 100, 1500])
def test_noncausal_small(dtype, d, N):
    B, H = 2, 3
    _log(f"noncausal dtype={dtype} d={d} N={N}")
    scale = 1.0 if dtype == torch.float32 else d ** -0.5
    q, k, v = inp.qkv((B, H, N, d), 900 + d + N, dtype, scale)
    ro, _, _ = oracle.noncausal(q, k, v, 1e-6)
    out = la.noncausal_fwd(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    assert heads_err(out.cpu(), ro, d) < TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [32, 64, 128])
def test_decode_small(dtype, d):
    B, H, P, T = 3, 5, 40, 7
    _log(f"decode dtype={dtype} d={d}")
    scale = 1.0 if dtype == torch.float32 else d ** -0.5
    q, k, v = inp.qkv((B, H, P + T, d), 70 + d, dtype, scale)
    ro, rz, rs = oracle.causal(q, k, v, 1e-6)
    _, z, s = run_causal(q[:, :, :P].to(DEV), k[:, :, :P].to(DEV), v[:, :, :P].to(DEV))
    for t in range(P, P + T):
        o = la.decode_step(q[:, :, t].contiguous().to(DEV), k[:, :, t].contiguous().to(DEV),
                           v[:, :, t].contiguous().to(DEV), z, s)
        torch.cuda.synchronize()
        assert heads_err(o.cpu(), ro[:, :, t], d) < TOL[dtype], t
    assert state_err(z.cpu(), torch.from_numpy(rz)) < TOL[dtype]
    assert state_err(s.cpu(), torch.from_numpy(rs)) < TOL[dtype]


# ---------------------------------------------------------------- edge cases and invariants
@pytest.mark.parametrize("d", [64, 128])
def test_state_only_equals_full_call(d):
    B, H, N = 2, 2, 999
    q, k, v = inp.qkv((B, H, N, d), 44, torch.bfloat16, d ** -0.5)
    z0, s0 = rand_state(B, H, d, 8)
    _, rz, rs = oracle.causal(q, k, v, 1e-6, z0, s0, want_out=False)
    z = torch.empty(B, H, d, d, device=DEV)
    s = torch.empty(B, H, d, device=DEV)
    la.la_causal_fwd(q.to(DEV), k.to(DEV), v.to(DEV), None, z_in=z0.to(DEV), s_in=s0.to(DEV), z_out=z, s_out=s)
    torch.cuda.synchronize()
    assert state_err(z.cpu(), torch.from_numpy(rz)) < 2e-3
    assert state_err(s.cpu(), torch.from_numpy(rs)) < 2e-3


def test_zero_length_passes_state_through():
    B, H, d = 2, 3, 64
    z0, s0 = rand_state(B, H, d, 9)
    e = torch.empty(B, H, 0, d, dtype=torch.bfloat16, device=DEV)
    z = torch.empty(B, H, d, d, device=DEV)
    s = torch.empty(B, H, d, device=DEV)
    la.la_causal_fwd(e, e, e, torch.empty(B, H, 0, d, device=DEV), z_in=z0.to(DEV), s_in=s0.to(DEV),
                     z_out=z, s_out=s)
    torch.cuda.synchronize()
    assert torch.equal(z.cpu(), z0) and torch.equal(s.cpu(), s0)
    la.la_causal_fwd(e, e, e, None, z_out=z, s_out=s)
    torch.cuda.synchronize()
    assert not z.cpu().any() and not s.cpu().any()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [200, 3000])
def test_inplace_state_matches_separate_buffers(N, d):
    B, H = 1, 3
    q, k, v = (t.to(DEV) for t in inp.qkv((B, H, N, d), 45, torch.bfloat16, d ** -0.5))
    z0, s0 = (t.to(DEV) for t in rand_state(B, H, d, 10))
    o1, z1, s1 = run_causal(q, k, v, z_in=z0, s_in=s0)
    z, s = z0.clone(), s0.clone()
    o2 = torch.empty_like(o1)
    la.la_causal_fwd(q, k, v, o2, z_in=z, s_in=s, z_out=z, s_out=s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(z1, z) and torch.equal(s1, s)


def test_strided_inputs():
    # [B, N, H, d] storage viewed as [B, H, N, d]; output into a wider buffer
    B, H, N, d = 2, 4, 777, 64
    g = torch.Generator().manual_seed(46)
    base = [(torch.randn(B, N, H, d, generator=g) * 0.125).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.permute(0, 2, 1, 3) for t in base)
    ro, _, _ = oracle.causal(q.contiguous(), k.contiguous(), v.contiguous(), 1e-6)
    qd, kd, vd = (t.to(DEV).permute(0, 2, 1, 3) for t in base)
    assert qd.stride(2) == H * d
    wide = torch.full((B, H, N, 2 * d), 7.0, device=DEV)
    out = wide[..., :d]
    la.la_causal_fwd(qd, kd, vd, out)
    torch.cuda.synchronize()
    assert heads_err(out.cpu(), ro, d) < 2e-3
    assert (wide[..., d:] == 7.0).all()


def test_bitwise_deterministic():
    B, H, N, d = 2, 4, 4096, 64
    q, k, v = (t.to(DEV) for t in inp.qkv((B, H, N, d), 47, torch.bfloat16, 0.125))
    a = run_causal(q, k, v)
    b = run_causal(q, k, v)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    n1 = la.noncausal_fwd(q, k, v)
    n2 = la.noncausal_fwd(q, k, v)
    assert torch.equal(n1, n2)


@pytest.mark.parametrize("d", [64, 128])
def test_reused_workspace_new_inputs(d):
    """Back-to-back multi-group calls on one workspace, each with new inputs:
    the partial states published between workgroups must be this call's."""
    B, H, N = 1, 2, 2048 if d == 128 else 4096
    _log(f"reused workspace d={d}")
    ws = torch.empty(la.la_causal_fwd_workspace(B, H, N, d, torch.bfloat16), dtype=torch.uint8, device=DEV)
    out = torch.empty(B, H, N, d, dtype=torch.float32, device=DEV)
    z = torch.empty(B, H, d, d, dtype=torch.float32, device=DEV)
    s = torch.empty(B, H, d, dtype=torch.float32, device=DEV)
    for call in range(3):
        q, k, v = inp.qkv((B, H, N, d), 60 + call, torch.bfloat16, d ** -0.5)
        la.la_causal_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, z_out=z, s_out=s, workspace=ws)
        torch.cuda.synchronize()
        ro, rz, rs = oracle.causal(q, k, v, 1e-6)
        assert heads_err(out.cpu(), ro, d) < TOL[torch.bfloat16], call
        assert state_err(z.cpu(), rz) < TOL[torch.bfloat16], call


def test_nan_key_propagates_forward_only():
    B, H, N, d = 1, 1, 500, 64
    q, k, v = inp.qkv((B, H, N, d), 48, torch.bfloat16, 0.125)
    t0 = 300
    k[0, 0, t0, 5] = float("nan")
    ro, _, _ = oracle.causal(q, k, v, 1e-6)
    out, z, _ = run_causal(q.to(DEV), k.to(DEV), v.to(DEV))
    oc = out.cpu()
    assert torch.isfinite(oc[0, 0, :t0]).all()
    assert heads_err(oc[0, 0, :t0], ro[0, 0, :t0], d) < 2e-3
    assert torch.isnan(oc[0, 0, t0:]).all(dim=-1).all()
    assert np.isnan(ro[0, 0, t0:]).all()


def test_errors_raise_before_launch():
    q = torch.zeros(1, 2, 8, 48, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(la.LinAttnError) as e:
        la.la_causal_fwd(q, q, q, torch.empty(1, 2, 8, 48, device=DEV))
    assert e.value.status == 5
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(la.LinAttnError) as e:
        la.la_causal_fwd(q, q, q, torch.empty(1, 2, 8, 64, device=DEV), eps=-1.0)
    assert e.value.status == 6
    big = torch.zeros(1, 2, 9, 64, dtype=torch.bfloat16, device=DEV)
    mis = big.view(-1)[1:1 + 2 * 8 * 64].view(1, 2, 8, 64)   # 2-byte offset
    with pytest.raises(la.LinAttnError) as e:
        la.la_causal_fwd(mis, q, q, torch.empty(1, 2, 8, 64, device=DEV))
    assert e.value.status == 4
