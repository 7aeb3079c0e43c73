"""GPU parity at the full sizes of the workloads: every output and the final
state of EVERY head against the fp64 oracle, through the C ABI, in the launch
configuration that bench.py times.

Workloads (segment_wise_compressive_amd.inputs): the causal headline
(B4 H8 N4096 d64), the 32-segment carried loop (B1 H16, 2048-token segments,
d128), the decode workload (1024-token prefix, then 1024 steps of B64 H32
d128), the non-causal workload (B8 H16 N16384 d64), the compressive-memory
loop (B1 H16, 32 segments of 2048, d128) and the headline shape through the
unnormalised entry point.

Tolerance: max row-wise relative error (max_j |x_j - y_j| / max_j |y_j| over
each output row, each head's Z block and each head's S) of 2e-3 for bf16
inputs with fp32 accumulation.  The oracle runs a head independently of the
others, so long workloads are compared in batches of heads.
"""
import numpy as np
import pytest
import torch

import oracle
import segment_wise_compressive_amd as la
from segment_wise_compressive_amd import inputs as inp
from reference_forms import rowwise_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 2e-3


def _log(msg):
    print(msg, flush=True)


def rows_err(gpu, ref, n):
    """row-wise error with rows of n values (an output vector, a Z block, an S)."""
    return rowwise_rel_err(np.asarray(gpu).reshape(-1, n), np.asarray(ref).reshape(-1, n))


def check(tag, gpu_out, ref_out, d, gpu_z=None, ref_z=None, gpu_s=None, ref_s=None):
    e = rows_err(gpu_out, ref_out, d)
    msg = f"{tag}: output rows {np.asarray(gpu_out).size // d}, max row-wise rel err {e:.3e}"
    assert e < TOL, msg
    if gpu_z is not None:
        ez = rows_err(gpu_z, ref_z, d * d)
        es = rows_err(gpu_s, ref_s, d)
        msg += f", Z {ez:.3e}, S {es:.3e}"
        assert ez < TOL and es < TOL, msg
    _log(msg)


def test_headline_every_head():
    w = inp.WORKLOADS[inp.HEADLINE]
    _log(f"workload {w.name}")
    q, k, v = inp.workload_inputs(w)
    out = torch.empty(w.B, w.H, w.N, w.d, device=DEV)
    z = torch.empty(w.B, w.H, w.d, w.d, device=DEV)
    s = torch.empty(w.B, w.H, w.d, device=DEV)
    la.la_causal_fwd(q.to(DEV), k.to(DEV), v.to(DEV), out, chunk=w.chunk, eps=w.eps, z_out=z, s_out=s)
    torch.cuda.synchronize()
    ro, rz, rs = oracle.causal(q, k, v, w.eps)
    check(w.name, out.cpu(), ro, w.d, z.cpu(), rz, s.cpu(), rs)


def test_unnormalized_headline_every_head():
    w = inp.WORKLOADS[inp.HEADLINE]
    _log(f"workload {w.name} (unnormalised)")
    q, k, v = inp.workload_inputs(w)
    out = torch.empty(w.B, w.H, w.N, w.d, device=DEV)
    z = torch.empty(w.B, w.H, w.d, w.d, device=DEV)
    s = torch.empty(w.B, w.H, w.d, device=DEV)
    la.la_causal_fwd_unnormalized(q.to(DEV), k.to(DEV), v.to(DEV), out, chunk=w.chunk, eps=w.eps,
                                  z_out=z, s_out=s)
    torch.cuda.synchronize()
    ro = oracle.causal_unnormalized(q, k, v)
    _, rz, rs = oracle.causal(q, k, v, w.eps, want_out=False)
    check(w.name + " unnormalised", out.cpu(), ro, w.d, z.cpu(), rz, s.cpu(), rs)


def _segment_loop(fn, w, q, k, v):
    """The bench's loop: one call per segment, the state carried between two
    ping-pong buffers (the first segment starts from no state)."""
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, device=DEV)
    zs = [torch.zeros(B, H, d, d, device=DEV) for _ in range(2)]
    ss = [torch.zeros(B, H, d, device=DEV) for _ in range(2)]
    nseg = N // w.segment
    for i in range(nseg):
        sl = slice(i * w.segment, (i + 1) * w.segment)
        fn(qd[:, :, sl], kd[:, :, sl], vd[:, :, sl], out[:, :, sl], eps=w.eps,
           z_in=zs[i & 1] if i else None, s_in=ss[i & 1] if i else None,
           z_out=zs[(i + 1) & 1], s_out=ss[(i + 1) & 1])
    torch.cuda.synchronize()
    return out.cpu(), zs[nseg & 1].cpu(), ss[nseg & 1].cpu()


def test_segmented_loop_every_head():
    # the oracle's single pass over the whole sequence is the reference (the
    # segment carry of the recurrent form is pinned on the CPU)
    w = inp.WORKLOADS[inp.SEGMENTED]
    _log(f"workload {w.name}")
    q, k, v = inp.workload_inputs(w)
    out, z, s = _segment_loop(la.la_causal_fwd, w, q, k, v)
    ro, rz, rs = oracle.causal(q, k, v, w.eps)
    check(w.name, out, ro, w.d, z, rz, s, rs)


def test_memory_loop_every_head():
    w = inp.WORKLOADS[inp.MEMORY]
    _log(f"workload {w.name}")
    q, k, v = inp.workload_inputs(w)
    out, z, s = _segment_loop(la.la_memory_fwd, w, q, k, v)
    zr = sr = None
    nseg = w.N // w.segment
    ref = np.empty((w.B, w.H, w.N, w.d))
    for i in range(nseg):
        sl = slice(i * w.segment, (i + 1) * w.segment)
        ref[:, :, sl], zr, sr = oracle.memory(q[:, :, sl], k[:, :, sl], v[:, :, sl], w.eps, zr, sr)
    # the first segment reads an empty memory: 0 / eps = 0 exactly
    assert not out[:, :, :w.segment].any()
    check(w.name, out, ref, w.d, z, zr, s, sr)


def test_noncausal_every_head():
    w = inp.WORKLOADS[inp.NONCAUSAL]
    _log(f"workload {w.name}")
    q, k, v = inp.workload_inputs(w)
    out = la.noncausal_fwd(q.to(DEV), k.to(DEV), v.to(DEV), eps=w.eps)
    torch.cuda.synchronize()
    oc = out.cpu()
    del out
    for b0 in range(0, w.B, 4):   # four batches of 4 x 16 heads
        ro, _, _ = oracle.noncausal(q[b0:b0 + 4], k[b0:b0 + 4], v[b0:b0 + 4], w.eps)
        check(f"{w.name} b {b0}..{b0 + 3}", oc[b0:b0 + 4], ro, w.d)


def test_decode_every_head():
    """The prefix state from a state-only la_causal_fwd call (no q), then
    1024 la_decode_step calls: every step's output and the final state of all
    2048 heads against the oracle's recurrent pass over prefix + steps."""
    w = inp.WORKLOADS[inp.DECODE]
    _log(f"workload {w.name}")
    (pq, pk, pv), (sq, sk, sv) = inp.workload_inputs(w)
    B, H, d, T = w.B, w.H, w.d, w.N
    z = torch.empty(B, H, d, d, device=DEV)
    s = torch.empty(B, H, d, device=DEV)
    la.la_causal_fwd(None, pk.to(DEV), pv.to(DEV), None, eps=w.eps, z_out=z, s_out=s)
    sqd, skd, svd = (t.to(DEV) for t in (sq, sk, sv))
    outs = torch.empty(T, B, H, d, device=DEV)
    calls = [la.prepare_decode_step(sqd[t], skd[t], svd[t], z, s, outs[t], eps=w.eps) for t in range(T)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    oc, zc, sc = outs.cpu(), z.cpu(), s.cpu()
    del outs, sqd, skd, svd
    for b0 in range(0, B, 8):   # eight batches of 8 x 32 heads
        sl = slice(b0, b0 + 8)
        qq = torch.cat([pq[sl], sq[:, sl].permute(1, 2, 0, 3)], 2)
        kk = torch.cat([pk[sl], sk[:, sl].permute(1, 2, 0, 3)], 2)
        vv = torch.cat([pv[sl], sv[:, sl].permute(1, 2, 0, 3)], 2)
        ro, rz, rs = oracle.causal(qq, kk, vv, w.eps)
        check(f"{w.name} b {b0}..{b0 + 7}", oc[:, sl].permute(1, 2, 0, 3), ro[:, :, w.prefix:], d,
              zc[sl], rz, sc[sl], rs)
