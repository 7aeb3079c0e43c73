"""la_causal_fwd_noalloc (the allocation-free causal forward, whose scratch
memory is a fixed per-GPU array inside the library) against la_causal_fwd
with a workspace of its own, through the C ABI.

Two calls in a row share the scratch array: first the causal headline shape
(B4 H8 N4096 d64, the column-split kernel with its look-back), then a smaller
d = 128 call with a carried-in state written back in place.  The kernels and
plans are those of la_causal_fwd, so the outputs and states must be bitwise
identical (and so within the 2e-3 bar of the bf16 parity tests).  (The
refusal of a call whose workspace would not fit is checked without a GPU in
test_abi.py.)
"""
import pytest
import torch

import segment_wise_compressive_amd as la
from segment_wise_compressive_amd import inputs as inp

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _pair(q, k, v, z0=None, s0=None, in_place=False):
    """(outputs, z, s) of la_causal_fwd and of la_causal_fwd_noalloc."""
    B, H, N, d = q.shape
    res = []
    for fn in (la.la_causal_fwd, la.la_causal_fwd_noalloc):
        out = torch.empty(B, H, N, d, device=DEV)
        if in_place:
            z, s = z0.clone(), s0.clone()
            fn(q, k, v, out, z_in=z, s_in=s, z_out=z, s_out=s)
        else:
            z = torch.empty(B, H, d, d, device=DEV)
            s = torch.empty(B, H, d, device=DEV)
            fn(q, k, v, out, z_in=z0, s_in=s0, z_out=z, s_out=s)
        torch.cuda.synchronize()
        res.append((out, z, s))
    return res


def test_noalloc_matches_workspace_call_twice():
    w = inp.WORKLOADS[inp.HEADLINE]
    print(f"no-alloc call 1: {w.name}", flush=True)
    q, k, v = (t.to(DEV) for t in inp.workload_inputs(w))
    assert la.la_causal_fwd_workspace(w.B, w.H, w.N, w.d) <= la.la_noalloc_scratch_bytes()
    (o1, z1, s1), (o2, z2, s2) = _pair(q, k, v)
    assert torch.isfinite(o2).all()
    assert torch.equal(o1, o2) and torch.equal(z1, z2) and torch.equal(s1, s2)

    B, H, N, d = 1, 2, 1000, 128
    print(f"no-alloc call 2: B{B} H{H} N{N} d{d}, state in place", flush=True)
    q, k, v = (t.to(DEV) for t in inp.qkv((B, H, N, d), 1900, torch.bfloat16, d ** -0.5))
    g = torch.Generator().manual_seed(1901)
    z0 = (torch.randn(B, H, d, d, generator=g) * 0.5).to(DEV)
    s0 = (torch.rand(B, H, d, generator=g) * 10 + 1).to(DEV)
    (o1, z1, s1), (o2, z2, s2) = _pair(q, k, v, z0, s0, in_place=True)
    assert torch.isfinite(o2).all()
    assert torch.equal(o1, o2) and torch.equal(z1, z2) and torch.equal(s1, s2)
