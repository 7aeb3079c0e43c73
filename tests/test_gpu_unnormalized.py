"""GPU parity of la_causal_fwd_unnormalized (the chunk formulas without the
denominator: out_t = phi(q_t)^T Z_t) against the fp64 oracle, through the C
ABI.  Same tolerances as the normalised form: row-wise relative error 2e-3
for bf16 inputs and 1e-5 for fp32 inputs.
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


def run(q, k, v, normalize, chunk=0, z_in=None, s_in=None):
    B, H, N, d = q.shape
    out = torch.empty(B, H, N, d, device=DEV)
    z = torch.empty(B, H, d, d, device=DEV)
    s = torch.empty(B, H, d, device=DEV)
    fn = la.la_causal_fwd if normalize else la.la_causal_fwd_unnormalized
    fn(q.to(DEV), k.to(DEV), v.to(DEV), out, chunk=chunk, z_in=None if z_in is None else z_in.to(DEV),
       s_in=None if s_in is None else s_in.to(DEV), z_out=z, s_out=s)
    torch.cuda.synchronize()
    return out.cpu(), z.cpu(), s.cpu()


def carried_state(B, H, d, seed, dtype):
    scale = 1.0 if dtype == torch.float32 else d ** -0.5
    q, k, v = inp.qkv((B, H, 200, d), seed, dtype, scale)
    _, z, s = oracle.causal(q, k, v, 1e-6, want_out=False)
    return torch.from_numpy(z).float(), torch.from_numpy(s).float()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("N", [1, 17, 300])
def test_unnormalized_small(dtype, d, N):
    B, H = 2, 3
    _log(f"unnormalized dtype={dtype} d={d} N={N}")
    scale = 1.0 if dtype == torch.float32 else d ** -0.5
    q, k, v = inp.qkv((B, H, N, d), 2000 + d + N, dtype, scale)
    z0, s0 = carried_state(B, H, d, 2100 + d, dtype)
    ref = oracle.causal_unnormalized(q, k, v, z0)
    out, z, s = run(q, k, v, False, z_in=z0, s_in=s0)
    assert heads_err(out, ref, d) < TOL[dtype]
    # the carried state is the normalised call's, bit for bit
    _, zn, sn = run(q, k, v, True, z_in=z0, s_in=s0)
    assert torch.equal(z, zn) and torch.equal(s, sn)


# chunk sizes that run as themselves (128 only at d <= 64, bf16)
@pytest.mark.parametrize("chunk,d", [(64, 64), (128, 64), (64, 128)])
def test_unnormalized_chunk_sizes_and_groups(chunk, d):
    B, H, N = 1, 4, 1000
    _log(f"unnormalized chunk={chunk} d={d}")
    q, k, v = inp.qkv((B, H, N, d), 2200 + chunk + d, torch.bfloat16, d ** -0.5)
    ref = oracle.causal_unnormalized(q, k, v)
    out, _, _ = run(q, k, v, False, chunk=chunk)
    assert heads_err(out, ref, d) < 2e-3


def test_unnormalized_strided_inputs():
    B, H, N, d = 2, 4, 777, 64
    g = torch.Generator().manual_seed(2300)
    base = [(torch.randn(B, N, H, d, generator=g) * 0.125).to(torch.bfloat16) for _ in range(3)]
    q, k, v = (t.permute(0, 2, 1, 3) for t in base)
    ref = oracle.causal_unnormalized(q.contiguous(), k.contiguous(), v.contiguous())
    qd, kd, vd = (t.to(DEV).permute(0, 2, 1, 3) for t in base)
    out = torch.empty(B, H, N, d, device=DEV)
    la.la_causal_fwd_unnormalized(qd, kd, vd, out)
    torch.cuda.synchronize()
    assert heads_err(out.cpu(), ref, d) < 2e-3
