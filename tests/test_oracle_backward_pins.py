"""Pins of the oracle's backward pass (oracle.causal_bwd), each independent
of the code it checks:

* reverse-mode autodiff (torch, float64, CPU) of the brute-force masked
  quadratic form -- the attention-matrix form of "Attention Kernel Mask",
  section "Cumsum" / mode 1 -- with a carried-in state and gradients
  reaching the final state;
* central differences of the FORWARD oracle (oracle.causal), inputs on a
  coarse binary grid so that every perturbed value is exact in float32;
* the adjoint state carried across a segment cut ("Segment-Wise Attention":
  the memory passed from segment to segment), against one pass over the
  whole sequence;
* closed forms: q = k = 0 (phi = 1, so every output is a weighted running
  mean of v and dv is a weighted suffix sum of dout); a single token; and
  constant v with eps = 0 (every output is exactly that constant, so dq and
  dk vanish).

The backward pass is not printed on the pages ("Training-Backward" is a row of
the table under "Causal Attention Training and Inferencing" with no mode
marked); the reading is the exact derivative of the forward definition.
"""
import numpy as np
import pytest
import torch

import oracle


def _grid(shape, seed, step=2.0 ** -8, scale=1.0):
    """float32 values on multiples of `step` (exact under +- 2^-12)."""
    g = np.random.default_rng(seed)
    return (np.round(g.standard_normal(shape) * scale / step) * step).astype(np.float32)


def _phi_t(x):
    return torch.where(x > 0, x + 1.0, torch.exp(torch.clamp(x, max=0.0)))


def _autograd(q, k, v, dout, eps, z_in, s_in, dz_out, ds_out):
    """Gradients of L = sum dout * out + sum dz_out * Z_N + ds_out . S_N by
    torch autograd through the brute-force masked quadratic form (one head
    at a time), all in float64."""
    BH, N, d = q.shape
    res = [np.empty((BH, N, d)) for _ in range(3)] + [np.empty((BH, d, d)), np.empty((BH, d))]
    for h in range(BH):
        qq, kk, vv = (torch.tensor(x[h], dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        zi = torch.tensor(z_in[h], dtype=torch.float64, requires_grad=True)
        si = torch.tensor(s_in[h], dtype=torch.float64, requires_grad=True)
        g, f = _phi_t(qq), _phi_t(kk)
        W = (g @ f.T) * torch.tril(torch.ones(N, N, dtype=torch.float64))
        out = (W @ vv + g @ zi) / (W.sum(1) + g @ si + eps)[:, None]
        Z, S = zi + f.T @ vv, si + f.sum(0)
        L = (out * torch.tensor(dout[h], dtype=torch.float64)).sum() + (Z * torch.tensor(dz_out[h])).sum() + \
            (S * torch.tensor(ds_out[h])).sum()
        L.backward()
        for i, t in enumerate((qq, kk, vv, zi, si)):
            res[i][h] = t.grad.numpy()
    return res


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("N,d", [(1, 4), (5, 2), (17, 8), (40, 16)])
@pytest.mark.parametrize("with_state", [False, True])
@pytest.mark.parametrize("eps", [1e-6, 0.3])
def test_backward_equals_autograd_of_quadratic_form(N, d, with_state, eps):
    BH = 3
    q, k, v = (_grid((BH, N, d), 10 * N + d + i) for i in range(3))
    dout = _grid((BH, N, d), 99 + N, scale=0.7)
    rng = np.random.default_rng(7 + N)
    if with_state:
        z_in = rng.standard_normal((BH, d, d))
        s_in = rng.random((BH, d)) * 5 + 1
        dz_out = rng.standard_normal((BH, d, d))
        ds_out = rng.standard_normal((BH, d))
    else:
        z_in, s_in = np.zeros((BH, d, d)), np.zeros((BH, d))
        dz_out, ds_out = np.zeros((BH, d, d)), np.zeros((BH, d))
    ref = _autograd(q, k, v, dout, eps, z_in, s_in, dz_out, ds_out)
    got = oracle.causal_bwd(q, k, v, dout, eps, z_in if with_state else None, s_in if with_state else None,
                            dz_out if with_state else None, ds_out if with_state else None)
    # dq and dk are differences of terms of size |dout| |v| that cancel (to
    # eps / D when v is nearly constant), so the bound has a floor at that size
    floor = 1e-13 * N * d * (np.abs(dout).max() * (np.abs(v).max() + 1) + np.abs(dz_out).max() + 1)
    for name, a, b in zip(("dq", "dk", "dv", "dz_in", "ds_in"), got, ref):
        err = np.abs(a - b).max()
        assert err <= 1e-11 * np.abs(b).max() + floor, (name, err, np.abs(b).max())


def _loss(q, k, v, dout, eps, z_in, s_in, dz_out, ds_out):
    out, Z, S = oracle.causal(q, k, v, eps, z_in, s_in)
    return float((out * dout).sum() + (Z * dz_out).sum() + (S * ds_out).sum())


def test_backward_equals_central_differences_of_forward_oracle():
    BH, N, d, eps = 2, 6, 3, 0.05
    q, k, v = (_grid((BH, N, d), 300 + i) for i in range(3))
    dout = _grid((BH, N, d), 310, scale=0.5).astype(np.float64)
    rng = np.random.default_rng(311)
    z_in = rng.standard_normal((BH, d, d))
    s_in = rng.random((BH, d)) * 3 + 1
    dz_out = rng.standard_normal((BH, d, d))
    ds_out = rng.standard_normal((BH, d))
    got = oracle.causal_bwd(q, k, v, dout.astype(np.float32), eps, z_in, s_in, dz_out, ds_out)
    h = 2.0 ** -12
    args = [q, k, v]
    for which in range(3):
        num = np.empty_like(args[which], dtype=np.float64)
        for idx in np.ndindex(*args[which].shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += np.float32(h)
            minus[which][idx] -= np.float32(h)
            assert plus[which][idx] - args[which][idx] == np.float32(h)   # exact on the grid
            num[idx] = (_loss(*plus, dout, eps, z_in, s_in, dz_out, ds_out) -
                        _loss(*minus, dout, eps, z_in, s_in, dz_out, ds_out)) / (2 * h)
        assert _rel(got[which], num) < 2e-5, ("dq dk dv"[3 * which:3 * which + 2], _rel(got[which], num))
    # the carried-in state (float64 inputs of the oracle)
    hz = 1e-6
    for which, base in ((3, z_in), (4, s_in)):
        num = np.empty_like(base)
        for idx in np.ndindex(*base.shape):
            p, m = base.copy(), base.copy()
            p[idx] += hz
            m[idx] -= hz
            zp, sp = (p, s_in) if which == 3 else (z_in, p)
            zm, sm = (m, s_in) if which == 3 else (z_in, m)
            num[idx] = (_loss(q, k, v, dout, eps, zp, sp, dz_out, ds_out) -
                        _loss(q, k, v, dout, eps, zm, sm, dz_out, ds_out)) / (2 * hz)
        assert _rel(got[which], num) < 1e-6, which


@pytest.mark.parametrize("cut", [1, 7, 31])
def test_adjoint_state_carried_across_a_segment_cut(cut):
    BH, N, d, eps = 2, 40, 8, 1e-6
    q, k, v = (_grid((BH, N, d), 400 + i, scale=0.5) for i in range(3))
    dout = _grid((BH, N, d), 410)
    rng = np.random.default_rng(411)
    z0, s0 = rng.standard_normal((BH, d, d)), rng.random((BH, d)) + 1
    dzN, dsN = rng.standard_normal((BH, d, d)), rng.standard_normal((BH, d))
    full = oracle.causal_bwd(q, k, v, dout, eps, z0, s0, dzN, dsN)
    a, b = slice(0, cut), slice(cut, N)
    _, za, sa = oracle.causal(q[:, a], k[:, a], v[:, a], eps, z0, s0, want_out=False)
    gb = oracle.causal_bwd(q[:, b], k[:, b], v[:, b], dout[:, b], eps, za, sa, dzN, dsN)
    ga = oracle.causal_bwd(q[:, a], k[:, a], v[:, a], dout[:, a], eps, z0, s0, gb[3], gb[4])
    for i in range(3):
        assert _rel(np.concatenate([ga[i], gb[i]], 1), full[i]) < 1e-12
    assert _rel(ga[3], full[3]) < 1e-12 and _rel(ga[4], full[4]) < 1e-12


def test_closed_form_q_k_zero():
    # phi = 1: out_t = d sum_{i<=t} v_i / (d (t + 1) + eps), so
    # dv_i = sum_{t>=i} dout_t d / (d (t + 1) + eps)
    BH, N, d, eps = 2, 30, 4, 0.25
    z = np.zeros((BH, N, d), np.float32)
    v = _grid((BH, N, d), 500)
    dout = _grid((BH, N, d), 501)
    _, _, dv, dz, ds = oracle.causal_bwd(z, z, v, dout, eps)
    w = d / (d * (np.arange(N) + 1.0) + eps)
    ref = np.flip(np.cumsum(np.flip(dout * w[None, :, None], 1), 1), 1)
    assert _rel(dv, ref) < 1e-13
    # the gradient reaching an (absent) carried-in state: sum_t g_t dn_t^T
    # with g = 1 and dn_t = dout_t / D_t, D_t = d (t + 1) + eps
    ref_dz = np.broadcast_to((dout / (d * (np.arange(N) + 1.0) + eps)[None, :, None]).sum(1)[:, None, :],
                             (BH, d, d))
    assert _rel(dz, ref_dz) < 1e-13


def test_closed_form_single_token():
    # out = w v / (w + eps) with w = phi(q) . phi(k): dv = dout w / (w + eps),
    # dL/dw = (dout . v) eps / (w + eps)^2, dq = phi(k) dL/dw phi'(q), dk alike
    BH, d, eps = 4, 5, 0.5
    q, k, v = (_grid((BH, 1, d), 600 + i) for i in range(3))
    dout = _grid((BH, 1, d), 603)
    dq, dk, dv, _, _ = oracle.causal_bwd(q, k, v, dout, eps)
    f64 = lambda x: x.astype(np.float64)[:, 0]
    phi = lambda x: np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    dphi = lambda x: np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    gq, fk = phi(f64(q)), phi(f64(k))
    w = (gq * fk).sum(1)
    dLdw = (f64(dout) * f64(v)).sum(1) * eps / (w + eps) ** 2
    assert _rel(dv[:, 0], f64(dout) * (w / (w + eps))[:, None]) < 1e-13
    assert _rel(dq[:, 0], fk * dLdw[:, None] * dphi(f64(q))) < 1e-12
    assert _rel(dk[:, 0], gq * dLdw[:, None] * dphi(f64(k))) < 1e-12


def test_constant_v_without_eps_has_no_q_or_k_gradient():
    BH, N, d = 2, 25, 6
    q, k = (_grid((BH, N, d), 700 + i) for i in range(2))
    c = _grid((BH, 1, d), 702)
    v = np.repeat(c, N, axis=1)
    dout = _grid((BH, N, d), 703)
    dq, dk, dv, _, _ = oracle.causal_bwd(q, k, v, dout, 0.0)
    scale = np.abs(dv).max()
    assert np.abs(dq).max() < 1e-12 * scale and np.abs(dk).max() < 1e-12 * scale
    assert scale > 0.1


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_backward_equals_chunked_materialised_form(C):
    # the chunk decomposition (every chunk's forward and adjoint state
    # materialised, then each chunk on its own) equals the recurrent oracle
    from reference_forms import chunked_bwd
    BH, N, d, eps = 2, 150, 8, 1e-6
    q, k, v = (_grid((BH, N, d), 800 + i, scale=0.5) for i in range(3))
    dout = _grid((BH, N, d), 810)
    rng = np.random.default_rng(811)
    z0, s0 = rng.standard_normal((BH, d, d)), rng.random((BH, d)) + 1
    dzN, dsN = rng.standard_normal((BH, d, d)), rng.standard_normal((BH, d))
    got = oracle.causal_bwd(q, k, v, dout, eps, z0, s0, dzN, dsN)
    for h in range(BH):
        ref = chunked_bwd(q[h], k[h], v[h], dout[h], eps, C, z0[h], s0[h], dzN[h], dsN[h])
        for i in range(5):
            assert _rel(got[i][h], ref[i]) < 1e-10, (h, i, _rel(got[i][h], ref[i]))
