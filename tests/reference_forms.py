"""Independent fp64 NumPy formulations used to pin the oracle.

These do not share code with the oracle (which is C) or with the HIP path.
They restate the method in the other forms the pages give:

* ``quadratic_masked``: the attention matrix form.  "Attention Kernel Mask"
  (allenlu2009.github.io), section "Cumsum": the prefix sums over positions
  <= t equal a product with the all-ones lower-triangular matrix; mode 1 of
  "How to accelerate causal linear attention" (pure quadratic mode).
* ``chunked``: mode 3 of the same section (chunk-sequential, non-materialising):
  an inter-chunk term from the state of all earlier tokens plus an
  intra-chunk masked quadratic term, then the state update with the chunk's
  keys and values.  The normaliser is chunked the same way.
* ``materialised``: mode 4 (all chunk states first, then every chunk's output
  independently from its own starting state).
"""
import numpy as np


def phi(x):
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().double().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def quadratic_masked(q, k, v, eps, z_in=None, s_in=None):
    """out_t = (g_t^T Z_in + sum_{i<=t} (g_t . f_i) v_i) / (g_t . S_in + sum_{i<=t} g_t . f_i + eps)
    for one head: q, k, v [N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    g, f = phi(q), phi(k)
    W = (g @ f.T) * np.tril(np.ones((N, N)))
    num = W @ v
    den = W.sum(axis=1)
    if z_in is not None:
        num = num + g @ _f64(z_in)
        den = den + g @ _f64(s_in)
    return num / (den + eps)[:, None]


def chunked(q, k, v, eps, C, z_in=None, s_in=None):
    """Mode-3 chunk-sequential evaluation of one head; returns (out, Z, S)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    Z = np.zeros((d, d)) if z_in is None else _f64(z_in).copy()
    S = np.zeros(d) if s_in is None else _f64(s_in).copy()
    out = np.zeros((N, d))
    for c0 in range(0, N, C):
        sl = slice(c0, min(c0 + C, N))
        gq, fk, vc = phi(q[sl]), phi(k[sl]), v[sl]
        n = gq.shape[0]
        M = np.tril(np.ones((n, n)))
        P = (gq @ fk.T) * M
        inter_num, inter_den = gq @ Z, gq @ S
        intra_num, intra_den = P @ vc, P.sum(axis=1)
        out[sl] = (inter_num + intra_num) / (inter_den + intra_den + eps)[:, None]
        Z = Z + fk.T @ vc
        S = S + fk.sum(axis=0)
    return out, Z, S


def materialised(q, k, v, eps, C, z_in=None, s_in=None):
    """Mode 4: scan all chunk states first, then each chunk independently."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    Z = np.zeros((d, d)) if z_in is None else _f64(z_in).copy()
    S = np.zeros(d) if s_in is None else _f64(s_in).copy()
    starts = []
    for c0 in range(0, N, C):
        starts.append((c0, Z.copy(), S.copy()))
        fk = phi(k[c0:c0 + C])
        Z = Z + fk.T @ v[c0:c0 + C]
        S = S + fk.sum(axis=0)
    out = np.zeros((N, d))
    for c0, Zs, Ss in starts:
        sl = slice(c0, min(c0 + C, N))
        out[sl] = quadratic_masked(q[sl], k[sl], v[sl], eps, Zs, Ss)
    return out, Z, S


def rowwise_rel_err(x, y):
    """max over rows r of max_j |x_rj - y_rj| / max_j |y_rj| (last axis = row)."""
    x, y = _f64(x), _f64(y)
    d = x.shape[-1]
    x2, y2 = x.reshape(-1, d), y.reshape(-1, d)
    num = np.abs(x2 - y2).max(axis=1)
    den = np.abs(y2).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(den > 0, num / np.where(den > 0, den, 1.0), np.where(num > 0, np.inf, 0.0))
    return float(r.max()) if r.size else 0.0


def chunked_bwd(q, k, v, dout, eps, C, z_in=None, s_in=None, dz_out=None, ds_out=None):
    """Backward pass of one head in chunk form with every chunk state
    materialised (mode 4 of "How to accelerate causal linear attention",
    applied to the forward state and to the adjoint state).  With
    A_ts = v_s . dn_t + dD_t and P_ts = g_t . f_s inside a chunk (inclusive
    masks), (Z_c, S_c) the state before chunk c and (R_c, r_c) the adjoint
    state after it:
      dq_t = phi'(q_t) (Z_c dn_t + S_c dD_t + sum_{s<=t} A_ts f_s)
      dk_s = phi'(k_s) (R_c v_s + r_c + sum_{t>=s} A_ts g_t)
      dv_s = R_c^T f_s + sum_{t>=s} P_ts dn_t
    Returns (dq, dk, dv, dz_in, ds_in)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    N, d = q.shape
    g, f = phi(q), phi(k)
    dphi_q, dphi_k = np.minimum(g, 1.0), np.minimum(f, 1.0)
    chunks = [slice(c0, min(c0 + C, N)) for c0 in range(0, N, C)]
    # forward chunk states, then the normalisers
    Zs, Ss = [], []
    Z = np.zeros((d, d)) if z_in is None else _f64(z_in).copy()
    S = np.zeros(d) if s_in is None else _f64(s_in).copy()
    den = np.zeros(N)
    num = np.zeros((N, d))
    for sl in chunks:
        Zs.append(Z.copy())
        Ss.append(S.copy())
        n = sl.stop - sl.start
        M = np.tril(np.ones((n, n)))
        P = (g[sl] @ f[sl].T) * M
        den[sl] = g[sl] @ S + P.sum(1) + eps
        num[sl] = g[sl] @ Z + P @ v[sl]
        Z = Z + f[sl].T @ v[sl]
        S = S + f[sl].sum(0)
    out = num / den[:, None]
    dn = dout / den[:, None]
    dD = -(dout * out).sum(1) / den
    # adjoint chunk states (after each chunk), from the last chunk back
    R = np.zeros((d, d)) if dz_out is None else _f64(dz_out).copy()
    r = np.zeros(d) if ds_out is None else _f64(ds_out).copy()
    Rs, rs = [None] * len(chunks), [None] * len(chunks)
    for i in reversed(range(len(chunks))):
        sl = chunks[i]
        Rs[i], rs[i] = R.copy(), r.copy()
        R = R + g[sl].T @ dn[sl]
        r = r + g[sl].T @ dD[sl]
    dq, dk, dv = np.zeros((N, d)), np.zeros((N, d)), np.zeros((N, d))
    for i, sl in enumerate(chunks):
        n = sl.stop - sl.start
        M = np.tril(np.ones((n, n)))
        A = (dn[sl] @ v[sl].T + dD[sl][:, None]) * M
        P = (g[sl] @ f[sl].T) * M
        dq[sl] = dphi_q[sl] * (dn[sl] @ Zs[i].T + dD[sl][:, None] * Ss[i][None, :] + A @ f[sl])
        dk[sl] = dphi_k[sl] * (v[sl] @ Rs[i].T + rs[i][None, :] + A.T @ g[sl])
        dv[sl] = f[sl] @ Rs[i] + P.T @ dn[sl]
    return dq, dk, dv, R, r
