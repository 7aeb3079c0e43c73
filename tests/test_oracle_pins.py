"""Pins of the fp64 oracle to things other than itself.

Each test ties the oracle to a fact the pages or the mathematics fix: a
hand-worked example with exact fractions, textbook values of the feature map,
the quadratic masked form and the chunked forms (independent NumPy code),
closed forms, and invariants.  The mutation tests in test_oracle_mutants.py
check that plausible slips in the oracle's C code fail these pins.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from reference_forms import chunked, materialised, phi, quadratic_masked, rowwise_rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TIGHT = 1e-12


def _load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = line.split("=", 1)
            vals[key.strip()] = np.array([float(Fraction(t)) for t in rhs.split()])
    return vals


def rnd(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).numpy().astype(np.float32)


# ---------------------------------------------------------------- golden
def test_golden_hand_worked_causal():
    gv = _load_golden("hand_worked_d2_n3.txt")
    q, k, v = (gv[n].reshape(1, 3, 2) for n in ("q", "k", "v"))
    out, z, s = oracle.causal(q, k, v, 0.0)
    np.testing.assert_allclose(out.reshape(-1), gv["causal_out"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(z.reshape(-1), gv["causal_z"], rtol=0, atol=0)
    np.testing.assert_allclose(s.reshape(-1), gv["causal_s"], rtol=0, atol=0)


def test_golden_hand_worked_noncausal_and_decode():
    gv = _load_golden("hand_worked_d2_n3.txt")
    q, k, v = (gv[n].reshape(1, 3, 2) for n in ("q", "k", "v"))
    out, z, s = oracle.noncausal(q, k, v, 0.0)
    np.testing.assert_allclose(out.reshape(-1), gv["noncausal_out"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(z.reshape(-1), gv["causal_z"], rtol=0, atol=0)
    # state after two tokens, then one decode step with the third token
    _, z1, s1 = oracle.causal(q[:, :2], k[:, :2], v[:, :2], 0.0)
    np.testing.assert_allclose(z1.reshape(-1), gv["state_after_t1_z"], rtol=0, atol=0)
    np.testing.assert_allclose(s1.reshape(-1), gv["state_after_t1_s"], rtol=0, atol=0)
    o2, z2, s2 = oracle.decode_step(q[:, 2], k[:, 2], v[:, 2], z1, s1, 0.0)
    np.testing.assert_allclose(o2.reshape(-1), gv["causal_out"][4:], rtol=1e-15, atol=0)
    np.testing.assert_allclose(z2.reshape(-1), gv["causal_z"], rtol=0, atol=0)


def test_golden_eps_added_once_to_denominator():
    gv = _load_golden("hand_worked_d2_n3.txt")
    q, k, v = (gv[n].reshape(1, 3, 2) for n in ("q", "k", "v"))
    eps = 0.5
    out, _, _ = oracle.causal(q, k, v, eps)
    # numerators 4,-4 / 17,-5 / 13,3 over denominators 4, 11, 10 (+ eps once)
    exp = np.array([4, -4, 17, -5, 13, 3], float) / np.repeat([4 + eps, 11 + eps, 10 + eps], 2)
    np.testing.assert_allclose(out.reshape(-1), exp, rtol=1e-15, atol=0)


# ---------------------------------------------------------------- feature map
@pytest.mark.parametrize("x, phix", [
    (0.0, 1.0),                  # both branches give 1
    (2.5, 3.5), (0.5, 1.5),      # x + 1 above zero (exact)
    (-1.0, math.exp(-1.0)),      # e^x at and below zero: 1/e
    (-2.0, math.exp(-2.0)),
])
def test_phi_textbook_values(x, phix):
    # Two tokens, d = 1, q = 0 (phi = 1), v = (1, 0), eps = 0:
    # out_1 = phi(k0) / (phi(k0) + phi(k1)); with k1 = 0, phi(k1) = 1.
    q = np.zeros((1, 2, 1), np.float32)
    k = np.array([x, 0.0], np.float32).reshape(1, 2, 1)
    v = np.array([1.0, 0.0], np.float32).reshape(1, 2, 1)
    out, _, _ = oracle.causal(q, k, v, 0.0)
    assert out[0, 1, 0] == pytest.approx(phix / (phix + 1.0), rel=1e-15)


def test_phi_minus_ln2_is_half():
    x = np.float32(-math.log(2.0))   # float32 rounding of -ln 2, relative 3e-8
    q = np.zeros((1, 2, 1), np.float32)
    k = np.array([x, 0.0], np.float32).reshape(1, 2, 1)
    v = np.array([1.0, 0.0], np.float32).reshape(1, 2, 1)
    out, _, _ = oracle.causal(q, k, v, 0.0)
    assert out[0, 1, 0] == pytest.approx(1.0 / 3.0, rel=1e-7)


def test_phi_positive_everywhere():
    x = np.linspace(-80, 80, 1001).astype(np.float32).reshape(1001, 1, 1)
    ones = np.ones((1001, 1, 1), np.float32)
    _, _, s = oracle.causal(ones, x, ones, 0.0)
    assert (s > 0).all()


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("d", [1, 2, 4, 8, 32])
@pytest.mark.parametrize("N", [1, 2, 7, 33, 64])
def test_oracle_matches_quadratic_masked(N, d):
    for seed in range(3):
        q, k, v = (rnd((1, N, d), 100 * seed + i) for i in range(3))
        out, _, _ = oracle.causal(q, k, v, 1e-6)
        ref = quadratic_masked(q[0], k[0], v[0], 1e-6)
        assert rowwise_rel_err(out[0], ref) < TIGHT


@pytest.mark.parametrize("d", [2, 8])
def test_oracle_with_state_in_matches_quadratic_masked(d):
    N = 21
    q, k, v = (rnd((1, N, d), 7 + i) for i in range(3))
    zi = rnd((1, d, d), 20).astype(np.float64)
    si = np.abs(rnd((1, d), 21)).astype(np.float64) + 1.0
    out, z, s = oracle.causal(q, k, v, 1e-6, zi, si)
    ref = quadratic_masked(q[0], k[0], v[0], 1e-6, zi[0], si[0])
    assert rowwise_rel_err(out[0], ref) < TIGHT
    zr = zi[0] + phi(k[0]).T @ v[0].astype(np.float64)
    np.testing.assert_allclose(z[0], zr, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s[0], si[0] + phi(k[0]).sum(0), rtol=1e-12)


@pytest.mark.parametrize("C", [1, 2, 3, 8, 16, 48])
def test_oracle_matches_chunked_any_chunk_size(C):
    N, d = 48, 16
    q, k, v = (rnd((1, N, d), 300 + i, 0.25) for i in range(3))
    out, z, s = oracle.causal(q, k, v, 1e-6)
    o2, z2, s2 = chunked(q[0], k[0], v[0], 1e-6, C)
    o3, z3, s3 = materialised(q[0], k[0], v[0], 1e-6, C)
    for o, zz, ss in ((o2, z2, s2), (o3, z3, s3)):
        assert rowwise_rel_err(out[0], o) < TIGHT
        np.testing.assert_allclose(z[0], zz, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(s[0], ss, rtol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_constant_v_gives_constant_output():
    N, d = 40, 8
    q, k = rnd((2, N, d), 1), rnd((2, N, d), 2)
    c = rnd((2, 1, d), 3)
    v = np.broadcast_to(c, (2, N, d)).copy()
    out, _, _ = oracle.causal(q, k, v, 0.0)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=1e-14, atol=1e-15)
    eps = 1e-6
    out, _, _ = oracle.causal(q, k, v, eps)
    A = np.einsum("htd,hid->hti", phi(q), phi(k)) * np.tril(np.ones((N, N)))
    A = A.sum(-1)
    bound = np.abs(c) * eps / A[..., None] * (1 + 1e-9) + 1e-15
    assert (np.abs(out - c) <= bound).all()


def test_zero_q_k_gives_scaled_running_mean():
    N, d, eps = 30, 4, 1e-3
    v = rnd((1, N, d), 5)
    z = np.zeros((1, N, d), np.float32)
    out, _, _ = oracle.causal(z, z, v, eps)
    t1 = np.arange(1, N + 1)[:, None].astype(np.float64)
    mean = np.cumsum(v[0].astype(np.float64), axis=0) / t1
    np.testing.assert_allclose(out[0], mean * (d * t1) / (d * t1 + eps), rtol=1e-13, atol=1e-15)


def test_equal_keys_give_uniform_weights():
    N, d, eps = 25, 6, 1e-6
    q, v = rnd((1, N, d), 8), rnd((1, N, d), 9)
    k = np.broadcast_to(rnd((1, 1, d), 10), (1, N, d)).copy()
    out, _, _ = oracle.causal(q, k, v, eps)
    t1 = np.arange(1, N + 1)[:, None].astype(np.float64)
    mean = np.cumsum(v[0].astype(np.float64), axis=0) / t1
    A = (phi(q[0]) @ phi(k[0, 0]))[:, None] * t1
    np.testing.assert_allclose(out[0], mean * A / (A + eps), rtol=1e-13, atol=1e-15)


def test_single_token():
    d, eps = 16, 1e-6
    q, k, v = (rnd((1, 1, d), 11 + i) for i in range(3))
    out, z, s = oracle.causal(q, k, v, eps)
    w = float(phi(q[0, 0]) @ phi(k[0, 0]))
    np.testing.assert_allclose(out[0, 0], v[0, 0].astype(np.float64) * w / (w + eps), rtol=1e-14)
    np.testing.assert_allclose(z[0], np.outer(phi(k[0, 0]), v[0, 0]), rtol=1e-15)


# ---------------------------------------------------------------- invariants
def test_linear_in_v():
    # v1, v2 on a 1/64 grid and a = 1/2, so v1 + a*v2 is exact in float32 and
    # linearity must hold to rounding of the fp64 arithmetic.
    N, d, a = 37, 8, 0.5
    q, k = rnd((2, N, d), 40), rnd((2, N, d), 41)
    v1 = np.round(rnd((2, N, d), 42) * 64) / 64
    v2 = np.round(rnd((2, N, d), 43) * 64) / 64
    v3 = (v1 + a * v2).astype(np.float32)
    assert np.array_equal(v3.astype(np.float64), v1.astype(np.float64) + a * v2.astype(np.float64))
    o1, _, _ = oracle.causal(q, k, v1.astype(np.float32), 1e-6)
    o2, _, _ = oracle.causal(q, k, v2.astype(np.float32), 1e-6)
    o3, _, _ = oracle.causal(q, k, v3, 1e-6)
    assert rowwise_rel_err(o1 + a * o2, o3) < 1e-11


@pytest.mark.parametrize("cuts", [(1,), (7,), (31, 32), (1, 2, 60), (16, 32, 48)])
def test_segment_carry_equals_full_sequence(cuts):
    N, d = 64, 8
    q, k, v = (rnd((3, N, d), 60 + i, 0.5) for i in range(3))
    full, zf, sf = oracle.causal(q, k, v, 1e-6)
    z = s = None
    pieces = []
    bounds = [0, *cuts, N]
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, z, s = oracle.causal(q[:, a:b], k[:, a:b], v[:, a:b], 1e-6, z, s)
        pieces.append(o)
    seg = np.concatenate(pieces, axis=1)
    assert rowwise_rel_err(seg, full) < TIGHT
    np.testing.assert_allclose(z, zf, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s, sf, rtol=1e-13)


def test_decode_steps_equal_causal():
    P, T, d = 10, 6, 8
    q, k, v = (rnd((4, P + T, d), 80 + i) for i in range(3))
    full, zf, sf = oracle.causal(q, k, v, 1e-6)
    _, z, s = oracle.causal(q[:, :P], k[:, :P], v[:, :P], 1e-6)
    for t in range(P, P + T):
        o, z, s = oracle.decode_step(q[:, t], k[:, t], v[:, t], z, s, 1e-6)
        assert rowwise_rel_err(o, full[:, t]) < TIGHT
    np.testing.assert_allclose(z, zf, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s, sf, rtol=1e-13)


def test_noncausal_properties():
    N, d = 29, 8
    q, k, v = (rnd((2, N, d), 90 + i) for i in range(3))
    out, z, s = oracle.noncausal(q, k, v, 1e-6)
    cout, cz, cs = oracle.causal(q, k, v, 1e-6)
    # the last query of the causal form already sees every key
    assert rowwise_rel_err(out[:, -1], cout[:, -1]) < TIGHT
    np.testing.assert_allclose(z, cz, rtol=1e-13, atol=1e-13)
    # the global state applied to every query
    g = phi(q)
    ref = np.einsum("htj,hjc->htc", g, cz) / (np.einsum("htj,hj->ht", g, cs) + 1e-6)[..., None]
    assert rowwise_rel_err(out, ref) < TIGHT
    # a joint permutation of (k_i, v_i) changes nothing
    perm = np.random.default_rng(0).permutation(N)
    out2, _, _ = oracle.noncausal(q, k[:, perm], v[:, perm], 1e-6)
    assert rowwise_rel_err(out2, out) < TIGHT
    # brute force: full (unmasked) quadratic form
    W = phi(q[0]) @ phi(k[0]).T
    ref0 = (W @ v[0].astype(np.float64)) / (W.sum(1) + 1e-6)[:, None]
    assert rowwise_rel_err(out[0], ref0) < TIGHT


def test_state_only_matches_full_call():
    N, d = 50, 8
    q, k, v = (rnd((2, N, d), 120 + i) for i in range(3))
    _, z1, s1 = oracle.causal(q, k, v, 1e-6)
    none, z2, s2 = oracle.causal(q, k, v, 1e-6, want_out=False)
    assert none is None
    np.testing.assert_array_equal(z1, z2)
    np.testing.assert_array_equal(s1, s2)


def test_zero_length_passes_state_through():
    d = 4
    e = np.zeros((2, 0, d), np.float32)
    zi = rnd((2, d, d), 130).astype(np.float64)
    si = rnd((2, d), 131).astype(np.float64)
    out, z, s = oracle.causal(e, e, e, 1e-6, zi, si)
    assert out.shape == (2, 0, d)
    np.testing.assert_array_equal(z, zi)
    np.testing.assert_array_equal(s, si)


# ---------------------------------------------------------------- compressive memory (retrieval, then update)
def _block_masked(q, k, v, bounds, eps):
    """Brute force over the attention matrix of the segment loop: token t of
    the segment [a, b) sees every token i < a (all earlier segments), none of
    its own segment; one head, q, k, v [N, d]."""
    g, f = phi(q), phi(k)
    N = q.shape[0]
    seg_start = np.empty(N, np.int64)
    for a, b in zip(bounds[:-1], bounds[1:]):
        seg_start[a:b] = a
    mask = (np.arange(N)[None, :] < seg_start[:, None]).astype(np.float64)
    W = (g @ f.T) * mask
    return (W @ v.astype(np.float64)) / (W.sum(axis=1) + eps)[:, None]


@pytest.mark.parametrize("cuts", [(5,), (1, 2, 30), (9, 9, 20), (16, 32, 48)])
def test_memory_chain_matches_block_masked_brute_force(cuts):
    N, d = 64, 6
    q, k, v = (rnd((2, N, d), 140 + i, 0.7) for i in range(3))
    bounds = [0, *cuts, N]
    z = s = None
    pieces = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        o, z, s = oracle.memory(q[:, a:b], k[:, a:b], v[:, a:b], 1e-6, z, s)
        pieces.append(o)
    out = np.concatenate(pieces, axis=1)
    first = bounds[1]
    # the first segment has an empty memory: 0 / eps
    assert np.array_equal(out[:, :first], np.zeros_like(out[:, :first]))
    for h in range(2):
        ref = _block_masked(q[h], k[h], v[h], bounds, 1e-6)
        assert rowwise_rel_err(out[h, first:], ref[first:]) < TIGHT
    # the memory after the last segment is the state of the whole sequence
    _, zf, sf = oracle.causal(q, k, v, 1e-6)
    np.testing.assert_allclose(z, zf, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s, sf, rtol=1e-13)


def test_memory_zero_q_k_reads_scaled_mean_of_earlier_values():
    N0, N1, d = 11, 5, 4
    z0 = np.zeros((1, N0, d), np.float32)
    v0 = rnd((1, N0, d), 150)
    _, zm, sm = oracle.memory(z0, z0, v0, 1e-6)
    q1 = np.zeros((1, N1, d), np.float32)
    out, _, _ = oracle.memory(q1, q1, rnd((1, N1, d), 151), 1e-6, zm, sm)
    # phi(0) = 1: every read is d * sum(v) / (d * N0 + eps), the same for all queries
    ref = d * v0[0].astype(np.float64).sum(axis=0) / (d * N0 + 1e-6)
    for t in range(N1):
        assert rowwise_rel_err(out[0, t], ref) < TIGHT


def test_memory_of_one_token_is_its_value_scaled():
    d = 5
    q0, k0, v0 = (rnd((1, 1, d), 160 + i) for i in range(3))
    _, zm, sm = oracle.memory(q0, k0, v0, 1e-6)
    q1 = rnd((1, 3, d), 163)
    out, _, _ = oracle.memory(q1, rnd((1, 3, d), 164), rnd((1, 3, d), 165), 1e-6, zm, sm)
    for t in range(3):
        w = float(phi(q1[0, t]) @ phi(k0[0, 0]))
        assert rowwise_rel_err(out[0, t], w * v0[0, 0].astype(np.float64) / (w + 1e-6)) < TIGHT


def test_memory_empty_memory_reads_zero_or_nan():
    d = 4
    q, k, v = (rnd((2, 3, d), 170 + i) for i in range(3))
    out, _, _ = oracle.memory(q, k, v, 1e-6)
    assert np.array_equal(out, np.zeros_like(out))
    out0, _, _ = oracle.memory(q, k, v, 0.0)   # 0 / 0
    assert np.isnan(out0).all()


def test_memory_zero_length_passes_state_through():
    d = 4
    e = np.zeros((2, 0, d), np.float32)
    zi = rnd((2, d, d), 180).astype(np.float64)
    si = rnd((2, d), 181).astype(np.float64)
    out, z, s = oracle.memory(e, e, e, 1e-6, zi, si)
    assert out.shape == (2, 0, d)
    np.testing.assert_array_equal(z, zi)
    np.testing.assert_array_equal(s, si)


# ---------------------------------------------------------------- unnormalised form
def test_unnormalized_matches_masked_numerator():
    N, d = 37, 6
    q, k, v = (rnd((2, N, d), 190 + i, 0.8) for i in range(3))
    z0 = rnd((2, d, d), 193).astype(np.float64)
    out = oracle.causal_unnormalized(q, k, v, z0)
    for h in range(2):
        g, f = phi(q[h]), phi(k[h])
        W = (g @ f.T) * np.tril(np.ones((N, N)))
        ref = W @ v[h].astype(np.float64) + g @ z0[h]
        assert rowwise_rel_err(out[h], ref) < TIGHT


def test_unnormalized_is_normalized_times_denominator():
    N, d = 41, 5
    q, k, v = (rnd((3, N, d), 200 + i, 0.6) for i in range(3))
    eps = 1e-3
    norm, _, _ = oracle.causal(q, k, v, eps)
    un = oracle.causal_unnormalized(q, k, v)
    den = np.einsum("htj,htj->ht", phi(q), np.cumsum(phi(k), axis=1)) + eps
    assert rowwise_rel_err(un, norm * den[..., None]) < 1e-11


def test_unnormalized_constant_v_and_zero_q_k():
    N, d = 9, 4
    z = np.zeros((1, N, d), np.float32)
    v = np.full((1, N, d), 0.5, np.float32)
    out = oracle.causal_unnormalized(z, z, v)
    # phi(0) = 1: out_t = d * (t + 1) * 0.5 in every column
    ref = (d * 0.5 * np.arange(1, N + 1))[:, None] * np.ones((1, d))
    np.testing.assert_allclose(out[0], ref, rtol=1e-15)


def test_unnormalized_segment_carry():
    N, d = 50, 6
    q, k, v = (rnd((2, N, d), 210 + i, 0.7) for i in range(3))
    full = oracle.causal_unnormalized(q, k, v)
    _, z, _ = oracle.causal(q[:, :17], k[:, :17], v[:, :17], 1e-6)
    tail = oracle.causal_unnormalized(q[:, 17:], k[:, 17:], v[:, 17:], z)
    assert rowwise_rel_err(tail, full[:, 17:]) < TIGHT
