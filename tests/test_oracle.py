"""Pins of the fp64 CPU oracle against facts the pages and the mathematics fix.

Nothing here compares the oracle with itself: every expected value comes from
a different formulation (the O(N^2) masked quadratic form, the cumulative-sum
form at lambda = 1, the non-causal closed form with library matmuls), a closed
form, an exact identity, or a hand derivation stored under tests/golden/.
"""
import json
import math
import os
import zlib
from fractions import Fraction

import numpy as np
import pytest

from seeded_inputs import make_omega

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- feature maps
def test_phi_elu1_closed_values(orc):
    # elu with alpha = 1, plus one ("From standard attention to linear attention", sec. 4.1)
    x = np.array([[0.0, 1.0, -1.0, 2.5, -3.0, 1e-12, -1e-12, -40.0]])
    got = orc.phi_map(x, "elu1")[0]
    want = [1.0, 2.0, math.exp(-1.0), 3.5, math.exp(-3.0), 1.0 + 1e-12,
            math.exp(-1e-12), math.exp(-40.0)]
    np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)
    assert np.all(got > 0)  # strictly positive features


def test_phi_rf_identity_omega_closed_form(orc):
    # omega = identity rows, so u = x' exactly: phi = exp(-|x'|^2/2)/sqrt(m) [cos x', sin x']
    rng = np.random.default_rng(0)
    dk = m = 4
    s = 0.7
    x = _rand(rng, 3, dk)
    got = orc.phi_map(x, "trig_rf", omega=np.eye(m), scale=s)
    xs = s * x
    c = np.exp(-0.5 * np.sum(xs * xs, axis=1, keepdims=True)) / math.sqrt(m)
    want = np.concatenate([c * np.cos(xs), c * np.sin(xs)], axis=1)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-16)


def test_phi_rf_norm_identity_and_zero(orc):
    rng = np.random.default_rng(1)
    dk, m = 16, 32
    om = make_omega(m, dk, seed=11)
    s = dk ** -0.25
    x = _rand(rng, 20, dk)
    p = orc.phi_map(x, "trig_rf", omega=om, scale=s)
    # cos^2 + sin^2 = 1  =>  |phi(x)|^2 = exp(-|x'|^2)
    np.testing.assert_allclose(np.sum(p * p, axis=1), np.exp(-np.sum((s * x) ** 2, axis=1)),
                               rtol=1e-13)
    p0 = orc.phi_map(np.zeros((1, dk)), "trig_rf", omega=om, scale=s)[0]
    want0 = np.concatenate([np.full(m, m ** -0.5), np.zeros(m)])
    np.testing.assert_allclose(p0, want0, rtol=1e-15, atol=0)


def test_phi_rf_kernel_monte_carlo(orc):
    # E[phi(x).phi(y)] = exp(-|x'|^2/2 - |y'|^2/2 - |x'-y'|^2/2) for omega ~ N(0, I)
    rng = np.random.default_rng(2)
    dk, m = 8, 8192
    om = make_omega(m, dk, seed=12)
    s = 0.8
    x = _rand(rng, 6, dk, scale=0.6)
    y = _rand(rng, 6, dk, scale=0.6)
    px = orc.phi_map(x, "trig_rf", omega=om, scale=s)
    py = orc.phi_map(y, "trig_rf", omega=om, scale=s)
    got = np.sum(px * py, axis=1)
    xs, ys = s * x, s * y
    want = np.exp(-0.5 * np.sum(xs ** 2, 1) - 0.5 * np.sum(ys ** 2, 1)
                  - 0.5 * np.sum((xs - ys) ** 2, 1))
    bound = 4.0 * math.sqrt(0.5 / m) * np.exp(-0.5 * (np.sum(xs ** 2, 1) + np.sum(ys ** 2, 1)))
    assert np.all(np.abs(got - want) < bound), (got, want, bound)


def test_phi_relu_closed_values(orc):
    # ReLU feature map ("Attention is also an FFN", sec. 5.1): max(x, 0) elementwise
    x = np.array([[0.0, 1.0, -1.0, 2.5, -3.0, 1e-12, -1e-12, -40.0]])
    got = orc.phi_map(x, "relu")[0]
    want = [0.0, 1.0, 0.0, 2.5, 0.0, 1e-12, 0.0, 0.0]
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("phi,sgn", [("trig_rf_plain", 0.0), ("trig_rf_softmax", 1.0)])
def test_phi_rf_prefactor_variants_identity_omega(orc, phi, sgn):
    # "From standard attention to linear attention", sec. 4.2: prefactor
    # exp(|x|^2/2) h(x) / sqrt(m); h = exp(-|x|^2/2) gives 1/sqrt(m), h = 1 gives
    # exp(+|x'|^2/2)/sqrt(m).  With omega = I, u = x' exactly.
    rng = np.random.default_rng(3)
    dk = m = 4
    s = 0.7
    x = _rand(rng, 3, dk)
    got = orc.phi_map(x, phi, omega=np.eye(m), scale=s)
    xs = s * x
    c = np.exp(0.5 * sgn * np.sum(xs * xs, axis=1, keepdims=True)) / math.sqrt(m)
    want = np.concatenate([c * np.cos(xs), c * np.sin(xs)], axis=1)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-16)


@pytest.mark.parametrize("phi,sgn", [("trig_rf_plain", 0.0), ("trig_rf_softmax", 1.0)])
def test_phi_rf_prefactor_variants_norm(orc, phi, sgn):
    # cos^2 + sin^2 = 1  =>  |phi(x)|^2 = exp(sgn |x'|^2): 1 (plain), exp(|x'|^2) (softmax)
    rng = np.random.default_rng(4)
    dk, m = 16, 32
    om = make_omega(m, dk, seed=13)
    s = dk ** -0.25
    x = _rand(rng, 20, dk)
    p = orc.phi_map(x, phi, omega=om, scale=s)
    np.testing.assert_allclose(np.sum(p * p, axis=1), np.exp(sgn * np.sum((s * x) ** 2, axis=1)),
                               rtol=1e-13)


@pytest.mark.parametrize("phi", ["trig_rf_plain", "trig_rf_softmax"])
def test_phi_rf_prefactor_variants_kernel_monte_carlo(orc, phi):
    # omega ~ N(0, I): E[cos(w.x') cos(w.y') + sin sin] = exp(-|x'-y'|^2/2), so
    # plain features estimate the Gaussian kernel and softmax ones exp(x'.y')
    rng = np.random.default_rng(5)
    dk, m = 8, 8192
    om = make_omega(m, dk, seed=14)
    s = 0.8
    x = _rand(rng, 6, dk, scale=0.6)
    y = _rand(rng, 6, dk, scale=0.6)
    got = np.sum(orc.phi_map(x, phi, omega=om, scale=s) * orc.phi_map(y, phi, omega=om, scale=s), axis=1)
    xs, ys = s * x, s * y
    if phi == "trig_rf_plain":
        want = np.exp(-0.5 * np.sum((xs - ys) ** 2, 1))
        scale_xy = np.ones(len(x))
    else:
        want = np.exp(np.sum(xs * ys, 1))
        scale_xy = np.exp(0.5 * (np.sum(xs ** 2, 1) + np.sum(ys ** 2, 1)))
    bound = 4.0 * math.sqrt(0.5 / m) * scale_xy
    assert np.all(np.abs(got - want) < bound), (got, want, bound)


# ---------------------------------------------------------------- recurrence
def _brute_force(pq, pk, v, lam, eps):
    """O(N^2) masked quadratic form, one (b,h) row:
    y_i = sum_{j<=i} lam^(i-j) (pq_i . pk_j) v_j / (sum_{j<=i} lam^(i-j) pq_i . pk_j + eps)."""
    N = pq.shape[0]
    y = np.zeros((N, v.shape[1]))
    for i in range(N):
        num = np.zeros(v.shape[1])
        den = 0.0
        for j in range(i + 1):
            w = 1.0 if i == j else lam ** (i - j)
            a = w * float(pq[i] @ pk[j])
            num += a * v[j]
            den += a
        y[i] = num / (den + eps)
    return y


CASES = [
    # phi, dk, m, lam, eps
    ("elu1", 2, 0, 1.0, 1e-6),
    ("elu1", 4, 0, 0.0, 1e-6),
    ("elu1", 4, 0, 0.3, 1e-6),
    ("elu1", 8, 0, 0.9, 1e-6),
    ("elu1", 8, 0, 0.999, 0.0),
    ("trig_rf", 4, 6, 1.0, 1e-6),
    ("trig_rf", 8, 4, 0.95, 1e-6),
    ("relu", 4, 0, 0.9, 1e-6),
    ("relu", 8, 0, 1.0, 1e-6),
    ("trig_rf_plain", 4, 6, 1.0, 1e-6),
    ("trig_rf_softmax", 8, 4, 0.95, 1e-6),
]


@pytest.mark.parametrize("phi,dk,m,lam,eps", CASES)
def test_causal_matches_bruteforce(orc, phi, dk, m, lam, eps):
    rng = np.random.default_rng(zlib.crc32(repr((phi, dk, m, lam)).encode()))
    B, H, N, dv = 2, 2, 37, 3
    q, k = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk)
    v = _rand(rng, B, H, N, dv)
    rf = phi.startswith("trig_rf")
    om = make_omega(m, dk, seed=5) if rf else None
    s = dk ** -0.25 if rf else 1.0
    lam_h = np.array([lam, lam])
    y = orc.causal(q, k, v, lam_h, eps, phi, om, s)
    pq = orc.phi_map(q, phi, om, s)
    pk = orc.phi_map(k, phi, om, s)
    for b in range(B):
        for h in range(H):
            want = _brute_force(pq[b, h], pk[b, h], v[b, h], lam, eps)
            np.testing.assert_allclose(y[b, h], want, rtol=1e-10, atol=1e-12)


def test_per_head_lambda_bruteforce(orc):
    rng = np.random.default_rng(7)
    B, H, N, dk, dv = 1, 3, 25, 4, 2
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    lam_h = np.array([0.5, 0.9, 1.0])
    y = orc.causal(q, k, v, lam_h, 1e-6)
    pq, pk = orc.phi_map(q), orc.phi_map(k)
    for h in range(H):
        np.testing.assert_allclose(y[0, h], _brute_force(pq[0, h], pk[0, h], v[0, h],
                                                          lam_h[h], 1e-6), rtol=1e-10)


def test_lambda_one_cumsum_identity(orc):
    # lambda = 1: S_i = cumsum_j phi(k_j) v_j^T, z_i = cumsum_j phi(k_j)
    rng = np.random.default_rng(3)
    B, H, N, dk, dv = 1, 2, 50, 6, 5
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    y, S, z = orc.causal(q, k, v, None, 1e-6, want_state=True)
    pq, pk = orc.phi_map(q), orc.phi_map(k)
    outer = pk[..., :, None] * v[..., None, :]            # [B,H,N,F,dv]
    Sc = np.cumsum(outer, axis=2)
    zc = np.cumsum(pk, axis=2)
    num = np.einsum("bhnf,bhnfd->bhnd", pq, Sc)
    den = np.einsum("bhnf,bhnf->bhn", pq, zc)
    np.testing.assert_allclose(y, num / (den[..., None] + 1e-6), rtol=1e-11)
    np.testing.assert_allclose(S, Sc[:, :, -1], rtol=1e-12)
    np.testing.assert_allclose(z, zc[:, :, -1], rtol=1e-12)


def test_noncausal_closed_form(orc):
    # phi(Q) (phi(K)^T V) / (phi(Q) . sum_j phi(k_j) + eps), two library matmuls
    rng = np.random.default_rng(4)
    B, H, N, dk, dv = 2, 2, 33, 8, 4
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    for phi, om, s in (("elu1", None, 1.0), ("trig_rf", make_omega(16, dk, 9), dk ** -0.25),
                       ("relu", None, 1.0), ("trig_rf_softmax", make_omega(16, dk, 9), dk ** -0.25)):
        y = orc.noncausal(q, k, v, 1e-6, phi, om, s)
        pq, pk = orc.phi_map(q, phi, om, s), orc.phi_map(k, phi, om, s)
        KV = np.swapaxes(pk, -1, -2) @ v
        num = pq @ KV
        den = pq @ pk.sum(axis=2)[..., None]
        np.testing.assert_allclose(y, num / (den + 1e-6), rtol=1e-11, atol=1e-14)


def test_golden_handcheck(orc):
    with open(os.path.join(GOLDEN, "handcheck_elu1_N2_d4.json")) as fh:
        g = json.load(fh)
    q = np.array(g["q"], dtype=float)[None, None]
    k = np.array(g["k"], dtype=float)[None, None]
    v = np.array(g["v"], dtype=float)[None, None]
    num = np.array([[float(Fraction(x)) for x in row] for row in g["num"]])
    den = np.array([float(Fraction(x)) for x in g["den"]])
    for eps in (0.0, 1e-6):
        y, S, z = orc.causal(q, k, v, [g["lambda"]], eps, want_state=True)
        np.testing.assert_allclose(y[0, 0], num / (den[:, None] + eps), rtol=1e-15)
    Sf = np.array([[float(Fraction(x)) for x in row] for row in g["S_final"]])
    zf = np.array([float(Fraction(x)) for x in g["z_final"]])
    np.testing.assert_array_equal(S[0, 0], Sf)
    np.testing.assert_array_equal(z[0, 0], zf)


# ---------------------------------------------------------------- invariants
def test_invariants_single_token_and_constant_v(orc):
    rng = np.random.default_rng(5)
    B, H, dk, dv = 1, 2, 4, 3
    eps = 1e-6
    # N = 1: y_0 = v_0 a / (a + eps), a = phi(q_0).phi(k_0)
    q, k, v = _rand(rng, B, H, 1, dk), _rand(rng, B, H, 1, dk), _rand(rng, B, H, 1, dv)
    y = orc.causal(q, k, v, [0.7, 0.2], eps)
    a = np.sum(orc.phi_map(q) * orc.phi_map(k), axis=-1)
    np.testing.assert_allclose(y, v * (a / (a + eps))[..., None], rtol=1e-14)
    # constant v_j = c: y_i = c den_i / (den_i + eps)
    N = 20
    q, k = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk)
    c = np.array([1.5, -2.0, 0.25])
    v = np.broadcast_to(c, (B, H, N, dv)).copy()
    y = orc.causal(q, k, v, [0.9, 1.0], eps)
    ratio = y / c
    np.testing.assert_allclose(ratio, ratio[..., :1].repeat(dv, -1), rtol=1e-12)
    assert np.all(ratio < 1.0) and np.all(ratio > 0.999)


def test_lambda_zero_is_diagonal(orc):
    # lambda = 0 (with 0^0 = 1): only the current token survives
    rng = np.random.default_rng(6)
    q, k, v = _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 4), _rand(rng, 1, 1, 9, 2)
    y = orc.causal(q, k, v, [0.0], 1e-6)
    a = np.sum(orc.phi_map(q) * orc.phi_map(k), axis=-1)
    np.testing.assert_allclose(y, v * (a / (a + 1e-6))[..., None], rtol=1e-14)


def test_linearity_in_v_and_permutation(orc):
    rng = np.random.default_rng(8)
    B, H, N, dk, dv = 2, 3, 15, 4, 2
    q, k = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk)
    v1, v2 = _rand(rng, B, H, N, dv), _rand(rng, B, H, N, dv)
    lam = [0.8, 0.95, 1.0]
    y1 = orc.causal(q, k, v1, lam)
    y2 = orc.causal(q, k, v2, lam)
    y12 = orc.causal(q, k, 2.0 * v1 - 0.5 * v2, lam)
    np.testing.assert_allclose(y12, 2.0 * y1 - 0.5 * y2, rtol=1e-10, atol=1e-12)
    # permuting batch rows permutes outputs (each (b,h) is independent)
    perm = [1, 0]
    yp = orc.causal(q[perm], k[perm], v1[perm], lam)
    np.testing.assert_allclose(yp, y1[perm], rtol=0, atol=0)


def test_split_resume_and_last_row_noncausal(orc):
    rng = np.random.default_rng(9)
    B, H, N, dk, dv = 1, 2, 40, 4, 3
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    lam = [0.9, 1.0]
    y, S, z = orc.causal(q, k, v, lam, want_state=True)
    n1 = 17
    ya, Sa, za = orc.causal(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], lam, want_state=True)
    yb, Sb, zb = orc.causal(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], lam, S0=Sa, z0=za,
                            want_state=True)
    np.testing.assert_allclose(np.concatenate([ya, yb], axis=2), y, rtol=1e-12)
    np.testing.assert_allclose(Sb, S, rtol=1e-12)
    np.testing.assert_allclose(zb, z, rtol=1e-12)
    # lambda = 1: the causal last row equals the non-causal row N-1
    y1 = orc.causal(q, k, v, [1.0, 1.0])
    yn = orc.noncausal(q, k, v)
    np.testing.assert_allclose(y1[:, :, -1], yn[:, :, -1], rtol=1e-12)


@pytest.mark.parametrize("phi", ["elu1", "relu"])
def test_decode_steps_match_bruteforce(orc, phi):
    # N decode steps from the zero state equal the quadratic form row by row
    rng = np.random.default_rng(10)
    B, H, N, dk, dv = 2, 2, 12, 4, 3
    lam = np.array([0.85, 1.0])
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    F = dk
    S = np.zeros((B, H, F, dv))
    z = np.zeros((B, H, F))
    ys = []
    for t in range(N):
        yt, S, z = orc.decode_step(q[:, :, t:t + 1], k[:, :, t:t + 1], v[:, :, t:t + 1],
                                   S, z, lam, 1e-6, phi)
        ys.append(yt)
    y = np.concatenate(ys, axis=2)
    pq, pk = orc.phi_map(q, phi), orc.phi_map(k, phi)
    for b in range(B):
        for h in range(H):
            np.testing.assert_allclose(y[b, h], _brute_force(pq[b, h], pk[b, h], v[b, h],
                                                             lam[h], 1e-6), rtol=1e-10)


@pytest.mark.parametrize("dv", [3, 4, 6])
def test_identity_initial_state_is_virtual_history(orc, dv):
    # "Attention is also an FFN", sec. 6: start S at the identity (a default
    # history).  S0 = alpha I (rectangular), z0 = alpha on the first min(F, dv)
    # features is the state of min(F, dv) virtual tokens phi(k) = e_f, v = e_f at
    # time -1, so token i reads it with weight alpha lam^(i+1):
    #   num_i = alpha lam^(i+1) phi(q_i)^T I + sum_{j<=i} lam^(i-j) (phi q_i . phi k_j) v_j
    #   den_i = alpha lam^(i+1) sum_{f<min(F,dv)} phi(q_i)_f + sum_{j<=i} lam^(i-j) phi q_i . phi k_j + eps
    rng = np.random.default_rng(40 + dv)
    B, H, N, dk = 1, 2, 19, 4
    alpha, eps = 0.7, 1e-6
    lam = np.array([0.8, 1.0])
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    F = dk
    eye = np.eye(F, dv)
    S0 = np.broadcast_to(alpha * eye, (B, H, F, dv)).copy()
    z0 = np.zeros((B, H, F))
    z0[..., :min(F, dv)] = alpha
    y = orc.causal(q, k, v, lam, eps, S0=S0, z0=z0)
    pq, pk = orc.phi_map(q), orc.phi_map(k)
    for h in range(H):
        for i in range(N):
            w0 = alpha * lam[h] ** (i + 1)
            num = w0 * (pq[0, h, i] @ eye)
            den = w0 * pq[0, h, i, :min(F, dv)].sum()
            for j in range(i + 1):
                a = lam[h] ** (i - j) * float(pq[0, h, i] @ pk[0, h, j])
                num = num + a * v[0, h, j]
                den += a
            np.testing.assert_allclose(y[0, h, i], num / (den + eps), rtol=1e-11, atol=1e-14)


def test_kappa_is_one_for_positive_features(orc):
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 1, 30, 4), _rand(rng, 1, 1, 30, 4), _rand(rng, 1, 1, 30, 2)
    # with eps = 0 the companion denominator equals |den| exactly for positive features
    _, kap = orc.causal(q, k, v, [0.9], 0.0, want_kappa=True)
    np.testing.assert_allclose(kap, 1.0, rtol=1e-12)


def test_rowwise_rel_err_definition(orc):
    ref = np.array([[1.0, -2.0, 0.0], [0.0, 0.0, 0.0]])
    y = np.array([[1.1, -2.0, 0.05], [0.0, 0.0, 0.0]])
    assert abs(orc.rowwise_rel_err(y, ref) - 0.05) < 1e-15


# ------------------------------------------------ masks, cross attention, var-len
def _brute_force_masked(pq, pk, v, lam, eps, keep):
    """O(N^2) quadratic form of one row with a key padding mask: a key with
    keep[j] == False is left out of numerator and denominator."""
    N = pq.shape[0]
    y = np.zeros((N, v.shape[1]))
    for i in range(N):
        num = np.zeros(v.shape[1])
        den = 0.0
        for j in range(i + 1):
            if not keep[j]:
                continue
            a = (1.0 if i == j else lam ** (i - j)) * float(pq[i] @ pk[j])
            num += a * v[j]
            den += a
        y[i] = num / (den + eps)
    return y


@pytest.mark.parametrize("phi,dk,m,lam", [("elu1", 4, 0, 0.9), ("elu1", 6, 0, 1.0),
                                          ("trig_rf", 4, 6, 0.95), ("relu", 4, 0, 0.8)])
def test_causal_key_padding_mask_bruteforce(orc, phi, dk, m, lam):
    rng = np.random.default_rng(zlib.crc32(repr(("kpm", phi, dk, lam)).encode()))
    B, H, N, dv = 2, 2, 29, 3
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    rf = phi.startswith("trig_rf")
    om = make_omega(m, dk, seed=5) if rf else None
    s = dk ** -0.25 if rf else 1.0
    mask = rng.random((B, N)) < 0.3
    mask[1, :4] = True  # leading padded keys: outputs 0 until the first kept key
    y, S, z = orc.causal(q, k, v, np.array([lam, lam]), 1e-6, phi, om, s,
                         want_state=True, key_padding_mask=mask)
    pq, pk = orc.phi_map(q, phi, om, s), orc.phi_map(k, phi, om, s)
    for b in range(B):
        for h in range(H):
            want = _brute_force_masked(pq[b, h], pk[b, h], v[b, h], lam, 1e-6, ~mask[b])
            np.testing.assert_allclose(y[b, h], want, rtol=1e-10, atol=1e-12)
            # final state: sum over kept keys of lam^(N-1-j) phi(k_j) [v_j, 1]^T
            w = np.where(mask[b], 0.0, lam ** (N - 1 - np.arange(N)))
            np.testing.assert_allclose(S[b, h], (pk[b, h] * w[:, None]).T @ v[b, h], rtol=1e-11)
            np.testing.assert_allclose(z[b, h], (pk[b, h] * w[:, None]).sum(0), rtol=1e-11)
    np.testing.assert_array_equal(y[1, :, :4], 0.0)


def test_causal_mask_none_and_all(orc):
    rng = np.random.default_rng(21)
    B, H, N, dk, dv = 2, 1, 17, 4, 3
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    S0, z0 = rng.standard_normal((B, H, dk, dv)), rng.random((B, H, dk)) + 0.5
    none = np.zeros((B, N), bool)
    a = orc.causal(q, k, v, [0.9], 1e-6, S0=S0, z0=z0, want_state=True)
    b = orc.causal(q, k, v, [0.9], 1e-6, S0=S0, z0=z0, want_state=True, key_padding_mask=none)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    # every key padded: the initial state decays untouched, y_i reads it
    y, S, z = orc.causal(q, k, v, [0.9], 1e-6, S0=S0, z0=z0, want_state=True,
                         key_padding_mask=~none)
    np.testing.assert_allclose(S, S0 * 0.9 ** N, rtol=1e-12)
    np.testing.assert_allclose(z, z0 * 0.9 ** N, rtol=1e-12)
    pq = orc.phi_map(q)
    li = 0.9 ** (np.arange(N) + 1)
    num = np.einsum("bhnf,bhfd->bhnd", pq, S0) * li[:, None]
    den = np.einsum("bhnf,bhf->bhn", pq, z0) * li
    np.testing.assert_allclose(y, num / (den[..., None] + 1e-6), rtol=1e-11)


@pytest.mark.parametrize("phi,m", [("elu1", 0), ("trig_rf", 8), ("relu", 0)])
def test_cross_closed_form_and_mask(orc, phi, m):
    # y = phi(Q) (phi(K)^T diag(keep) V) / (phi(Q) phi(K)^T keep + eps) with
    # two library matmuls; Nq != Nk
    rng = np.random.default_rng(zlib.crc32(repr(("cross", phi)).encode()))
    B, H, Nq, Nk, dk, dv = 2, 3, 11, 23, 8, 5
    q, k, v = _rand(rng, B, H, Nq, dk), _rand(rng, B, H, Nk, dk), _rand(rng, B, H, Nk, dv)
    rf = phi.startswith("trig_rf")
    om = make_omega(m, dk, seed=3) if rf else None
    s = dk ** -0.25 if rf else 1.0
    mask = rng.random((B, Nk)) < 0.4
    pq, pk = orc.phi_map(q, phi, om, s), orc.phi_map(k, phi, om, s)
    for kpm in (None, mask):
        keep = np.ones((B, Nk)) if kpm is None else (~kpm).astype(float)
        y = orc.cross(q, k, v, 1e-6, phi, om, s, key_padding_mask=kpm)
        pkk = pk * keep[:, None, :, None]
        num = pq @ (np.swapaxes(pkk, -1, -2) @ v)
        den = pq @ pkk.sum(axis=2)[..., None]
        np.testing.assert_allclose(y, num / (den + 1e-6), rtol=1e-11, atol=1e-14)


def test_cross_reduces_to_noncausal_and_to_key_subset(orc):
    rng = np.random.default_rng(22)
    B, H, N, dk, dv = 1, 2, 19, 4, 3
    q, k, v = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dv)
    # Nq == Nk and no mask: the self-attention non-causal form (its own C loop)
    np.testing.assert_allclose(orc.cross(q, k, v, 1e-6), orc.noncausal(q, k, v, 1e-6),
                               rtol=1e-13)
    # a mask equals dropping the masked keys and values
    mask = np.zeros((B, N), bool)
    mask[0, [0, 3, 4, 11, 18]] = True
    keep = ~mask[0]
    np.testing.assert_allclose(orc.cross(q, k, v, 1e-6, key_padding_mask=mask),
                               orc.cross(q, k[:, :, keep], v[:, :, keep], 1e-6), rtol=1e-13)
    # a single key: every query returns that key's value (up to eps)
    y1 = orc.cross(q, k[:, :, :1], v[:, :, :1], 0.0)
    np.testing.assert_allclose(y1, np.broadcast_to(v[:, :, :1], y1.shape), rtol=1e-12)


def test_varlen_per_sequence_bruteforce(orc):
    rng = np.random.default_rng(23)
    H, dk, dv, lam = 2, 4, 3, 0.85
    lens = [5, 0, 13, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1]) + 3  # three trailing tokens belong to no sequence
    q, k, v = _rand(rng, 1, H, T, dk), _rand(rng, 1, H, T, dk), _rand(rng, 1, H, T, dv)
    B = len(lens)
    S0, z0 = rng.standard_normal((B, H, dk, dv)), rng.random((B, H, dk)) + 0.5
    y, S, z = orc.causal_varlen(q, k, v, cu, lam=[lam, 0.5], S0=S0, z0=z0)
    pq, pk = orc.phi_map(q), orc.phi_map(k)
    for h, lh in enumerate([lam, 0.5]):
        for b in range(B):
            lo, hi = cu[b], cu[b + 1]
            St, zt = S0[b, h].copy(), z0[b, h].copy()
            for i in range(lo, hi):  # the recurrence restarted at each sequence
                St = lh * St + np.outer(pk[0, h, i], v[0, h, i])
                zt = lh * zt + pk[0, h, i]
                want = pq[0, h, i] @ St / (pq[0, h, i] @ zt + 1e-6)
                np.testing.assert_allclose(y[0, h, i], want, rtol=1e-11)
            np.testing.assert_allclose(S[b, h], St, rtol=1e-12)
            np.testing.assert_allclose(z[b, h], zt, rtol=1e-12)
    np.testing.assert_array_equal(y[:, :, cu[-1]:], 0.0)


def test_varlen_single_sequence_and_reordering(orc):
    rng = np.random.default_rng(24)
    H, T, dk, dv = 2, 31, 4, 3
    q, k, v = _rand(rng, 1, H, T, dk), _rand(rng, 1, H, T, dk), _rand(rng, 1, H, T, dv)
    y1, S1, z1 = orc.causal_varlen(q, k, v, [0, T], lam=[0.9, 1.0])
    y, S, z = orc.causal(q, k, v, [0.9, 1.0], want_state=True)
    np.testing.assert_array_equal(y1, y)
    np.testing.assert_array_equal(S1, S)
    # swapping two packed sequences swaps their outputs and states
    a, b = 12, T - 12
    perm = np.r_[a:T, 0:a]
    yp, Sp, zp = orc.causal_varlen(q[:, :, perm], k[:, :, perm], v[:, :, perm], [0, b, T],
                                   lam=[0.9, 1.0])
    ys, Ss, zs = orc.causal_varlen(q, k, v, [0, a, T], lam=[0.9, 1.0])
    np.testing.assert_allclose(yp[:, :, :b], ys[:, :, a:], rtol=1e-13)
    np.testing.assert_allclose(yp[:, :, b:], ys[:, :, :a], rtol=1e-13)
    np.testing.assert_allclose(Sp[[1, 0]], Ss, rtol=1e-13)
    np.testing.assert_allclose(zp[[1, 0]], zs, rtol=1e-13)


# ------------------------------------------------------------------ backward
def _torch_quadratic_loss(q, k, v, g, lam, eps, phi, omega, scale, S0, z0, dS_out, dz_out, keep):
    """The causal forward written as the O(N^2) quadratic form in torch fp64
    (not the recurrence), plus the final-state terms, as a scalar loss."""
    import torch
    if phi == "elu1":
        pq, pk = torch.nn.functional.elu(q) + 1.0, torch.nn.functional.elu(k) + 1.0
    elif phi == "relu":
        pq, pk = torch.relu(q), torch.relu(k)
    else:
        sgn = {"trig_rf": -1.0, "trig_rf_plain": 0.0, "trig_rf_softmax": 1.0}[phi]
        m = omega.shape[0]

        def rf(x):
            xs = scale * x
            u = xs @ omega.T
            c = torch.exp(0.5 * sgn * (xs * xs).sum(-1, keepdim=True)) / math.sqrt(m)
            return c * torch.cat([torch.cos(u), torch.sin(u)], -1)
        pq, pk = rf(q), rf(k)
    pk = pk * keep[:, None, :, None]
    B, H, N, _ = q.shape
    idx = torch.arange(N, dtype=torch.float64)
    E = idx[:, None] - idx[None, :]
    causal = (E >= 0).to(torch.float64)
    lamh = lam.reshape(1, H, 1, 1)
    W = torch.pow(lamh, E.clamp(min=0)) * causal                      # lambda^(i-j), j <= i
    A = (pq @ pk.transpose(-1, -2)) * W
    li = torch.pow(lamh.reshape(1, H, 1), idx + 1)                    # lambda^(i+1)
    num = A @ v + li[..., None] * (pq @ S0)
    den = A.sum(-1) + li * (pq * z0[:, :, None, :]).sum(-1) + eps
    y = num / den[..., None]
    wN = torch.pow(lamh.reshape(1, H, 1), (N - 1 - idx))              # lambda^(N-1-j)
    S_fin = (pk * wN[..., None]).transpose(-1, -2) @ v + torch.pow(lam, N).reshape(1, H, 1, 1) * S0
    z_fin = (pk * wN[..., None]).sum(2) + torch.pow(lam, N).reshape(1, H, 1) * z0
    return (g * y).sum() + (dS_out * S_fin).sum() + (dz_out * z_fin).sum()


@pytest.mark.parametrize("phi,dk,m,lams,masked", [
    ("elu1", 4, 0, (0.9, 1.0), False), ("elu1", 6, 0, (0.3, 0.95), True),
    ("relu", 4, 0, (0.8, 1.0), True), ("trig_rf", 4, 6, (0.9, 0.99), False),
    ("trig_rf_softmax", 4, 4, (1.0, 0.7), False), ("trig_rf_plain", 6, 4, (0.6, 0.9), True)])
def test_backward_matches_torch_autograd_of_quadratic_form(orc, phi, dk, m, lams, masked):
    import torch
    rng = np.random.default_rng(zlib.crc32(repr(("bwd", phi, dk, lams)).encode()))
    B, H, N, dv = 2, 2, 19, 3
    q, k, v, g = (_rand(rng, B, H, N, d) for d in (dk, dk, dv, dv))
    rf = phi.startswith("trig_rf")
    om = make_omega(m, dk, seed=5) if rf else None
    s = dk ** -0.25 if rf else 1.0
    F = 2 * m if rf else dk
    S0 = rng.standard_normal((B, H, F, dv)) * 0.2
    z0 = rng.random((B, H, F)) + 0.5 if not rf else rng.standard_normal((B, H, F)) * 0.05
    dS_out, dz_out = rng.standard_normal((B, H, F, dv)), rng.standard_normal((B, H, F))
    mask = (rng.random((B, N)) < 0.3) if masked else None
    got = orc.backward(q, k, v, g, np.array(lams), 1e-6, phi, om, s, S0, z0, dS_out, dz_out,
                       key_padding_mask=mask)
    t = {n: torch.tensor(a, dtype=torch.float64, requires_grad=True)
         for n, a in (("q", q), ("k", k), ("v", v), ("S0", S0), ("z0", z0), ("lam", np.array(lams)))}
    keep = torch.ones(B, N, dtype=torch.float64) if mask is None else torch.tensor(~mask, dtype=torch.float64)
    loss = _torch_quadratic_loss(t["q"], t["k"], t["v"], torch.tensor(g), t["lam"], 1e-6, phi,
                                 None if om is None else torch.tensor(om, dtype=torch.float64), s,
                                 t["S0"], t["z0"], torch.tensor(dS_out), torch.tensor(dz_out), keep)
    loss.backward()
    for name, ref in (("dq", t["q"].grad), ("dk", t["k"].grad), ("dv", t["v"].grad),
                      ("dS0", t["S0"].grad), ("dz0", t["z0"].grad)):
        np.testing.assert_allclose(got[name], ref.numpy(), rtol=1e-9, atol=1e-11, err_msg=name)
    np.testing.assert_allclose(got["dlam"].sum(0), t["lam"].grad.numpy(), rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("lams,masked", [((0.0, 0.93), False), ((0.5, 1.0), True)])
def test_backward_directional_finite_differences(orc, lams, masked):
    # <grad, delta> against central differences of the forward oracle, for every
    # input at once (step 1e-5: truncation ~1e-10, well inside the bound).
    # lambda = 0 is included (the recurrence is a polynomial in lambda), but
    # not with a mask: a padded key then leaves den = eps, where the loss is
    # too curved for a finite difference.
    rng = np.random.default_rng(31)
    B, H, N, dk, dv = 1, 2, 40, 4, 3
    q, k, v, g = (_rand(rng, B, H, N, d) for d in (dk, dk, dv, dv))
    S0, z0 = rng.standard_normal((B, H, dk, dv)) * 0.2, rng.random((B, H, dk)) + 0.5
    dS_out, dz_out = rng.standard_normal((B, H, dk, dv)), rng.standard_normal((B, H, dk))
    lam = np.array(lams)
    mask = (rng.random((B, N)) < 0.2) if masked else None
    gr = orc.backward(q, k, v, g, lam, 1e-6, S0=S0, z0=z0, dS_out=dS_out, dz_out=dz_out,
                      key_padding_mask=mask)
    d = {n: rng.standard_normal(a.shape) for n, a in (("q", q), ("k", k), ("v", v), ("S0", S0),
                                                      ("z0", z0), ("lam", lam))}

    def loss(h):
        y, S, z = orc.causal(q + h * d["q"], k + h * d["k"], v + h * d["v"], lam + h * d["lam"], 1e-6,
                             S0=S0 + h * d["S0"], z0=z0 + h * d["z0"], want_state=True,
                             key_padding_mask=mask)
        return (g * y).sum() + (dS_out * S).sum() + (dz_out * z).sum()

    hstep = 1e-5
    fd = (loss(hstep) - loss(-hstep)) / (2 * hstep)
    an = sum((gr[n] * d[x]).sum() for n, x in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dS0", "S0"),
                                               ("dz0", "z0")))
    an += (gr["dlam"].sum(0) * d["lam"]).sum()
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


@pytest.mark.parametrize("phi,m", [("elu1", 0), ("relu", 0), ("trig_rf", 5), ("trig_rf_softmax", 3),
                                   ("trig_rf_plain", 4)])
def test_phi_vjp_finite_differences(orc, phi, m):
    rng = np.random.default_rng(zlib.crc32(phi.encode()))
    dk = 6
    om = make_omega(m, dk, seed=2) if m else None
    s = 0.7 if m else 1.0
    x = rng.standard_normal((5, dk))
    x[np.abs(x) < 1e-2] += 0.1  # keep ReLU away from its kink
    F = 2 * m if m else dk
    dp = rng.standard_normal((5, F))
    got = orc.phi_vjp(x, dp, phi, om, s)
    h = 1e-6
    for c in range(dk):
        e = np.zeros(dk)
        e[c] = h
        fd = ((orc.phi_map(x + e, phi, om, s) - orc.phi_map(x - e, phi, om, s)) / (2 * h) * dp).sum(-1)
        np.testing.assert_allclose(got[:, c], fd, rtol=1e-6, atol=1e-8)


def test_backward_without_tokens_passes_state_gradient(orc):
    rng = np.random.default_rng(32)
    dS = rng.standard_normal((1, 1, 4, 3))
    dz = rng.standard_normal((1, 1, 4))
    q = np.zeros((1, 1, 0, 4))
    v = np.zeros((1, 1, 0, 3))
    gr = orc.backward(q, q, v, v, [0.5], dS_out=dS, dz_out=dz)
    np.testing.assert_array_equal(gr["dS0"], dS)
    np.testing.assert_array_equal(gr["dz0"], dz)
    assert gr["dlam"][0, 0] == 0.0


def test_backward_kappa_bounds(orc):
    # kappa >= 1 always; no cancellation (positive features, positive dy, and
    # values making every term of dv positive) gives kappa_dv = 1; the first
    # token's dq cancels exactly but for eps (kappa huge)
    rng = np.random.default_rng(33)
    B, H, N, dk, dv = 1, 2, 30, 4, 3
    q, k = _rand(rng, B, H, N, dk), _rand(rng, B, H, N, dk)
    v, g = _rand(rng, B, H, N, dv), np.abs(_rand(rng, B, H, N, dv)) + 0.1
    r = orc.backward(q, k, v, g, [0.9, 1.0], want_kappa=True)
    for n in ("kappa_dq", "kappa_dk", "kappa_dv"):
        assert np.all(r[n] >= 1.0 - 1e-12), n
    np.testing.assert_allclose(r["kappa_dv"], 1.0, rtol=1e-12)
    assert np.all(r["kappa_dq"][:, :, 0] > 1e6)
    # the gradients themselves are unchanged by asking for kappa
    r0 = orc.backward(q, k, v, g, [0.9, 1.0])
    for n in ("dq", "dk", "dv", "dS0", "dz0", "dlam"):
        np.testing.assert_array_equal(r[n], r0[n])


@pytest.mark.parametrize("phi,m,masked", [("elu1", 0, False), ("relu", 0, True), ("trig_rf", 6, True)])
def test_cross_backward_matches_torch_autograd(orc, phi, m, masked):
    # the non-causal closed form phi(Q)(phi(K)^T V) / (phi(Q) sum phi(k) + eps)
    # in torch fp64, differentiated by autograd; Nq != Nk
    import torch
    rng = np.random.default_rng(zlib.crc32(repr(("xbwd", phi)).encode()))
    B, H, Nq, Nk, dk, dv = 2, 2, 9, 14, 4, 3
    q, k, v, g = _rand(rng, B, H, Nq, dk), _rand(rng, B, H, Nk, dk), _rand(rng, B, H, Nk, dv), _rand(rng, B, H, Nq, dv)
    rf = phi.startswith("trig_rf")
    om = make_omega(m, dk, seed=2) if rf else None
    s = dk ** -0.25 if rf else 1.0
    mask = (rng.random((B, Nk)) < 0.3) if masked else None
    got = orc.cross_backward(q, k, v, g, 1e-6, phi, om, s, key_padding_mask=mask)
    t = {n: torch.tensor(a, requires_grad=True) for n, a in (("q", q), ("k", k), ("v", v))}

    def feat(x):
        if phi == "elu1":
            return torch.nn.functional.elu(x) + 1.0
        if phi == "relu":
            return torch.relu(x)
        xs = s * x
        uu = xs @ torch.tensor(om, dtype=torch.float64).T
        c = torch.exp(-0.5 * (xs * xs).sum(-1, keepdim=True)) / math.sqrt(m)
        return c * torch.cat([torch.cos(uu), torch.sin(uu)], -1)

    pq, pk = feat(t["q"]), feat(t["k"])
    if mask is not None:
        pk = pk * torch.tensor(~mask, dtype=torch.float64)[:, None, :, None]
    y = (pq @ (pk.transpose(-1, -2) @ t["v"])) / (pq @ pk.sum(2)[..., None] + 1e-6)
    (torch.tensor(g) * y).sum().backward()
    for n in ("q", "k", "v"):
        np.testing.assert_allclose(got["d" + n], t[n].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=n)


def test_cross_backward_finite_differences_and_noncausal_case(orc):
    rng = np.random.default_rng(34)
    B, H, Nq, Nk, dk, dv = 1, 2, 7, 11, 4, 3
    q, k, v, g = _rand(rng, B, H, Nq, dk), _rand(rng, B, H, Nk, dk), _rand(rng, B, H, Nk, dv), _rand(rng, B, H, Nq, dv)
    gr = orc.cross_backward(q, k, v, g)
    d = {n: rng.standard_normal(a.shape) for n, a in (("q", q), ("k", k), ("v", v))}

    def loss(h):
        return (g * orc.cross(q + h * d["q"], k + h * d["k"], v + h * d["v"])).sum()

    fd = (loss(1e-5) - loss(-1e-5)) / 2e-5
    an = sum((gr["d" + n] * d[n]).sum() for n in ("q", "k", "v"))
    assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_cross_backward_kappa_bounds(orc):
    # kappa >= 1; positive dy makes every term of dv positive (kappa_dv = 1);
    # with a single key y_i = v (but for eps) whatever q_i and k are, so dq
    # and dk cancel down to the eps term (kappa huge) while their terms do not
    rng = np.random.default_rng(35)
    B, H, Nq, Nk, dk, dv = 1, 2, 9, 13, 4, 3
    q, k, v = _rand(rng, B, H, Nq, dk), _rand(rng, B, H, Nk, dk), _rand(rng, B, H, Nk, dv)
    g = np.abs(_rand(rng, B, H, Nq, dv)) + 0.1
    r = orc.cross_backward(q, k, v, g, want_kappa=True)
    for n in ("kappa_dq", "kappa_dk", "kappa_dv"):
        assert np.all(r[n] >= 1.0 - 1e-12), n
    np.testing.assert_allclose(r["kappa_dv"], 1.0, rtol=1e-12)
    r0 = orc.cross_backward(q, k, v, g)
    for n in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(r[n], r0[n])
    one = orc.cross_backward(q, k[:, :, :1], v[:, :, :1], g, want_kappa=True)
    assert np.all(one["kappa_dq"] > 1e4) and np.all(one["kappa_dk"] > 1e4)
