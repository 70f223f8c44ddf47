"""Pins of the fp64 gradient oracle (oracle/la_backward.py).

The gradients are checked against central finite differences of the forward
oracle (itself pinned in test_oracle_pins.py), against closed forms for
uniform features, and against the scale invariance of the normalised output,
so a dropped term, a wrong sign of the normaliser's gradient, a transposed
weight matrix or a wrong feature-map derivative fails at least one of them.
"""
import numpy as np
import pytest

import oracle as orc
from oracle import la_backward as bwd

RNG = np.random.default_rng(4321)


def _loss(Q, K, V, dO, fmap, omega, causal, gate, eps, S0=None, z0=None):
    if causal:
        o, _, _ = orc.causal_recurrent(Q, K, V, fmap, omega, gate, eps, S0=S0, z0=z0)
    else:
        o = orc.noncausal(Q, K, V, fmap, omega, eps)
    return float(np.sum(o * dO))


CASES = [("elu1", False, "none", False), ("elu1", True, "none", False), ("elu1", True, "decay", False),
         ("elu1", True, "decay", True), ("elu1", True, "none", True), ("favor", False, "none", False),
         ("favor", True, "none", True), ("favor", True, "decay", False),
         ("identity", True, "none", False), ("identity", True, "decay", True)]


@pytest.mark.parametrize("fmap,causal,gate_kind,with_state", CASES)
def test_gradients_match_finite_differences(fmap, causal, gate_kind, with_state):
    """Directional derivatives of L = sum dO . o along random directions equal
    <grad, direction> (central differences, step 1e-6, fp64)."""
    B, H, n, d, e = 1, 2, 9, 5, 3
    r = 8 if fmap == "favor" else d
    Q = RNG.standard_normal((B, H, n, d)) * 0.7
    K = RNG.standard_normal((B, H, n, d)) * 0.7
    V = RNG.standard_normal((B, H, n, e))
    dO = RNG.standard_normal((B, H, n, e))
    omega = RNG.standard_normal((r, d)) if fmap == "favor" else None
    gate = ("decay", np.array([0.9, 0.6])) if gate_kind == "decay" else None
    S0 = z0 = None
    if with_state:
        S0 = np.abs(RNG.standard_normal((B, H, r, e)))
        z0 = np.abs(RNG.standard_normal((B, H, r))) + 0.5
    eps = 1e-3
    dQ, dK, dV = bwd.backward(Q, K, V, dO, fmap, omega, causal, gate, eps, S0, z0)
    step = 1e-6
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        U = RNG.standard_normal(X.shape)
        args = {"Q": Q, "K": K, "V": V}
        args[name] = X + step * U
        lp = _loss(args["Q"], args["K"], args["V"], dO, fmap, omega, causal, gate, eps, S0, z0)
        args[name] = X - step * U
        lm = _loss(args["Q"], args["K"], args["V"], dO, fmap, omega, causal, gate, eps, S0, z0)
        fd = (lp - lm) / (2 * step)
        an = float(np.sum(G * U))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_uniform_features_closed_form():
    """Q = K = 0 gives phi = 1 (elu+1), so W_ij = d for j <= i and causal
    o_i = d sum_{j<=i} v_j / (d (i + 1) + eps). Then dV_j = d sum_{i>=j} dO_i / den_i,
    and every entry of dQ_i is eps (dO_i . o_i) / (d den_i): the output depends
    on the scale of phi(q_i) only through eps."""
    B, H, n, d, e = 1, 1, 12, 4, 3
    Q = np.zeros((B, H, n, d))
    K = np.zeros((B, H, n, d))
    V = RNG.standard_normal((B, H, n, e))
    dO = RNG.standard_normal((B, H, n, e))
    eps = 0.25
    dQ, dK, dV = bwd.backward(Q, K, V, dO, "elu1", None, True, None, eps)
    den = d * np.arange(1, n + 1) + eps
    o = d * np.cumsum(V[0, 0], axis=0) / den[:, None]
    want_dV = np.array([d * np.sum(dO[0, 0, j:] / den[j:, None], axis=0) for j in range(n)])
    np.testing.assert_allclose(dV[0, 0], want_dV, rtol=1e-13, atol=1e-13)
    want_dQ = eps * np.sum(dO[0, 0] * o, axis=1) / (d * den)
    np.testing.assert_allclose(dQ[0, 0], np.repeat(want_dQ[:, None], d, axis=1), rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("causal,gate_kind", [(False, "none"), (True, "none"), (True, "decay")])
def test_output_invariant_to_query_feature_scale(causal, gate_kind):
    """With eps = 0, o_i depends on phi(q_i) only through its direction, so
    sum_f dL/dphi(q_i)_f phi(q_i)_f = 0. With all q > 0, elu+1 has phi' = 1 and
    phi(q) = q + 1, so this reads sum_f dQ_if (q_if + 1) = 0."""
    B, H, n, d, e = 1, 2, 10, 6, 4
    Q = np.abs(RNG.standard_normal((B, H, n, d))) + 0.1
    K = RNG.standard_normal((B, H, n, d))
    V = RNG.standard_normal((B, H, n, e))
    dO = RNG.standard_normal((B, H, n, e))
    gate = ("decay", np.array([0.8, 0.95])) if gate_kind == "decay" else None
    dQ, _, _ = bwd.backward(Q, K, V, dO, "elu1", None, causal, gate, 0.0)
    s = np.sum(dQ * (Q + 1.0), axis=-1)
    assert np.max(np.abs(s)) < 1e-12 * np.max(np.abs(dQ))


@pytest.mark.parametrize("fmap,with_state", [("elu1", False), ("elu1", True), ("identity", False),
                                             ("identity", True)])
def test_gla_gradients_match_finite_differences(fmap, with_state):
    """dQ, dK, dV and the gradient of the raw gate input g of the GLA form,
    against central differences of the recurrent oracle (which applies the gate
    step by step and is pinned against the explicit weights)."""
    B, H, n, d, e = 1, 2, 8, 4, 3
    tau = 3.0
    Q = RNG.standard_normal((B, H, n, d)) * 0.7
    K = RNG.standard_normal((B, H, n, d)) * 0.7
    V = RNG.standard_normal((B, H, n, e))
    G = RNG.standard_normal((B, H, n, d))
    dO = RNG.standard_normal((B, H, n, e))
    S0 = z0 = None
    if with_state:
        S0 = np.abs(RNG.standard_normal((B, H, d, e)))
        z0 = np.abs(RNG.standard_normal((B, H, d))) + 0.5
    eps = 1e-3
    dQ, dK, dV, dg = bwd.backward_gla(Q, K, V, dO, G, tau, fmap, None, eps, S0, z0)

    def loss(Q_, K_, V_, G_):
        o, _, _ = orc.causal_recurrent(Q_, K_, V_, fmap, None, ("gla", G_, tau), eps, S0=S0, z0=z0)
        return float(np.sum(o * dO))
    step = 1e-6
    for idx, (X, Gr) in enumerate(((Q, dQ), (K, dK), (V, dV), (G, dg))):
        U = RNG.standard_normal(X.shape)
        args = [Q, K, V, G]
        args[idx] = X + step * U
        lp = loss(*args)
        args[idx] = X - step * U
        lm = loss(*args)
        fd = (lp - lm) / (2 * step)
        an = float(np.sum(Gr * U))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (idx, fd, an)


def test_gla_unit_gates_reduce_to_ungated():
    """Gates that are exactly 1 (g = +inf) leave dQ, dK, dV of the ungated form
    and give dg = 0."""
    B, H, n, d, e = 1, 1, 7, 4, 3
    Q = RNG.standard_normal((B, H, n, d))
    K = RNG.standard_normal((B, H, n, d))
    V = RNG.standard_normal((B, H, n, e))
    dO = RNG.standard_normal((B, H, n, e))
    G = np.full((B, H, n, d), np.inf)
    got = bwd.backward_gla(Q, K, V, dO, G, 16.0, "elu1", None, 1e-3)
    want = bwd.backward(Q, K, V, dO, "elu1", None, True, None, 1e-3)
    for a, b in zip(got[:3], want):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    assert np.all(got[3] == 0.0)


@pytest.mark.parametrize("fmap,with_state", [("elu1", False), ("elu1", True), ("identity", True)])
def test_outer_gradients_match_finite_differences(fmap, with_state):
    """The outer-product gate: dQ, dK, dV and the gradients of both raw gate
    inputs (g per feature, gv per value column) against central differences of
    the recurrent oracle, which applies (alpha_t beta_t^T) * S step by step."""
    B, H, n, d, e = 1, 2, 8, 4, 3
    tau = 3.0
    Q = RNG.standard_normal((B, H, n, d)) * 0.7
    K = RNG.standard_normal((B, H, n, d)) * 0.7
    V = RNG.standard_normal((B, H, n, e))
    G = RNG.standard_normal((B, H, n, d))
    GV = RNG.standard_normal((B, H, n, e))
    dO = RNG.standard_normal((B, H, n, e))
    S0 = z0 = None
    if with_state:
        S0 = RNG.standard_normal((B, H, d, e))
        z0 = np.abs(RNG.standard_normal((B, H, d))) + 0.5
    eps = 1e-3
    grads = bwd.backward_outer(Q, K, V, dO, G, GV, tau, fmap, None, eps, S0, z0)
    assert grads[3].shape == G.shape and grads[4].shape == GV.shape

    def loss(Q_, K_, V_, G_, GV_):
        o, _, _ = orc.causal_recurrent(Q_, K_, V_, fmap, None, ("outer", G_, GV_, tau), eps, S0=S0, z0=z0)
        return float(np.sum(o * dO))
    step = 1e-6
    for idx, (X, Gr) in enumerate(zip((Q, K, V, G, GV), grads)):
        U = RNG.standard_normal(X.shape)
        args = [Q, K, V, G, GV]
        args[idx] = X + step * U
        lp = loss(*args)
        args[idx] = X - step * U
        lm = loss(*args)
        fd = (lp - lm) / (2 * step)
        an = float(np.sum(Gr * U))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (idx, fd, an)


def test_outer_unit_value_gate_reduces_to_gla():
    """beta = 1 (gv = +inf) is the GLA gate: the same dQ, dK, dV, dg as
    backward_gla, and dgv = 0."""
    B, H, n, d, e = 1, 2, 7, 4, 3
    Q = RNG.standard_normal((B, H, n, d))
    K = RNG.standard_normal((B, H, n, d))
    V = RNG.standard_normal((B, H, n, e))
    G = RNG.standard_normal((B, H, n, d))
    dO = RNG.standard_normal((B, H, n, e))
    S0 = RNG.standard_normal((B, H, d, e))
    z0 = np.abs(RNG.standard_normal((B, H, d))) + 0.5
    GV = np.full((B, H, n, e), np.inf)
    got = bwd.backward_outer(Q, K, V, dO, G, GV, 2.0, "elu1", None, 1e-3, S0, z0)
    want = bwd.backward_gla(Q, K, V, dO, G, 2.0, "elu1", None, 1e-3, S0, z0)
    for a, b in zip(got[:4], want):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    assert np.all(got[4] == 0.0)


def test_outer_single_step_value_gate_closed_form():
    """One step after a carried state: o_e = (beta_e phi(q)^T S0[:, e] + w v_e) /
    (phi(q).z0 + w + eps) with w = phi(q).phi(k) (alpha = 1, beta_e =
    sigmoid(gv_e)^(1/tau)); dL/dgv_e = dO_e phi(q)^T S0[:, e] / den *
    beta_e sigmoid(-gv_e) / tau."""
    d, e, tau, eps = 3, 2, 4.0, 1e-3
    q = RNG.standard_normal(d)
    k = RNG.standard_normal(d)
    v = RNG.standard_normal(e)
    dO = RNG.standard_normal(e)
    S0 = RNG.standard_normal((d, e))
    z0 = np.abs(RNG.standard_normal(d)) + 0.5
    gv = np.array([0.3, -1.1])
    pq, pk = orc.feature_map(q, "elu1"), orc.feature_map(k, "elu1")
    beta = (1.0 / (1.0 + np.exp(-gv))) ** (1.0 / tau)
    den = pq @ z0 + pq @ pk + eps
    want = dO * (pq @ S0) / den * beta * (1.0 / (1.0 + np.exp(gv))) / tau
    sh = lambda x: x.reshape((1, 1) + x.shape)
    got = bwd.backward_outer(sh(q[None]), sh(k[None]), sh(v[None]), sh(dO[None]), np.full((1, 1, 1, d), np.inf),
                             sh(gv[None]), tau, "elu1", None, eps, sh(S0), sh(z0))[4]
    np.testing.assert_allclose(got[0, 0, 0], want, rtol=1e-12, atol=1e-15)


def test_identity_gradients_closed_form():
    """The state-space read-out y = tril(Q K^T) V is bilinear: dV = tril(Q K^T)^T dO,
    dQ = tril(dO V^T) K, dK = tril(dO V^T)^T Q (numpy matmuls)."""
    B, H, n, d, e = 1, 1, 7, 4, 3
    Q = RNG.standard_normal((B, H, n, d))
    K = RNG.standard_normal((B, H, n, d))
    V = RNG.standard_normal((B, H, n, e))
    dO = RNG.standard_normal((B, H, n, e))
    dQ, dK, dV = bwd.backward(Q, K, V, dO, "identity", None, True, None, 1e-6)
    A = np.tril(Q[0, 0] @ K[0, 0].T)
    M = np.tril(dO[0, 0] @ V[0, 0].T)
    np.testing.assert_allclose(dV[0, 0], A.T @ dO[0, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dQ[0, 0], M @ K[0, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dK[0, 0], M.T @ Q[0, 0], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmap,with_state", [("elu1", False), ("elu1", True), ("identity", True)])
def test_sel_gradients_match_finite_differences(fmap, with_state):
    """The selective scalar gate: dQ, dK, dV and the gradient of its raw
    per-step input g [B, H, n], against central differences of the recurrent
    oracle, which applies a_t = sigmoid(g_t)^(1/tau) step by step."""
    B, H, n, d, e = 1, 2, 9, 4, 3
    tau = 2.0
    Q = RNG.standard_normal((B, H, n, d)) * 0.7
    K = RNG.standard_normal((B, H, n, d)) * 0.7
    V = RNG.standard_normal((B, H, n, e))
    G = RNG.standard_normal((B, H, n))
    dO = RNG.standard_normal((B, H, n, e))
    S0 = z0 = None
    if with_state:
        S0 = np.abs(RNG.standard_normal((B, H, d, e)))
        z0 = np.abs(RNG.standard_normal((B, H, d))) + 0.5
    eps = 1e-3
    dQ, dK, dV, dg = bwd.backward_sel(Q, K, V, dO, G, tau, fmap, None, eps, S0, z0)
    assert dg.shape == G.shape

    def loss(Q_, K_, V_, G_):
        o, _, _ = orc.causal_recurrent(Q_, K_, V_, fmap, None, ("sel", G_, tau), eps, S0=S0, z0=z0)
        return float(np.sum(o * dO))
    step = 1e-6
    for idx, (X, Gr) in enumerate(((Q, dQ), (K, dK), (V, dV), (G, dg))):
        U = RNG.standard_normal(X.shape)
        args = [Q, K, V, G]
        args[idx] = X + step * U
        lp = loss(*args)
        args[idx] = X - step * U
        lm = loss(*args)
        fd = (lp - lm) / (2 * step)
        an = float(np.sum(Gr * U))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (idx, fd, an)


def test_sel_single_step_gate_gradient_closed_form():
    """One step after a carried state: o = (a phi(q)^T S0 + phi(q)^T phi(k) v) /
    (a phi(q).z0 + phi(q).phi(k) + eps) with a = sigmoid(g)^(1/tau), so
    dL/dg = dL/da * a sigmoid(-g) / tau, with dL/da by the quotient rule."""
    d, e, tau, eps = 3, 2, 4.0, 1e-3
    q = RNG.standard_normal(d)
    k = RNG.standard_normal(d)
    v = RNG.standard_normal(e)
    dO = RNG.standard_normal(e)
    S0 = np.abs(RNG.standard_normal((d, e)))
    z0 = np.abs(RNG.standard_normal(d)) + 0.5
    gv = 0.3
    pq, pk = orc.feature_map(q, "elu1"), orc.feature_map(k, "elu1")
    a = (1.0 / (1.0 + np.exp(-gv))) ** (1.0 / tau)
    num = a * (pq @ S0) + (pq @ pk) * v
    den = a * (pq @ z0) + pq @ pk + eps
    dL_da = float(dO @ ((pq @ S0) * den - num * (pq @ z0)) / den ** 2)
    want = dL_da * a * (1.0 / (1.0 + np.exp(gv))) / tau
    sh = lambda x: x.reshape((1, 1) + x.shape)
    got = bwd.backward_sel(sh(q[None]), sh(k[None]), sh(v[None]), sh(dO[None]), np.array([[[gv]]]), tau, "elu1",
                           None, eps, sh(S0), sh(z0))[3]
    assert abs(float(got[0, 0, 0]) - want) <= 1e-12 * max(1.0, abs(want))


@pytest.mark.parametrize("fmap", ["elu1", "identity"])
def test_gla_sampled_rows_equal_the_explicit_form(fmap):
    """backward_gla_rows (per-row sums, O(n r) memory, for full-length
    sequences) equals backward_gla (the explicit [n, n, r] form) at every row
    and every tail step."""
    n, d, e, tau = 23, 4, 3, 5.0
    Q = RNG.standard_normal((n, d)) * 0.7
    K = RNG.standard_normal((n, d)) * 0.7
    V = RNG.standard_normal((n, e))
    G = RNG.standard_normal((n, d))
    dO = RNG.standard_normal((n, e))
    sh = lambda x: x[None, None]
    want = bwd.backward_gla(sh(Q), sh(K), sh(V), sh(dO), sh(G), tau, fmap, None, 1e-3)
    rows = [0, 1, 7, n - 1]
    got = bwd.backward_gla_rows(Q, K, V, dO, G, tau, fmap, 1e-3, rows=rows, tail=n)
    for a, b in zip(got[:3], want[:3]):
        np.testing.assert_allclose(a, b[0, 0][rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got[3], want[3][0, 0], rtol=1e-10, atol=1e-12)


def test_sel_sampled_rows_equal_the_explicit_form():
    n, d, e, tau = 19, 4, 3, 3.0
    Q = RNG.standard_normal((n, d)) * 0.7
    K = RNG.standard_normal((n, d)) * 0.7
    V = RNG.standard_normal((n, e))
    G = RNG.standard_normal(n)
    dO = RNG.standard_normal((n, e))
    sh = lambda x: x[None, None]
    want = bwd.backward_sel(sh(Q), sh(K), sh(V), sh(dO), sh(G), tau, "elu1", None, 1e-3)
    rows = [0, 5, n - 1]
    got = bwd.backward_sel_rows(Q, K, V, dO, G, tau, "elu1", 1e-3, rows=rows, tail=n)
    for a, b in zip(got[:3], want[:3]):
        np.testing.assert_allclose(a, b[0, 0][rows], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got[3], want[3][0, 0], rtol=1e-10, atol=1e-12)
