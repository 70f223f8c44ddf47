"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names the passage of the pages (or the mathematical fact) it checks,
and is chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign or index, an off-by-one mask, a transposed operand, a gate applied at the
wrong time, an ungated normaliser) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch

import oracle as orc

RNG = np.random.default_rng(1234)


def _rand(*shape, scale=1.0, rng=RNG):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- feature maps

def test_elu1_closed_form_points():
    # elu(x)+1 at hand-computed points: x+1 above zero, exp(x) at and below
    x = np.array([2.5, 1.0, 1e-3, 0.0, -1.0, -30.0])
    want = np.array([3.5, 2.0, 1.001, 1.0, math.exp(-1.0), math.exp(-30.0)])
    np.testing.assert_allclose(orc.phi_elu1(x), want, rtol=1e-15, atol=0)


def test_elu1_matches_library_elu():
    x = _rand(1000, scale=3.0)
    lib = torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0).numpy() + 1.0
    np.testing.assert_allclose(orc.phi_elu1(x), lib, rtol=1e-14, atol=1e-15)
    assert np.all(orc.phi_elu1(x) > 0)


def test_favor_unbiased_for_exp_kernel():
    """E[phi(q).phi(k)] = exp(q.k) for w ~ N(0, I): the FAVOR+ property
    ("Choosing the Feature Map phi"). A flipped sign of |x|^2/2, a missing
    1/sqrt(r) or a transposed omega all move the mean by many sigmas."""
    rng = np.random.default_rng(7)
    d, r, draws = 4, 64, 4000
    q = np.array([0.3, -0.2, 0.4, 0.1])
    k = np.array([-0.1, 0.5, 0.2, -0.3])
    est = np.empty(draws)
    for t in range(draws):
        om = rng.standard_normal((r, d))
        est[t] = orc.phi_favor(q, om) @ orc.phi_favor(k, om)
    mean, sem = est.mean(), est.std(ddof=1) / math.sqrt(draws)
    assert abs(mean - math.exp(q @ k)) < 6 * sem
    assert sem < 0.01 * math.exp(q @ k)


def test_favor_features_positive():
    om = _rand(256, 64)
    x = _rand(10, 64, scale=64 ** -0.25)
    assert np.all(orc.phi_favor(x, om) > 0)


@pytest.mark.parametrize("causal", [False, True])
def test_favor_converges_to_softmax_attention(causal):
    """With many random features the FAVOR+ output approaches softmax attention
    with weights exp(q.k) (library SDPA with scale 1)."""
    rng = np.random.default_rng(11)
    n, d, r = 6, 4, 1 << 16
    Q = rng.standard_normal((1, 1, n, d)) * 0.5
    K = rng.standard_normal((1, 1, n, d)) * 0.5
    V = rng.standard_normal((1, 1, n, 3))
    om = rng.standard_normal((r, d))
    if causal:
        o = orc.causal_recurrent(Q, K, V, "favor", om, None, eps=0.0)[0]
    else:
        o = orc.noncausal(Q, K, V, "favor", om, eps=0.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V),
        is_causal=causal, scale=1.0).numpy()
    assert orc.rowwise_rel_err(o, ref) < 3e-2


# ---------------------------------------------------------------- non-causal

def _nc_inputs(n=256, d=32, dv=32, seed=0, scale=None):
    rng = np.random.default_rng(seed)
    s = d ** -0.5 if scale is None else scale
    return (rng.standard_normal((1, 1, n, d)) * s, rng.standard_normal((1, 1, n, d)) * s,
            rng.standard_normal((1, 1, n, dv)) * s)


def test_noncausal_reassociation_equals_explicit_matrix():
    """(phiQ phiK^T) V == phiQ (phiK^T V): the reassociation identity, at the
    non-causal workload's full size (explicit 256 x 256 weight matrix)."""
    Q, K, V = _nc_inputs()
    a = orc.noncausal(Q, K, V, eps=1e-6)
    b = orc.brute(Q, K, V, causal=False, eps=1e-6)
    assert orc.rowwise_rel_err(a, b) < 1e-12


def test_noncausal_rectangular_favor_reassociation():
    # r != d_k != d_v: a transposed operand anywhere breaks the shapes or values
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((2, 3, 9, 5)) * 0.4
    K = rng.standard_normal((2, 3, 9, 5)) * 0.4
    V = rng.standard_normal((2, 3, 9, 7))
    om = rng.standard_normal((16, 5))
    a = orc.noncausal(Q, K, V, "favor", om, eps=1e-6)
    b = orc.brute(Q, K, V, "favor", om, causal=False, eps=1e-6)
    assert a.shape == (2, 3, 9, 7)
    assert orc.rowwise_rel_err(a, b) < 1e-12


def test_noncausal_permutation_invariant():
    Q, K, V = _nc_inputs(n=64, scale=1.0)
    p = np.random.default_rng(5).permutation(64)
    a = orc.noncausal(Q, K, V)
    b = orc.noncausal(Q, K[:, :, p], V[:, :, p])
    assert orc.rowwise_rel_err(a, b) < 1e-13


def test_uniform_weights_give_plain_mean():
    """Q = K = 0 makes every elu+1 feature exactly 1: non-causal output is the
    mean of V, causal output is the running (prefix) mean."""
    rng = np.random.default_rng(9)
    n, d = 50, 8
    Z = np.zeros((1, 1, n, d))
    V = rng.standard_normal((1, 1, n, 3))
    nc = orc.noncausal(Z, Z, V, eps=0.0)
    np.testing.assert_allclose(nc, np.broadcast_to(V.mean(axis=2, keepdims=True), nc.shape), rtol=1e-13)
    c = orc.causal_recurrent(Z, Z, V, eps=0.0)[0]
    prefix = np.cumsum(V, axis=2) / np.arange(1, n + 1)[None, None, :, None]
    np.testing.assert_allclose(c, prefix, rtol=1e-12, atol=1e-15)


def test_constant_values_and_eps():
    # V == c everywhere: o = c * den / (den + eps), den = phi(q).sum(phi(k))
    Q, K, _ = _nc_inputs(n=40, scale=1.0)
    V = np.full((1, 1, 40, 4), 2.5)
    eps = 1e-2
    pq, pk = orc.phi_elu1(Q), orc.phi_elu1(K)
    den = np.einsum("bhir,bhjr->bhi", pq, pk)
    want = 2.5 * den / (den + eps)
    np.testing.assert_allclose(orc.noncausal(Q, K, V, eps=eps), np.broadcast_to(want[..., None], (1, 1, 40, 4)), rtol=1e-13)


# ---------------------------------------------------------------- causal forms

CASES = [("elu1", "none"), ("elu1", "decay"), ("elu1", "gla"), ("elu1", "sel"),
         ("favor", "none"), ("favor", "decay"), ("favor", "gla"),
         ("identity", "none"), ("identity", "decay"), ("identity", "gla"), ("identity", "sel")]


def _causal_case(fmap, gate, B=2, H=3, n=23, d=6, dv=5, r=12, seed=0):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, n, d)) * 0.7
    K = rng.standard_normal((B, H, n, d)) * 0.7
    V = rng.standard_normal((B, H, n, dv))
    om = rng.standard_normal((r, d)) if fmap == "favor" else None
    rr = r if fmap == "favor" else d
    if gate == "none":
        gt = None
    elif gate == "decay":
        gt = ("decay", 1.0 - 2.0 ** (-1.0 - np.arange(H)))
    elif gate == "sel":
        gt = ("sel", rng.standard_normal((B, H, n)) * 2.0, 4.0)
    else:
        gt = ("gla", rng.standard_normal((B, H, n, rr)) * 2.0, 4.0)
    return Q, K, V, om, gt


@pytest.mark.parametrize("fmap,gate", CASES)
def test_parallel_equals_recurrent(fmap, gate):
    """The parallel (masked weight matrix) and recurrent forms agree: the
    duality of "Recurrent Reformulation" / "The recurrent form (causal)"."""
    Q, K, V, om, gt = _causal_case(fmap, gate)
    a = orc.brute(Q, K, V, fmap, om, causal=True, gate=gt, eps=1e-6)
    b = orc.causal_recurrent(Q, K, V, fmap, om, gt, eps=1e-6)[0]
    assert orc.rowwise_rel_err(b, a) < 1e-12


@pytest.mark.parametrize("fmap,gate", CASES)
def test_split_sequence_resumes(fmap, gate):
    """Carrying (S, z) out of a prefix and into the rest equals one pass."""
    Q, K, V, om, gt = _causal_case(fmap, gate, n=30)
    full, Sf, zf = orc.causal_recurrent(Q, K, V, fmap, om, gt)
    m = 11

    def cut(gg, sl):
        if gg is None or gg[0] not in ("gla", "sel"):
            return gg
        return (gg[0], gg[1][:, :, sl], gg[2])
    a, S1, z1 = orc.causal_recurrent(Q[:, :, :m], K[:, :, :m], V[:, :, :m], fmap, om, cut(gt, slice(0, m)))
    b, S2, z2 = orc.causal_recurrent(Q[:, :, m:], K[:, :, m:], V[:, :, m:], fmap, om, cut(gt, slice(m, None)),
                                     S0=S1, z0=z1)
    assert orc.rowwise_rel_err(np.concatenate([a, b], axis=2), full) < 1e-12
    np.testing.assert_allclose(S2, Sf, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, zf, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmap,gate", CASES)
def test_decode_step_is_one_recurrence_step(fmap, gate):
    Q, K, V, om, gt = _causal_case(fmap, gate, n=8)
    full, _, _ = orc.causal_recurrent(Q, K, V, fmap, om, gt)
    pre = gt
    if gt is not None and gt[0] in ("gla", "sel"):
        pre = (gt[0], gt[1][:, :, :7], gt[2])
    _, S7, z7 = orc.causal_recurrent(Q[:, :, :7], K[:, :, :7], V[:, :, :7], fmap, om, pre)
    step_gate = gt if gt is None or gt[0] not in ("gla", "sel") else (gt[0], gt[1][:, :, 7], gt[2])
    o, _, _ = orc.decode_step(S7, z7, Q[:, :, 7], K[:, :, 7], V[:, :, 7], fmap, om, step_gate)
    np.testing.assert_allclose(o, full[:, :, 7], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("gate", ["none", "decay", "gla"])
def test_first_token_state_is_outer_product(gate):
    """From a zero state, one token leaves S = phi(k) v^T and z = phi(k) under
    any gate (the gate multiplies the previous state, not the new token), and
    o_0 = v_0 * w / (w + eps) with w = phi(q).phi(k)."""
    Q, K, V, om, gt = _causal_case("elu1", gate, n=1)
    eps = 0.3
    o, S, z = orc.causal_recurrent(Q, K, V, "elu1", None, gt, eps=eps)
    pk, pq = orc.phi_elu1(K[:, :, 0]), orc.phi_elu1(Q[:, :, 0])
    np.testing.assert_allclose(S, pk[..., :, None] * V[:, :, 0, None, :], rtol=1e-15)
    np.testing.assert_allclose(z, pk, rtol=1e-15)
    w = np.sum(pq * pk, axis=-1)
    np.testing.assert_allclose(o[:, :, 0], V[:, :, 0] * (w / (w + eps))[..., None], rtol=1e-14)


def test_decay_geometric_closed_form():
    """RetNet weights gamma^(i-j) ("Gating and Selective State Updates"): with
    all features 1 and a single unit value at t = 0, the output is
    gamma^i (1 - gamma) / (1 - gamma^(i+1)). An undecayed normaliser or a
    wrong exponent fails this."""
    n, H = 40, 3
    gam = np.array([0.5, 0.9, 1.0 - 2.0 ** -12])
    Z = np.zeros((1, H, n, 4))
    V = np.zeros((1, H, n, 1))
    V[:, :, 0, 0] = 1.0
    o = orc.causal_recurrent(Z, Z, V, gate=("decay", gam), eps=0.0)[0][0, :, :, 0]
    i = np.arange(n)[None, :]
    g = gam[:, None]
    want = g ** i * (1 - g) / (1 - g ** (i + 1))
    np.testing.assert_allclose(o, want, rtol=1e-10)


def test_decay_matches_iir_filter():
    """With all features 1, numerator and denominator are first-order IIR
    filters y_i = gamma y_{i-1} + x_i (scipy.signal.lfilter)."""
    rng = np.random.default_rng(21)
    n, gam = 64, 0.8
    Z = np.zeros((1, 1, n, 4))
    V = rng.standard_normal((1, 1, n, 2))
    o = orc.causal_recurrent(Z, Z, V, gate=("decay", np.array([gam])), eps=0.0)[0][0, 0]
    num = scipy.signal.lfilter([1.0], [1.0, -gam], V[0, 0] * 4.0, axis=0)
    den = scipy.signal.lfilter([1.0], [1.0, -gam], np.full(n, 4.0))
    np.testing.assert_allclose(o, num / den[:, None], rtol=1e-12)


@pytest.mark.parametrize("fmap", ["elu1", "favor"])
def test_unit_gates_reduce_to_ungated(fmap):
    """gamma = 1 and alpha = 1 (g -> +inf) give plain causal linear attention
    ("When G_t = 1 everywhere, the model behaves like standard linear
    attention")."""
    Q, K, V, om, _ = _causal_case(fmap, "none")
    base = orc.causal_recurrent(Q, K, V, fmap, om, None)[0]
    d1 = orc.causal_recurrent(Q, K, V, fmap, om, ("decay", np.ones(3)))[0]
    rr = om.shape[0] if om is not None else Q.shape[-1]
    g1 = orc.causal_recurrent(Q, K, V, fmap, om, ("gla", np.full(Q.shape[:3] + (rr,), 1e4), 16.0))[0]
    assert orc.rowwise_rel_err(d1, base) == 0.0
    assert orc.rowwise_rel_err(g1, base) == 0.0


def test_zero_gate_overwrites_state():
    """alpha = 0 (g -> -inf) fully overwrites the state ("When G_t = 0, the
    state is fully overwritten"): o_t = v_t * w_t / (w_t + eps)."""
    Q, K, V, _, _ = _causal_case("elu1", "none")
    eps = 0.05
    o = orc.causal_recurrent(Q, K, V, gate=("gla", np.full(Q.shape, -1e4), 16.0), eps=eps)[0]
    w = np.sum(orc.phi_elu1(Q) * orc.phi_elu1(K), axis=-1)
    np.testing.assert_allclose(o, V * (w / (w + eps))[..., None], rtol=1e-13)


def test_constant_gla_equals_decay():
    """A GLA gate that is constant over time and features is a fixed decay with
    gamma = sigmoid(g)^(1/tau)."""
    Q, K, V, _, _ = _causal_case("elu1", "none")
    gval, tau = 0.7, 16.0
    gam = scipy.special.expit(gval) ** (1.0 / tau)
    a = orc.causal_recurrent(Q, K, V, gate=("gla", np.full(Q.shape, gval), tau))[0]
    b = orc.causal_recurrent(Q, K, V, gate=("decay", np.full(3, gam)))[0]
    assert orc.rowwise_rel_err(a, b) < 1e-13
    assert abs(orc.gla_alpha(0.0, 16.0) - 2.0 ** (-1.0 / 16.0)) < 1e-15


ATTN_CASES = [c for c in CASES if c[0] != "identity"]   # the normalised (positive-feature) forms


@pytest.mark.parametrize("fmap,gate", ATTN_CASES)
def test_normaliser_positive_and_outputs_convex(fmap, gate):
    """Similarities are non-negative ("must keep similarities >= 0"), so the
    denominator is at least eps and each output coordinate, rescaled by
    (den + eps) / den, lies between the min and max of the values it mixes."""
    Q, K, V, om, gt = _causal_case(fmap, gate, n=20)
    W = orc.kernel_weights(Q, K, fmap, om, True, gt)
    assert np.all(W >= 0)
    eps = 1e-6
    o = orc.attention_from_weights(W, V, eps)
    den = W.sum(-1)
    assert np.all(den + eps >= eps)
    scaled = o * ((den + eps) / den)[..., None]
    for i in range(Q.shape[2]):
        lo = V[:, :, :i + 1].min(axis=2)
        hi = V[:, :, :i + 1].max(axis=2)
        assert np.all(scaled[:, :, i] >= lo - 1e-12) and np.all(scaled[:, :, i] <= hi + 1e-12)


@pytest.mark.parametrize("gate", ["none", "decay", "gla"])
def test_exact_zero_probe_causal_mask(gate):
    """A single unit value at position p: every output before p is exactly
    zero (no future leak), and o_p is positive in the marked column."""
    Q, K, _, _, gt = _causal_case("elu1", gate, n=30)
    V = np.zeros(Q.shape[:3] + (5,))
    p, col = 17, 2
    V[:, :, p, col] = 1.0
    o = orc.causal_recurrent(Q, K, V, gate=gt)[0]
    assert np.all(o[:, :, :p] == 0.0)
    assert np.all(o[:, :, p, col] > 0)
    others = np.delete(o, col, axis=-1)
    assert np.all(others == 0.0)


# ---------------------------------------------------------------- the one printed figure

def test_quadratic_baseline_figure(repo_root):
    """Golden: the page's size of one n = 16384 float16 score matrix."""
    vals = {}
    with open(os.path.join(repo_root, "tests", "golden", "quadratic_baseline.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = (s.strip() for s in line.split("="))
                vals[k] = float(v)
    n = int(vals["n"])
    assert abs(orc.softmax_score_matrix_bytes(n, 1) - vals["entries_approx"]) / vals["entries_approx"] < 0.005
    assert abs(orc.softmax_score_matrix_bytes(n, 2) - vals["bytes_fp16_approx"]) / vals["bytes_fp16_approx"] < 0.005
    assert orc.softmax_score_matrix_bytes(n, 2) == 536_870_912


# ---------------------------------------------------------------- metric

def test_rowwise_metric():
    ref = np.array([[1.0, -2.0, 0.5], [0.0, 0.0, 0.0], [3.0, 0.0, 0.0]])
    got = ref.copy()
    assert orc.rowwise_rel_err(got, ref) == 0.0
    got[0, 2] += 0.02  # 0.02 / 2.0
    assert abs(orc.rowwise_rel_err(got, ref) - 0.01) < 1e-15
    got[1, 0] = 1e-9  # a nonzero where the reference row is all zero
    assert orc.rowwise_rel_err(got, ref) == math.inf
    got[1, 0] = np.nan
    assert orc.rowwise_rel_err(got, ref) == math.inf


# ------------------------------------------------------- state-space read-out

@pytest.mark.parametrize("gate", ["none", "decay", "gla", "sel"])
def test_identity_is_masked_matrix_product(gate):
    """The state-space form y_t = C_t^T h_t, h_t = A_t h_{t-1} + B_t x_t
    ("State Space Models as Linear Attention") unrolls to y = (M o (C B^T)) X
    with M the causal decay mask. The gate enters through the cumulative
    log-gate c_t = sum_{u<=t} log a_u: the weight of key j at query i is
    exp(c_i - c_j) per feature, so y = tril((C e^c)(B e^-c)^T) X, written here
    with numpy matmuls (no loop over steps, no product of gates)."""
    rng = np.random.default_rng(5)
    B, H, n, d, dv = 2, 3, 29, 5, 4
    C = rng.standard_normal((B, H, n, d))
    Bk = rng.standard_normal((B, H, n, d))
    X = rng.standard_normal((B, H, n, dv))
    if gate == "none":
        logs = np.zeros((B, H, n, d))
        gt = None
    elif gate == "decay":
        gam = np.array([0.5, 0.8, 0.97])
        logs = np.broadcast_to(np.log(gam)[None, :, None, None], (B, H, n, d))
        gt = ("decay", gam)
    elif gate == "sel":
        g = rng.standard_normal((B, H, n)) * 2.0
        tau = 3.0
        logs = np.broadcast_to((np.log(scipy.special.expit(g)) / tau)[..., None], (B, H, n, d))
        gt = ("sel", g, tau)
    else:
        g = rng.standard_normal((B, H, n, d)) * 2.0
        tau = 3.0
        logs = np.log(scipy.special.expit(g)) / tau
        gt = ("gla", g, tau)
    c = np.cumsum(logs, axis=2)
    W = np.tril((C * np.exp(c)) @ np.swapaxes(Bk * np.exp(-c), -1, -2))
    want = W @ X
    got = orc.causal_recurrent(C, Bk, X, "identity", None, gt)[0]
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)


def test_identity_decay_matches_iir_filter():
    """One state feature with C = B = 1: y_t = gamma y_{t-1} + x_t, a
    first-order IIR filter (scipy.signal.lfilter), with no normaliser."""
    rng = np.random.default_rng(22)
    n, gam = 50, 0.85
    one = np.ones((1, 1, n, 1))
    X = rng.standard_normal((1, 1, n, 3))
    y = orc.causal_recurrent(one, one, X, "identity", None, ("decay", np.array([gam])))[0][0, 0]
    np.testing.assert_allclose(y, scipy.signal.lfilter([1.0], [1.0, -gam], X[0, 0], axis=0), rtol=1e-12)


def test_identity_is_linear_in_values():
    """The unnormalised read-out is linear in the values (a normaliser or a
    feature map applied to the inputs would break it: y(2x + x') = 2 y(x) + y(x'))."""
    Q, K, V, om, gt = _causal_case("identity", "gla", seed=3)
    V2 = np.random.default_rng(4).standard_normal(V.shape)
    a = orc.causal_recurrent(Q, K, 2.0 * V + V2, "identity", None, gt)[0]
    b = 2.0 * orc.causal_recurrent(Q, K, V, "identity", None, gt)[0] + orc.causal_recurrent(Q, K, V2, "identity",
                                                                                               None, gt)[0]
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    # and also linear (odd) in the queries, which a positive feature map is not
    c = orc.causal_recurrent(-Q, K, V, "identity", None, gt)[0]
    np.testing.assert_allclose(c, -orc.causal_recurrent(Q, K, V, "identity", None, gt)[0], rtol=1e-12)


# ------------------------------------------------------- scalar selective gate

def test_constant_selective_gate_equals_decay():
    """A selective gate whose input is constant in time is a fixed decay:
    a = sigmoid(g)^(1/tau) per head reproduces the RetNet form."""
    rng = np.random.default_rng(31)
    B, H, n = 2, 3, 19
    Q, K, V = rng.standard_normal((B, H, n, 5)), rng.standard_normal((B, H, n, 5)), rng.standard_normal((B, H, n, 4))
    gh = np.array([-1.0, 0.5, 3.0])
    tau = 2.0
    g = np.broadcast_to(gh[None, :, None], (B, H, n)).copy()
    gam = scipy.special.expit(gh) ** (1.0 / tau)
    for fmap in ("elu1", "identity"):
        a = orc.causal_recurrent(Q, K, V, fmap, None, ("sel", g, tau))[0]
        b = orc.causal_recurrent(Q, K, V, fmap, None, ("decay", gam))[0]
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_selective_gate_is_gla_shared_by_features():
    """The scalar selective gate is the diagonal GLA gate with the same input
    on every feature (A_t = a_t I)."""
    rng = np.random.default_rng(32)
    B, H, n, d = 2, 2, 17, 6
    Q, K, V = rng.standard_normal((B, H, n, d)), rng.standard_normal((B, H, n, d)), rng.standard_normal((B, H, n, 3))
    g = rng.standard_normal((B, H, n)) * 2.0
    a = orc.causal_recurrent(Q, K, V, "elu1", None, ("sel", g, 3.0))[0]
    b = orc.causal_recurrent(Q, K, V, "elu1", None, ("gla", np.repeat(g[..., None], d, axis=-1), 3.0))[0]
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------- outer-product gate

def _outer_inputs(rng, B=2, H=2, n=13, d=4, dv=3):
    Q, K = rng.standard_normal((B, H, n, d)), rng.standard_normal((B, H, n, d))
    V = rng.standard_normal((B, H, n, dv))
    g, gv = rng.standard_normal((B, H, n, d)) * 2.0, rng.standard_normal((B, H, n, dv)) * 2.0
    return Q, K, V, g, gv


def test_outer_gate_with_unit_value_side_is_gla():
    """beta = 1 (gv -> +inf) leaves the diagonal GLA gate: outputs and states."""
    rng = np.random.default_rng(41)
    Q, K, V, g, gv = _outer_inputs(rng)
    gv = np.full_like(gv, np.inf)
    for fmap in ("elu1", "identity"):
        a = orc.causal_recurrent(Q, K, V, fmap, None, ("outer", g, gv, 3.0))
        b = orc.causal_recurrent(Q, K, V, fmap, None, ("gla", g, 3.0))
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(orc.brute(Q, K, V, fmap, None, True, ("outer", g, gv, 3.0)), b[0],
                                   rtol=1e-10, atol=1e-12)


def test_outer_gate_explicit_equals_recurrent():
    """The explicit per-entry products of alpha and beta equal the step-by-step
    recurrence, for both elementwise feature maps."""
    rng = np.random.default_rng(42)
    Q, K, V, g, gv = _outer_inputs(rng)
    for fmap in ("elu1", "identity"):
        gate = ("outer", g, gv, 2.0)
        a = orc.causal_recurrent(Q, K, V, fmap, None, gate)[0]
        b = orc.brute(Q, K, V, fmap, None, True, gate)
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_outer_gate_value_side_is_an_iir_filter_per_column():
    """One key feature with alpha = 1 and a value-side gate constant in time:
    column e of the state is h_t = beta_e h_{t-1} + k_t v_te, a first-order IIR
    filter (scipy.signal.lfilter), and y_t = q_t h_t."""
    rng = np.random.default_rng(43)
    n, dv, tau = 40, 3, 2.0
    q, k, V = rng.standard_normal(n), rng.standard_normal(n), rng.standard_normal((n, dv))
    gvc = np.array([-2.0, 0.3, 4.0])
    beta = scipy.special.expit(gvc) ** (1.0 / tau)
    sh = lambda x: x.reshape((1, 1) + x.shape)
    gate = ("outer", sh(np.full((n, 1), np.inf)), sh(np.broadcast_to(gvc, (n, dv)).copy()), tau)
    got = orc.causal_recurrent(sh(q[:, None]), sh(k[:, None]), sh(V), "identity", None, gate)[0][0, 0]
    for e in range(dv):
        h = scipy.signal.lfilter([1.0], [1.0, -beta[e]], k * V[:, e])
        np.testing.assert_allclose(got[:, e], q * h, rtol=1e-12, atol=1e-12)


def test_outer_gate_normaliser_takes_the_key_side_only():
    """z evolves as under the GLA gate whatever beta is, and with identical
    value columns of one gate the output columns stay identical."""
    rng = np.random.default_rng(44)
    Q, K, V, g, gv = _outer_inputs(rng)
    a = orc.causal_recurrent(Q, K, V, "elu1", None, ("outer", g, gv, 3.0))
    b = orc.causal_recurrent(Q, K, V, "elu1", None, ("gla", g, 3.0))
    np.testing.assert_allclose(a[2], b[2], rtol=1e-12)
    Vs = np.repeat(V[..., :1], 3, axis=-1)
    gvs = np.repeat(gv[..., :1], 3, axis=-1)
    o = orc.causal_recurrent(Q, K, Vs, "elu1", None, ("outer", g, gvs, 3.0))[0]
    np.testing.assert_allclose(o[..., 1], o[..., 0], rtol=1e-13)
    np.testing.assert_allclose(o[..., 2], o[..., 0], rtol=1e-13)


def test_outer_gate_decode_steps_equal_recurrence():
    rng = np.random.default_rng(45)
    Q, K, V, g, gv = _outer_inputs(rng, n=6)
    o, S, z = orc.causal_recurrent(Q, K, V, "elu1", None, ("outer", g, gv, 3.0))
    S1, z1 = np.zeros_like(S), np.zeros_like(z)
    for t in range(Q.shape[2]):
        ot, S1, z1 = orc.decode_step(S1, z1, Q[:, :, t], K[:, :, t], V[:, :, t], "elu1", None,
                                     ("outer", g[:, :, t], gv[:, :, t], 3.0))
        np.testing.assert_allclose(ot, o[:, :, t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S1, S, rtol=1e-12)


# ------------------------------------------------------- blocked form

@pytest.mark.parametrize("fmap", ["elu1", "favor", "identity"])
@pytest.mark.parametrize("gate", ["none", "decay", "gla", "sel", "outer"])
def test_blocked_form_equals_recurrent_and_explicit(fmap, gate):
    """The blocked form (explicit weights inside a block, the carried state
    across blocks) equals the token recurrence and, without a carried state,
    the explicit n x n form, for block sizes that split the sequence at and
    between chunk-like edges, with a ragged last block."""
    rng = np.random.default_rng(21)
    B, H, n, d, dv = 2, 3, 37, 8, 5
    Q = rng.standard_normal((B, H, n, d)) * 0.5
    K = rng.standard_normal((B, H, n, d)) * 0.5
    V = rng.standard_normal((B, H, n, dv))
    omega = rng.standard_normal((16, d)) if fmap == "favor" else None
    r = 16 if fmap == "favor" else d
    g = {"none": None, "decay": ("decay", np.array([0.9, 0.5, 0.99])),
         "gla": ("gla", rng.standard_normal((B, H, n, r)), 2.0), "sel": ("sel", rng.standard_normal((B, H, n)), 2.0),
         "outer": ("outer", rng.standard_normal((B, H, n, r)), rng.standard_normal((B, H, n, dv)), 2.0)}[gate]
    S0 = rng.standard_normal((B, H, r, dv))
    z0 = np.abs(rng.standard_normal((B, H, r))) + 1.0
    a, Sa, za = orc.causal_recurrent(Q, K, V, fmap, omega, g, 1e-6, S0, z0)
    ex = orc.brute(Q, K, V, fmap, omega, True, g, 1e-6)
    for blk in (1, 4, 7, 36, 64):
        b, Sb, zb = orc.causal_blocked(Q, K, V, fmap, omega, g, 1e-6, S0, z0, block=blk)
        assert orc.rowwise_rel_err(b, a) < 1e-11
        assert np.max(np.abs(Sb - Sa)) / np.max(np.abs(Sa)) < 1e-12
        assert np.max(np.abs(zb - za)) / np.max(np.abs(za)) < 1e-12
        c, _, _ = orc.causal_blocked(Q, K, V, fmap, omega, g, 1e-6, block=blk)
        assert orc.rowwise_rel_err(c, ex) < 1e-11
