"""A CPU model of where the GLA backward's dq pass rounds to bf16, checked
against the fp64 gradient oracle (oracle.la_backward.backward_gla).

The chunked dq pass ("Gating and Selective State Updates", dileepadev page:
alpha_t = sigmoid(g_t)^(1/tau) per feature) works in 64-token chunks on the
gated tiles Q~ = phi(q) e^{b}, K~ = phi(k) e^{-b} (b the chunk's cumulative
log-gate), the state S and normaliser z entering the chunk, g = dO / den and
h = -g . o:
    dq_i = (sum_{j<=i} dW_ij K~_j + S g_i + z h_i) e^{b_i} phi'(q_i),
    dW_ij = g_i . v_j + h_i.
The model runs exactly that in fp64 and rounds chosen operands to bf16 where
the kernel stores them as bf16. With no rounding it reproduces the oracle; with
the operands the kernel keeps single bf16 (Q~, K~ in the scores, the state in o,
g, e^{b} phi'(q)) the error over the head's largest dq entry stays under 1e-2.
The two roundings the kernel avoids by hi + lo pairs, the state's image in dq's
own state product and the gated keys in the state update, are the two largest
single terms, and together they would at least double the error. Model only: it
shares nothing with the HIP path.
"""
import numpy as np
import pytest
import torch

from oracle import la_backward as obwd
from oracle.la_oracle import feature_map


def _bf(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def _dq_model(Q, K, V, dO, g, tau, eps, rounded):
    """dq of one head through the chunked pass, with the operands named in
    ``rounded`` taken as bf16: 'Q', 'K' (the gated tiles in the scores and o),
    'Ku' (the gated keys in the state update), 'S' (the state in o), 'Sd' (the
    state in dq's state product), 'g', 'qd' (e^{b} phi'(q))."""
    n, d = Q.shape
    pq, pk = feature_map(Q, "elu1"), feature_map(K, "elu1")
    dphi = np.where(Q > 0, 1.0, np.exp(np.minimum(Q, 0.0)))
    logalpha = -np.logaddexp(0.0, -g) / tau
    r = lambda name, x: _bf(x) if name in rounded else x
    dq = np.zeros((n, d))
    S = np.zeros((d, V.shape[1]))
    z = np.zeros(d)
    for c0 in range(0, n, 64):
        c1 = min(n, c0 + 64)
        b = np.cumsum(logalpha[c0:c1], axis=0)
        Qt, Kt = pq[c0:c1] * np.exp(b), pk[c0:c1] * np.exp(-b)
        v, do = V[c0:c1], dO[c0:c1]
        A = np.tril(r("Q", Qt) @ r("K", Kt).T)
        den = A.sum(1) + r("Q", Qt) @ z + eps
        o = (r("Q", Qt) @ r("S", S) + A @ v) / den[:, None]
        gg = r("g", do / den[:, None])
        h = -np.sum(gg * o, axis=1)
        dW = np.tril(gg @ v.T + h[:, None])
        dq[c0:c1] = (dW @ Kt + gg @ r("Sd", S).T + np.outer(h, z)) * r("qd", np.exp(b) * dphi[c0:c1])
        S = np.exp(b[-1])[:, None] * (S + r("Ku", Kt).T @ v)
        z = np.exp(b[-1]) * (z + r("Ku", Kt).sum(0))
    return dq


@pytest.fixture(scope="module")
def head():
    rng = np.random.default_rng(0)
    n, d, tau = 777, 64, 16.0
    draw = lambda s: _bf(rng.standard_normal((n, d)) * s)
    Q, K, V, dO, g = draw(d ** -0.5), draw(d ** -0.5), draw(d ** -0.5), draw(1.0), draw(1.0)
    ref = obwd.backward_gla(Q[None, None], K[None, None], V[None, None], dO[None, None], g[None, None], tau)[0][0, 0]
    return Q, K, V, dO, g, tau, ref


def _err(head, rounded):
    Q, K, V, dO, g, tau, ref = head
    return float(np.max(np.abs(_dq_model(Q, K, V, dO, g, tau, 1e-6, rounded) - ref)) / np.max(np.abs(ref)))


def test_model_without_rounding_is_the_oracle(head):
    assert _err(head, set()) < 1e-11


KEPT = {"Q", "K", "S", "g", "qd"}  # single bf16 in the kernel
SPLIT = {"Sd", "Ku"}  # hi + lo pairs in the kernel


def test_kernel_roundings_stay_within_the_bound(head):
    assert _err(head, KEPT) < 1e-2


def test_split_operands_are_the_largest_terms(head):
    assert _err(head, KEPT | SPLIT) > 2.0 * _err(head, KEPT)
    for split in SPLIT:
        for name in KEPT:
            assert _err(head, {split}) > _err(head, {name}), (split, name)
