"""Plain fp64 CPU oracle for the gradients of kernelized linear attention.

TEST INFRASTRUCTURE ONLY, like ``la_oracle``: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may use it; it shares no code with
the HIP library.

Training uses the parallel form of the layer and inference the recurrent one
(the dileepadev page, "Recurrent Reformulation"; the train/infer duality of
the blog.vguerra.net page, "The recurrent form (causal)"). This module gives
the gradients of the forward pass: for a loss L with dL/do_i = dO_i (the
vector-Jacobian product the backward pass of a training step needs), it
returns dL/dQ, dL/dK, dL/dV. It differentiates the explicit weight-matrix form
of ``la_oracle`` (W_ij = phi(q_i).phi(k_j) D_ij, o_i = sum_j W_ij v_j /
(sum_j W_ij + eps), plus the read-out of a carried-in state S0, z0) by the
chain rule written out step by step below; nothing is blocked or reordered.

Gates covered: none and the RetNet decay (gamma is a fixed per-head constant,
so it has no gradient). The diagonal GLA gate is not covered here.
Pinned by ``tests/test_oracle_backward_pins.py`` against central finite differences of
the pinned forward oracle and against closed forms.
"""
from __future__ import annotations

import numpy as np

from .la_oracle import feature_map

__all__ = ["feature_map_vjp", "forward_terms", "backward"]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def feature_map_vjp(x, dphi, fmap="elu1", omega=None):
    """dL/dx from dL/dphi(x) for the named feature map (last axis).

    elu+1: phi'(x) = 1 for x > 0 and exp(x) for x <= 0 (the derivative of
    elu(x) + 1 with slope parameter 1; both sides give 1 at x = 0).
    FAVOR+: phi_m = exp(w_m.x - |x|^2/2) / sqrt(r) has d phi_m / dx =
    phi_m (w_m - x), so dL/dx = sum_m dphi_m phi_m (w_m - x).
    """
    x = _f64(x)
    dphi = _f64(dphi)
    if fmap == "elu1":
        return dphi * np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    if fmap == "favor":
        om = _f64(omega)
        phi = feature_map(x, "favor", om)
        a = dphi * phi                                     # [..., r]
        return np.einsum("...m,md->...d", a, om) - x * a.sum(axis=-1, keepdims=True)
    raise ValueError(f"unknown feature map {fmap!r}")


def _decay_matrix(n, H, causal, gate):
    """D[h, i, j]: 1 (non-causal), [j <= i] (causal), [j <= i] gamma_h^(i-j) (RetNet)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    mask = (j <= i) if causal else np.ones((n, n), dtype=bool)
    kind = "none" if gate is None else gate[0]
    if kind == "none":
        return np.broadcast_to(mask.astype(np.float64), (H, n, n))
    if kind == "decay":
        if not causal:
            raise ValueError("gates are defined for the causal form only")
        gam = _f64(gate[1]).reshape(H, 1, 1)
        expo = np.where(mask, i - j, 0)
        return np.where(mask[None], gam ** expo[None], 0.0)
    raise NotImplementedError("gradients of the GLA gate are not covered")


def _state_decay(n, H, gate):
    """c[h, i]: weight of a carried-in state at step i (gamma^(i+1) for RetNet, else 1)."""
    kind = "none" if gate is None else gate[0]
    t = np.arange(n)[None, :]
    if kind == "decay":
        return _f64(gate[1]).reshape(H, 1) ** (t + 1)
    return np.ones((H, n))


def forward_terms(Q, K, V, fmap="elu1", omega=None, causal=True, gate=None, eps=1e-6, S0=None, z0=None):
    """Forward quantities of the weight-matrix form: (phi_q, phi_k, D, c, W, num, den, o).

    W_ij = (phi(q_i).phi(k_j)) D_ij; num_i = sum_j W_ij v_j + c_i phi(q_i)^T S0;
    den_i = sum_j W_ij + c_i phi(q_i).z0 + eps; o_i = num_i / den_i
    ("The Kernel Trick for Attention" and "Recurrent Reformulation" on the
    dileepadev page, the eps of the sadullah page's routine; the carried-in
    state is the recurrence's S_{-1}, decayed like every earlier key).
    """
    V = _f64(V)
    pq = feature_map(Q, fmap, omega)
    pk = feature_map(K, fmap, omega)
    B, H, n, r = pq.shape
    D = _decay_matrix(n, H, causal, gate)                  # [H, n, n]
    c = _state_decay(n, H, gate)                           # [H, n]
    W = np.einsum("bhir,bhjr->bhij", pq, pk) * D[None]
    num = np.einsum("bhij,bhje->bhie", W, V)
    den = W.sum(axis=-1) + eps
    if S0 is not None:
        S0 = _f64(S0)
        z0 = _f64(z0)
        num = num + c[None, :, :, None] * np.einsum("bhir,bhre->bhie", pq, S0)
        den = den + c[None] * np.einsum("bhir,bhr->bhi", pq, z0)
    o = num / den[..., None]
    return pq, pk, D, c, W, num, den, o


def backward(Q, K, V, dO, fmap="elu1", omega=None, causal=True, gate=None, eps=1e-6, S0=None, z0=None):
    """(dQ, dK, dV) of L = sum_i dO_i . o_i, all [B, H, n, d] float64.

    Chain rule through the forward of ``forward_terms``:
      o_i = num_i / den_i            => dnum_i = dO_i / den_i = g_i,
                                        dden_i = -(dO_i . o_i) / den_i = h_i
      num_i, den_i linear in W_ij    => dW_ij = g_i . v_j + h_i,  dV_j = sum_i W_ij g_i
      W_ij = (phi_q_i . phi_k_j) D_ij => dM_ij = dW_ij D_ij,
                                        dphi_q_i = sum_j dM_ij phi_k_j + c_i (S0 g_i + h_i z0),
                                        dphi_k_j = sum_i dM_ij phi_q_i
      phi = feature map               => dQ, dK by ``feature_map_vjp``.
    """
    V = _f64(V)
    dO = _f64(dO)
    pq, pk, D, c, W, num, den, o = forward_terms(Q, K, V, fmap, omega, causal, gate, eps, S0, z0)
    g = dO / den[..., None]
    h = -np.sum(dO * o, axis=-1) / den
    dW = np.einsum("bhie,bhje->bhij", g, V) + h[..., None]
    dV = np.einsum("bhij,bhie->bhje", W, g)
    dM = dW * D[None]
    dpq = np.einsum("bhij,bhjr->bhir", dM, pk)
    dpk = np.einsum("bhij,bhir->bhjr", dM, pq)
    if S0 is not None:
        S0 = _f64(S0)
        z0 = _f64(z0)
        dpq = dpq + c[None, :, :, None] * (np.einsum("bhre,bhie->bhir", S0, g) + h[..., None] * z0[:, :, None, :])
    dQ = feature_map_vjp(Q, dpq, fmap, omega)
    dK = feature_map_vjp(K, dpk, fmap, omega)
    return dQ, dK, dV
