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

Gates covered: none, the RetNet decay (gamma is a fixed per-head constant, so
it has no gradient), the diagonal GLA gate, whose raw input g also gets a
gradient (``backward_gla``), the selective scalar gate (``backward_sel``) and
the outer-product gate, with gradients of both raw inputs g and gv
(``backward_outer``).
Pinned by ``tests/test_oracle_backward_pins.py`` against central finite differences of
the pinned forward oracle and against closed forms.
"""
from __future__ import annotations

import numpy as np

from .la_oracle import feature_map, normalised

__all__ = ["feature_map_vjp", "forward_terms", "backward", "backward_gla", "backward_sel", "backward_outer",
           "backward_gla_rows", "backward_sel_rows"]


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def feature_map_vjp(x, dphi, fmap="elu1", omega=None):
    """dL/dx from dL/dphi(x) for the named feature map (last axis).

    elu+1: phi'(x) = 1 for x > 0 and exp(x) for x <= 0 (the derivative of
    elu(x) + 1 with slope parameter 1; both sides give 1 at x = 0).
    identity (the state-space form): phi'(x) = 1.
    FAVOR+: phi_m = exp(w_m.x - |x|^2/2) / sqrt(r) has d phi_m / dx =
    phi_m (w_m - x), so dL/dx = sum_m dphi_m phi_m (w_m - x).
    """
    x = _f64(x)
    dphi = _f64(dphi)
    if fmap == "identity":
        return dphi
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
    if not normalised(fmap):
        den = np.ones_like(den)   # the state-space read-out o = num
    o = num / den[..., None]
    return pq, pk, D, c, W, num, den, o


def backward(Q, K, V, dO, fmap="elu1", omega=None, causal=True, gate=None, eps=1e-6, S0=None, z0=None):
    """(dQ, dK, dV) of L = sum_i dO_i . o_i, all [B, H, n, d] float64.

    Chain rule through the forward of ``forward_terms``:
      o_i = num_i / den_i            => dnum_i = dO_i / den_i = g_i,
                                        dden_i = -(dO_i . o_i) / den_i = h_i
      (the state-space read-out o_i = num_i has g_i = dO_i and h_i = 0)
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
    h = -np.sum(dO * o, axis=-1) / den if normalised(fmap) else np.zeros(den.shape)
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


def backward_gla(Q, K, V, dO, g, tau, fmap="elu1", omega=None, eps=1e-6, S0=None, z0=None):
    """(dQ, dK, dV, dg) of L = sum_i dO_i . o_i for the causal form with the
    diagonal GLA gate, all float64.

    Forward ("Gating and Selective State Updates", dileepadev page): with
    alpha_t = sigmoid(g_t)^(1/tau) per feature and B_t = sum_{u<=t} log alpha_u,
    W_ij = sum_k phi(q_i)_k phi(k_j)_k D_ijk with D_ijk = exp(B_ik - B_jk) =
    prod_{u=j+1}^{i} alpha_uk for j <= i, and the carried-in state enters step i
    with the factor c_ik = exp(B_ik) on row k (the gate of every step up to i).
    Chain rule, as in ``backward`` with the per-feature factors inside the sums:
      dphi_q_ik = sum_j dW_ij phi_k_jk D_ijk + c_ik (S0 g_i + h_i z0)_k
      dphi_k_jk = sum_i dW_ij phi_q_ik D_ijk
      dB_tk     = sum_{i,j} dW_ij phi_q_ik phi_k_jk D_ijk ([t = i] - [t = j])
                  + c_tk phi_q_tk (S0 g_t + h_t z0)_k
                = dphi_q_tk phi_q_tk - dphi_k_tk phi_k_tk
      d log alpha_uk = sum_{t >= u} dB_tk     (B_t sums the log-gates up to t)
      dg_uk = d log alpha_uk * sigmoid(-g_uk) / tau   (log alpha = -softplus(-g) / tau)
    """
    V = _f64(V)
    dO = _f64(dO)
    g = _f64(g)
    pq = feature_map(Q, fmap, omega)
    pk = feature_map(K, fmap, omega)
    B, H, n, r = pq.shape
    with np.errstate(over="ignore"):
        logalpha = -np.logaddexp(0.0, -g) / float(tau)            # log sigmoid(g) / tau
    Bc = np.cumsum(logalpha, axis=2)                             # [B, H, n, r]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    mask = (j <= i)
    # D[b, h, i, j, k] = exp(B_ik - B_jk) on and below the diagonal
    D = np.where(mask[None, None, :, :, None], np.exp(np.minimum(Bc[:, :, :, None, :] - Bc[:, :, None, :, :], 0.0)),
                 0.0)
    W = np.einsum("bhik,bhjk,bhijk->bhij", pq, pk, D)
    num = np.einsum("bhij,bhje->bhie", W, V)
    den = W.sum(axis=-1) + eps
    c = np.exp(Bc)
    if S0 is not None:
        S0 = _f64(S0)
        z0 = _f64(z0)
        num = num + np.einsum("bhik,bhke->bhie", pq * c, S0)
        den = den + np.einsum("bhik,bhk->bhi", pq * c, z0)
    if not normalised(fmap):
        den = np.ones_like(den)   # the state-space read-out o = num
    o = num / den[..., None]
    gg = dO / den[..., None]
    h = -np.sum(dO * o, axis=-1) / den if normalised(fmap) else np.zeros(den.shape)
    dW = (np.einsum("bhie,bhje->bhij", gg, V) + h[..., None]) * mask[None, None]
    dV = np.einsum("bhij,bhie->bhje", W, gg)
    dpq = np.einsum("bhij,bhjk,bhijk->bhik", dW, pk, D)
    dpk = np.einsum("bhij,bhik,bhijk->bhjk", dW, pq, D)
    if S0 is not None:
        dpq = dpq + c * (np.einsum("bhke,bhie->bhik", S0, gg) + h[..., None] * z0[:, :, None, :])
    dB = dpq * pq - dpk * pk
    dlogalpha = np.flip(np.cumsum(np.flip(dB, axis=2), axis=2), axis=2)
    with np.errstate(over="ignore"):
        sig_neg = 1.0 / (1.0 + np.exp(g))                        # sigmoid(-g)
    dg = dlogalpha * sig_neg / float(tau)
    dQ = feature_map_vjp(Q, dpq, fmap, omega)
    dK = feature_map_vjp(K, dpk, fmap, omega)
    return dQ, dK, dV, dg


def backward_sel(Q, K, V, dO, g, tau, fmap="elu1", omega=None, eps=1e-6, S0=None, z0=None):
    """(dQ, dK, dV, dg) for the selective scalar gate: one input-dependent
    decay a_t = sigmoid(g_t)^(1/tau) per step and head, g of shape [B, H, n].

    The recurrence is S_t = a_t S_{t-1} + phi(k_t) v_t^T: the diagonal gate of
    ``backward_gla`` with alpha_tk = a_t on every feature k (the selective
    recurrence with A_t = a_t I, dileepadev page, "Gating and Selective State
    Updates"). dQ, dK, dV are therefore those of the GLA form with g repeated
    over the features, and since every alpha_tk is the same function of g_t,
    dL/dg_t = sum_k dL/dg_tk (the chain rule for a shared input).
    """
    g = _f64(g)
    r = feature_map(Q[..., :1, :], fmap, omega).shape[-1]
    G = np.repeat(g[..., None], r, axis=-1)
    dQ, dK, dV, dG = backward_gla(Q, K, V, dO, G, tau, fmap, omega, eps, S0, z0)
    return dQ, dK, dV, dG.sum(axis=-1)


def backward_outer(Q, K, V, dO, g, gv, tau, fmap="elu1", omega=None, eps=1e-6, S0=None, z0=None):
    """(dQ, dK, dV, dg, dgv) of L = sum_i dO_i . o_i for the causal form with
    the outer-product gate G_t = alpha_t beta_t^T, all float64.

    Forward (the dileepadev page, "Gating and Selective State Updates", a gate
    matrix applied elementwise to the state; read as a key-side factor
    alpha_t = sigmoid(g_t)^(1/tau) per feature times a value-side factor
    beta_t = sigmoid(gv_t)^(1/tau) per value column, z gated by alpha only):
    with A_t = sum_{u<=t} log alpha_u and C_t = sum_{u<=t} log beta_u,
      W_ij   = sum_k phi(q_i)_k phi(k_j)_k exp(A_ik - A_jk)          (j <= i)
      num_ie = sum_{j<=i} W_ij v_je exp(C_ie - C_je) + exp(C_ie) sum_k phi(q_i)_k exp(A_ik) S0_ke
      den_i  = sum_{j<=i} W_ij + sum_k phi(q_i)_k exp(A_ik) z0_k + eps,   o_i = num_i / den_i.
    Chain rule, written out:
      g_i = dO_i / den_i,  h_i = -(dO_i . o_i) / den_i
      dW_ij = sum_e g_ie v_je exp(C_ie - C_je) + h_i      (num and den through W_ij)
      dv_je = sum_{i>=j} W_ij g_ie exp(C_ie - C_je)
      dphi_q, dphi_k and dA_t = dphi_q_t phi_q_t - dphi_k_t phi_k_t as in
        ``backward_gla`` with this dW (the carried state adds
        exp(A_ik) (sum_e S0_ke exp(C_ie) g_ie + z0_k h_i) to dphi_q_ik)
      dC_te = g_te num_te - dv_te v_te   (C_t enters num_t with + and every
        later query's pair with key t with -)
      d log alpha_u = sum_{t>=u} dA_t,  d log beta_u = sum_{t>=u} dC_t
      dg = d log alpha sigmoid(-g) / tau,  dgv = d log beta sigmoid(-gv) / tau.
    """
    V = _f64(V)
    dO = _f64(dO)
    g = _f64(g)
    gv = _f64(gv)
    pq = feature_map(Q, fmap, omega)
    pk = feature_map(K, fmap, omega)
    B, H, n, r = pq.shape
    with np.errstate(over="ignore"):
        loga = -np.logaddexp(0.0, -g) / float(tau)
        logb = -np.logaddexp(0.0, -gv) / float(tau)
    Ac = np.cumsum(loga, axis=2)                                  # [B, H, n, r]
    Cc = np.cumsum(logb, axis=2)                                  # [B, H, n, d_v]
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    mask = (j <= i)
    Dk = np.where(mask[None, None, :, :, None], np.exp(np.minimum(Ac[:, :, :, None, :] - Ac[:, :, None, :, :], 0.0)),
                  0.0)                                            # [B, H, i, j, r]
    Dv = np.where(mask[None, None, :, :, None], np.exp(np.minimum(Cc[:, :, :, None, :] - Cc[:, :, None, :, :], 0.0)),
                  0.0)                                            # [B, H, i, j, d_v]
    W = np.einsum("bhik,bhjk,bhijk->bhij", pq, pk, Dk)
    num = np.einsum("bhij,bhije,bhje->bhie", W, Dv, V)
    den = W.sum(axis=-1) + eps
    ca = np.exp(Ac)
    cb = np.exp(Cc)
    if S0 is not None:
        S0 = _f64(S0)
        z0 = _f64(z0)
        num = num + cb * np.einsum("bhik,bhke->bhie", pq * ca, S0)
        den = den + np.einsum("bhik,bhk->bhi", pq * ca, z0)
    if not normalised(fmap):
        den = np.ones_like(den)   # the state-space read-out o = num
    o = num / den[..., None]
    gg = dO / den[..., None]
    h = -np.sum(dO * o, axis=-1) / den if normalised(fmap) else np.zeros(den.shape)
    dW = (np.einsum("bhie,bhije,bhje->bhij", gg, Dv, V) + h[..., None]) * mask[None, None]
    dV = np.einsum("bhij,bhije,bhie->bhje", W, Dv, gg)
    dpq = np.einsum("bhij,bhjk,bhijk->bhik", dW, pk, Dk)
    dpk = np.einsum("bhij,bhik,bhijk->bhjk", dW, pq, Dk)
    if S0 is not None:
        dpq = dpq + ca * (np.einsum("bhke,bhie->bhik", S0, gg * cb) + h[..., None] * z0[:, :, None, :])
    dA = dpq * pq - dpk * pk
    dC = gg * num - dV * V
    suffix = lambda x: np.flip(np.cumsum(np.flip(x, axis=2), axis=2), axis=2)
    with np.errstate(over="ignore"):
        dg = suffix(dA) / (1.0 + np.exp(g)) / float(tau)
        dgv = suffix(dC) / (1.0 + np.exp(gv)) / float(tau)
    dQ = feature_map_vjp(Q, dpq, fmap, omega)
    dK = feature_map_vjp(K, dpk, fmap, omega)
    return dQ, dK, dV, dg, dgv


def backward_gla_rows(Q, K, V, dO, g, tau, fmap="elu1", eps=1e-6, rows=(), tail=0, return_forward=False):
    """Sampled entries of ``backward_gla`` for ONE head at any sequence length.

    Q, K [n, d_k]; V, dO [n, d_v]; g [n, r] (no carried state). Returns
    (dQ[rows], dK[rows], dV[rows], dg[n - tail:]). ``backward_gla`` holds an
    [n, n, r] decay tensor; here each sampled row sums over its own partners
    with the decays of that row only, so memory is O(n r):
      forward: z_t = alpha_t * z_{t-1} + phi(k_t), S_t = diag(alpha_t) S_{t-1}
               + phi(k_t) v_t^T (the recurrence of "Gating and Selective State
               Updates", dileepadev page), den_t = phi(q_t).z_t + eps, o_t;
      g_t = dO_t / den_t, h_t = -(dO_t . o_t) / den_t (state-space: dO_t, 0);
      key row j:   D_ij = exp(B_i - B_j) for i >= j, W_ij = sum_k phi(q_i)_k
                   phi(k_j)_k D_ijk, dV_j = sum_i W_ij g_i, dphi(k_j) =
                   sum_i (g_i . v_j + h_i) phi(q_i) D_ij;
      query row i: dphi(q_i) = sum_{j <= i} (g_i . v_j + h_i) phi(k_j) D_ij;
      tail u:      d log alpha_u = sum_{t >= u} (dphi(q_t) phi(q_t) -
                   dphi(k_t) phi(k_t)), dg_u = d log alpha_u sigmoid(-g_u) / tau;
    then the feature map's vjp, as in ``backward_gla``. With return_forward,
    also (den, o) of every token.
    """
    Q, K, V, dO, g = (_f64(x) for x in (Q, K, V, dO, g))
    pq = feature_map(Q, fmap)
    pk = feature_map(K, fmap)
    n, r = pq.shape
    dv = V.shape[1]
    with np.errstate(over="ignore"):
        la = -np.logaddexp(0.0, -g) / float(tau)
    Bc = np.cumsum(la, axis=0)
    al = np.exp(la)
    S = np.zeros((r, dv))
    z = np.zeros(r)
    o = np.empty((n, dv))
    den = np.ones(n)
    norm = normalised(fmap)
    for t in range(n):
        S = al[t][:, None] * S + np.outer(pk[t], V[t])
        z = al[t] * z + pk[t]
        o[t] = pq[t] @ S
        if norm:
            den[t] = pq[t] @ z + eps
            o[t] /= den[t]
    gg = dO / den[:, None]
    h = -np.sum(dO * o, axis=1) / den if norm else np.zeros(n)

    def dphi_k(j):
        D = np.exp(Bc[j:] - Bc[j])                       # [n - j, r], i >= j
        dW = gg[j:] @ V[j] + h[j:]
        W = (pq[j:] * D) @ pk[j]
        return (dW[:, None] * pq[j:] * D).sum(axis=0), W @ gg[j:]

    def dphi_q(i):
        D = np.exp(Bc[i] - Bc[:i + 1])                   # [i + 1, r], j <= i
        dW = V[:i + 1] @ gg[i] + h[i]
        return (dW[:, None] * pk[:i + 1] * D).sum(axis=0)

    rows = list(rows)
    dQ = np.array([feature_map_vjp(Q[i], dphi_q(i), fmap) for i in rows]).reshape(len(rows), -1)
    dK, dV = [], []
    for j in rows:
        dpk, dvj = dphi_k(j)
        dK.append(feature_map_vjp(K[j], dpk, fmap))
        dV.append(dvj)
    dK = np.array(dK).reshape(len(rows), -1)
    dV = np.array(dV).reshape(len(rows), dv)
    dB = np.array([dphi_q(t) * pq[t] - dphi_k(t)[0] * pk[t] for t in range(n - tail, n)]).reshape(tail, r)
    dlog = np.flip(np.cumsum(np.flip(dB, axis=0), axis=0), axis=0)
    with np.errstate(over="ignore"):
        dg = dlog / (1.0 + np.exp(g[n - tail:])) / float(tau)
    if return_forward:
        return dQ, dK, dV, dg, den, o
    return dQ, dK, dV, dg


def backward_sel_rows(Q, K, V, dO, g, tau, fmap="elu1", eps=1e-6, rows=(), tail=0):
    """``backward_gla_rows`` for the selective scalar gate (g [n]): the GLA
    form with g repeated over the features, dg summed over them (as in
    ``backward_sel``)."""
    g = _f64(g)
    r = feature_map(_f64(Q)[:1], fmap).shape[-1]
    dQ, dK, dV, dG = backward_gla_rows(Q, K, V, dO, np.repeat(g[:, None], r, axis=1), tau, fmap, eps, rows, tail)
    return dQ, dK, dV, dG.sum(axis=1)
