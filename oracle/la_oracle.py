"""Plain fp64 CPU oracle for kernelized linear attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only the test suite, the smoke check and the CPU-baseline leg of
the benchmark use it. It shares no code with the HIP library; the two meet only
through the seeded inputs produced by ``workloads``.

Everything is computed in float64 from the exact values the GPU sees (bf16 or
fp32 inputs upcast without change). Each function follows one passage of the
pages it cites; nothing is blocked, fused or reordered beyond what that passage
states. Array layout everywhere: ``[B, H, n, d]``; the state ``S`` is
``[B, H, r, d_v]`` and the normaliser ``z`` is ``[B, H, r]``.

Pages cited (title, site):
  * "Linear Attention Mechanisms" (sadullah.online)          -- [LAM-s]
  * "Linear Attention Mechanisms" (dileepadev.github.io)     -- [LAM-d]
  * "Attention-Free / Sub-Quadratic Architectures"
    (blog.vguerra.net)                                       -- [AFA]

Readings taken where the pages are silent or garbled are listed with each
function; every one of them is pinned by a test in ``tests/test_oracle_pins.py``
except where a docstring says "parity unpinned".
"""
from __future__ import annotations

import numpy as np

FMAPS = ("elu1", "favor", "identity")
GATES = ("none", "decay", "gla", "sel", "outer")


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Feature maps
# ---------------------------------------------------------------------------

def phi_elu1(x):
    """phi(x) = elu(x) + 1, elementwise, with the ELU slope parameter 1.

    [LAM-d] "Choosing the Feature Map phi", ELU-based features (Linear
    Transformer); [AFA] "Feature maps phi (must keep similarities >= 0)".
    elu(x) is x for x > 0 and exp(x) - 1 otherwise, so elu(x) + 1 is x + 1 for
    x > 0 and exp(x) for x <= 0 (the exp branch is written directly, which is
    the same number without the cancellation of (exp(x) - 1) + 1).
    """
    x = _f64(x)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_favor(x, omega):
    """FAVOR+ positive random features phi(x)_m = exp(w_m.x - |x|^2/2) / sqrt(r).

    [LAM-d] "Choosing the Feature Map phi": positive (and orthogonal) random
    features whose inner product is an unbiased estimate of exp(q.k); [AFA]
    "Feature maps phi": phi(q).phi(k) approximates exp(q.k).
    Reading: the page prints exp(w.x)/sqrt(r) without the -|x|^2/2 term; only
    the form with that term has expectation exp(q.k) for w ~ N(0, I), which is
    the property both pages state, so that form is used. ``omega`` is [r, d]
    (the random frequencies are an input, drawn outside this module).
    """
    x = _f64(x)
    om = _f64(omega)
    r = om.shape[0]
    proj = np.einsum("...d,md->...m", x, om)
    half_sq = 0.5 * np.sum(x * x, axis=-1, keepdims=True)
    return np.exp(proj - half_sq) / np.sqrt(r)


def feature_map(x, fmap="elu1", omega=None):
    """Apply the named feature map phi over the last axis.

    "identity" is the state-space reading ([LAM-d] "State Space Models as
    Linear Attention": h_t = A_t h_{t-1} + B_t x_t, y_t = C_t^T h_t; [AFA]
    "Evolution: add decay/gating", the bridge to Mamba): the inputs C_t = q_t
    and B_t = k_t enter as they are, and the read-out is not normalised (see
    ``normalised``).
    """
    if fmap == "identity":
        return _f64(x)
    if fmap == "elu1":
        return phi_elu1(x)
    if fmap == "favor":
        if omega is None:
            raise ValueError("favor feature map needs omega")
        return phi_favor(x, omega)
    raise ValueError(f"unknown feature map {fmap!r}")


def normalised(fmap):
    """Whether the read-out divides by phi(q).z + eps.

    The attention forms are normalised ([LAM-d] "The Kernel Trick for
    Attention"). The state-space form reads y_t = C_t^T h_t directly ([LAM-d]
    "State Space Models as Linear Attention"); its inputs may be negative, so a
    denominator phi(q).z would have no sign ([AFA] notes the normaliser's
    fragility). Reading: the identity feature map means the SSM read-out.
    """
    return fmap != "identity"


# ---------------------------------------------------------------------------
# Gates
# ---------------------------------------------------------------------------

def gla_alpha(g, tau):
    """Per-step diagonal GLA gate alpha_t = sigmoid(g_t) ** (1 / tau).

    [LAM-d] "Gating and Selective State Updates", Gated Linear Attention: a
    data-dependent gate in (0, 1) multiplies the previous state. Reading: the
    gate is diagonal on the key (feature) axis, G_t = alpha_t 1^T, i.e. row k
    of S is scaled by alpha_{t,k}; alpha comes from a raw input g through a
    sigmoid raised to 1/tau.
    """
    g = _f64(g)
    with np.errstate(over="ignore"):  # exp(-g) -> inf gives sigmoid 0 exactly
        sig = 1.0 / (1.0 + np.exp(-g))
    return sig ** (1.0 / float(tau))


def sel_alpha(g, tau):
    """Per-step scalar selective gate a_t = sigmoid(g_t) ** (1 / tau) per head.

    [LAM-d] "State Space Models as Linear Attention": Mamba makes A_t depend
    on the input; [AFA] "Evolution: add decay/gating": Mamba is the
    content-dependent (selective) version of the gated recurrence
    S_i = gamma S_{i-1} + phi(k_i) v_i^T. Reading: the selective A_t is one
    number per step and head (A_t = a_t I, the RetNet decay made
    input-dependent), from a raw input g [B, H, n] through the same sigmoid
    and 1/tau as the GLA gate; the per-feature A_t is the GLA gate itself.
    """
    return gla_alpha(g, tau)


def _gate_factor(gate, t, B, H):
    """Multiplier applied to the previous state before step t.

    Returns an array broadcastable to S [B, H, r, 1] rows (shape [B, H, r],
    [B, H, 1] or [1, H, 1]), or None when there is no gate.
    """
    if gate is None or gate[0] == "none":
        return None
    kind = gate[0]
    if kind == "decay":
        gamma = _f64(gate[1]).reshape(1, H, 1)
        return gamma
    if kind == "gla":
        g, tau = gate[1], gate[2]
        return gla_alpha(np.asarray(g)[:, :, t, :], tau)
    if kind == "sel":
        g, tau = gate[1], gate[2]
        return sel_alpha(np.asarray(g)[:, :, t], tau)[:, :, None]
    if kind == "outer":
        g, tau = gate[1], gate[3]
        return gla_alpha(np.asarray(g)[:, :, t, :], tau)
    raise ValueError(f"unknown gate {kind!r}")


def outer_beta(gv, tau):
    """Value-side factor of the outer-product gate, beta_t = sigmoid(gv_t) ** (1 / tau).

    [LAM-d] "Gating and Selective State Updates" gives the gate as a matrix
    G_t in (0, 1)^{d x d} applied elementwise to the state. Reading: the
    outer-product gate G_t = alpha_t beta_t^T, a key-side factor alpha_t (the
    diagonal GLA gate) times a value-side factor beta_t per value column, both
    from raw inputs through the GLA gate's sigmoid and 1/tau. Beta = 1 is the
    GLA gate. The normaliser z, S's column for a constant value of 1, takes
    the key side only (that constant is not a value column with a gate).
    """
    return gla_alpha(gv, tau)


def _gate_factor_v(gate, t):
    """Value-side multiplier of the previous state before step t ([B, H, d_v]),
    or None (every gate but the outer-product one)."""
    if gate is None or gate[0] != "outer":
        return None
    return outer_beta(np.asarray(gate[2])[:, :, t, :], gate[3])


# ---------------------------------------------------------------------------
# Non-causal form (reassociated)
# ---------------------------------------------------------------------------

def noncausal(Q, K, V, fmap="elu1", omega=None, eps=1e-6):
    """Non-causal read-out o_i = phi(q_i).S / (phi(q_i).z + eps) over all keys.

    [LAM-d] "The Kernel Trick for Attention": S = sum_j phi(k_j) v_j^T and
    z = sum_j phi(k_j), both formed once and shared by every query; [AFA]
    "Linear Attention (the core trick)". The eps added to the denominator
    follows [LAM-s] "The linear attention trick: drop or approximate the
    softmax". Here z is kept as the last column of one augmented state: it is
    the state column of a value that is the constant 1, so a single product
    phi(q_i)^T [S | z] gives numerator and denominator together.
    """
    if not normalised(fmap):
        raise ValueError("the state-space read-out is defined for the causal form only")
    V = _f64(V)
    ones = np.ones(V.shape[:-1] + (1,))
    Va = np.concatenate([V, ones], axis=-1)                           # [B, H, n, d_v + 1]
    Sa = np.matmul(np.swapaxes(feature_map(K, fmap, omega), -1, -2), Va)  # [B, H, r, d_v + 1] = [S | z]
    y = np.matmul(feature_map(Q, fmap, omega), Sa)                    # [B, H, n, d_v + 1]
    return y[..., :-1] / (y[..., -1:] + eps)


# ---------------------------------------------------------------------------
# Explicit n x n kernel-matrix form (quadratic; tiny inputs only)
# ---------------------------------------------------------------------------

def kernel_weights(Q, K, fmap="elu1", omega=None, causal=False, gate=None):
    """Explicit weights W_ij = sum_k phi(q_i)_k phi(k_j)_k D_ijk, shape [B, H, n, n].

    [LAM-d] "The Kernel Trick for Attention": the similarity of query i and key
    j is phi(q_i)^T phi(k_j). Causal: only j <= i contributes ([LAM-d]
    "Recurrent Reformulation"; [AFA] "The recurrent form (causal)"). RetNet:
    key j is discounted by gamma^(i-j) ([LAM-d] "Gating and Selective State
    Updates"). GLA: key j is multiplied, per feature k, by the product of the
    gates of the steps after j up to i, which is what unrolling
    S_t = G_t * S_{t-1} + phi(k_t) v_t^T gives; the scalar selective gate the
    same with one factor per step shared by all features.
    """
    pq = feature_map(Q, fmap, omega)
    pk = feature_map(K, fmap, omega)
    B, H, n, r = pq.shape
    kind = "none" if gate is None else gate[0]
    if kind != "none" and not causal:
        raise ValueError("gates are defined for the causal form only")
    W = np.zeros((B, H, n, n))
    if kind == "gla":
        alpha = gla_alpha(gate[1], gate[2])  # [B, H, n, r]
    if kind == "sel":
        alpha = sel_alpha(gate[1], gate[2])[..., None]  # [B, H, n, 1]
    for i in range(n):
        for j in range(n):
            if causal and j > i:
                continue
            if kind == "none":
                D = 1.0
            elif kind == "decay":
                D = (_f64(gate[1]) ** (i - j)).reshape(1, H, 1)
            else:
                D = np.prod(alpha[:, :, j + 1:i + 1, :], axis=2)  # empty product = 1
            W[:, :, i, j] = np.sum(pq[:, :, i, :] * pk[:, :, j, :] * D, axis=-1)
    return W


def attention_from_weights(W, V, eps=1e-6, normalise=True):
    """o_i = sum_j W_ij v_j / (sum_j W_ij + eps), or sum_j W_ij v_j unnormalised.

    [LAM-d] "The Kernel Trick for Attention" (the ratio form of o_i) with the
    eps of [LAM-s] "The linear attention trick"; the unnormalised sum is the
    read-out of [LAM-d] "State Space Models as Linear Attention".
    """
    V = _f64(V)
    num = np.einsum("bhij,bhje->bhie", W, V)
    if not normalise:
        return num
    den = W.sum(axis=-1) + eps
    return num / den[..., None]


def brute(Q, K, V, fmap="elu1", omega=None, causal=False, gate=None, eps=1e-6):
    """Quadratic reference: explicit weight matrix, then the mix (normalised
    unless ``fmap`` is the state-space "identity")."""
    if gate is not None and gate[0] == "outer":
        return brute_outer(Q, K, V, fmap, omega, gate, eps)
    W = kernel_weights(Q, K, fmap, omega, causal, gate)
    return attention_from_weights(W, V, eps, normalised(fmap))


def brute_outer(Q, K, V, fmap, omega, gate, eps=1e-6):
    """Explicit form of the causal outer-product gate ("outer", g, gv, tau).

    Unrolling S_t = (alpha_t beta_t^T) * S_{t-1} + phi(k_t) v_t^T, key j reaches
    query i >= j with the factor prod_{u=j+1..i} alpha_uk beta_ue on state
    entry (k, e): o_ie = sum_j W_ij D_ije v_je / (sum_j W_ij + eps), where W are
    the GLA weights of the key side (``kernel_weights`` with ("gla", g, tau))
    and D_ije = prod_{u=j+1..i} beta_ue; the denominator has no value-side
    factor (z takes the key side only, see ``outer_beta``).
    """
    V = _f64(V)
    W = kernel_weights(Q, K, fmap, omega, True, ("gla", gate[1], gate[3]))
    beta = outer_beta(gate[2], gate[3])  # [B, H, n, d_v]
    B, H, n, dv = V.shape
    num = np.zeros((B, H, n, dv))
    for i in range(n):
        for j in range(i + 1):
            D = np.prod(beta[:, :, j + 1:i + 1, :], axis=2)  # empty product = 1
            num[:, :, i, :] += W[:, :, i, j, None] * D * V[:, :, j, :]
    if not normalised(fmap):
        return num
    den = W.sum(axis=-1) + eps
    return num / den[..., None]


# ---------------------------------------------------------------------------
# Causal recurrent form (the matrix-state RNN)
# ---------------------------------------------------------------------------

def causal_recurrent(Q, K, V, fmap="elu1", omega=None, gate=None, eps=1e-6,
                     S0=None, z0=None):
    """Token-by-token recurrence; returns (o, S_final, z_final).

    [LAM-d] "Recurrent Reformulation": S_t = S_{t-1} + phi(k_t) v_t^T,
    z_t = z_{t-1} + phi(k_t), o_t = phi(q_t)^T S_t / (phi(q_t)^T z_t); [AFA]
    "The recurrent form (causal)". Gated variants ([LAM-d] "Gating and
    Selective State Updates"; [AFA] "Evolution: add decay/gating"):
    S_t = G_t * S_{t-1} + phi(k_t) v_t^T with G_t = gamma_h (RetNet) or
    alpha_t scaling row k by alpha_{t,k} (GLA).
    Readings: the gate multiplies the previous state only (the current token
    enters with weight 1); z is gated exactly like S (z is S's column for a
    value of constant 1), which keeps the weights of each output summing to
    one; eps is added to the denominator as in [LAM-s]'s routine; the page
    calls z's update "scalar" but z has r entries (it is summed elementwise).
    ``gate`` is None, ("decay", gamma[H]), ("gla", g[B,H,n,r], tau),
    ("sel", g[B,H,n], tau) or ("outer", g[B,H,n,r], gv[B,H,n,d_v], tau) (the
    state entry (k, e) scaled by alpha_{t,k} beta_{t,e}, z by alpha_t; see
    ``outer_beta``). With the "identity" feature map the read-out is o_t = q_t^T S_t, the
    state-space y_t = C_t^T h_t (z is still carried, unused).
    """
    V = _f64(V)
    norm = normalised(fmap)
    pq = feature_map(Q, fmap, omega)
    pk = feature_map(K, fmap, omega)
    B, H, n, r = pq.shape
    dv = V.shape[-1]
    S = np.zeros((B, H, r, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros((B, H, r)) if z0 is None else _f64(z0).copy()
    out = np.empty((B, H, n, dv))
    for t in range(n):
        G = _gate_factor(gate, t, B, H)
        if G is not None:
            S = S * G[..., None]
            z = z * G
        Gv = _gate_factor_v(gate, t)
        if Gv is not None:
            S = S * Gv[:, :, None, :]
        S = S + pk[:, :, t, :, None] * V[:, :, t, None, :]
        z = z + pk[:, :, t, :]
        num = np.einsum("bhr,bhre->bhe", pq[:, :, t, :], S)
        if not norm:
            out[:, :, t, :] = num
            continue
        den = np.einsum("bhr,bhr->bh", pq[:, :, t, :], z) + eps
        out[:, :, t, :] = num / den[..., None]
    return out, S, z


def _step_log_gates(gate, B, H, n, dv):
    """Per-step log of the state multiplier: (key side [B, H, n, r or 1], value
    side [B, H, n, d_v] or None). The recurrence multiplies the previous state by
    exp of these before adding step t (see ``causal_recurrent``)."""
    kind = "none" if gate is None else gate[0]
    if kind == "none":
        return np.zeros((B, H, n, 1)), None
    if kind == "decay":
        return np.broadcast_to(np.log(_f64(gate[1])).reshape(1, H, 1, 1), (B, H, n, 1)), None
    if kind == "gla":
        return np.log(gla_alpha(gate[1], gate[2])), None
    if kind == "sel":
        return np.log(sel_alpha(gate[1], gate[2]))[..., None], None
    if kind == "outer":
        return np.log(gla_alpha(gate[1], gate[3])), np.log(outer_beta(gate[2], gate[3]))
    raise ValueError(f"unknown gate {kind!r}")


def causal_blocked(Q, K, V, fmap="elu1", omega=None, gate=None, eps=1e-6, S0=None, z0=None, block=256):
    """The causal form evaluated block by block; returns (o, S_final, z_final).

    The same quantities as ``causal_recurrent`` ([LAM-d] "Recurrent
    Reformulation" with the gates of "Gating and Selective State Updates"),
    grouped into blocks of ``block`` tokens: inside a block the explicit
    weights W_ij = sum_k phi(q_i)_k phi(k_j)_k D_ijk of ``kernel_weights``
    (j <= i, D the product of the gates of steps j+1 .. i, formed as the exp of
    a difference of cumulative log-gates, which is <= 0), and from the blocks
    before it the carried state, decayed by the gates of steps block start .. i.
    At the block's end the state takes the block: S <- D_end S + sum_j
    (phi(k_j) D_end,j) v_j^T (the outer-product gate also decays value column e
    by its own factors; z takes the key side only). Nothing here is a kernel
    optimisation: it is the sum of ``kernel_weights`` split at block edges, so
    that long sequences need O(n block r) memory, and its products run on the
    host's BLAS. Gates must be > 0 (their logs finite); a gate of exactly zero
    is the recurrent form's case.
    """
    V = _f64(V)
    norm = normalised(fmap)
    pq = feature_map(Q, fmap, omega)
    pk = feature_map(K, fmap, omega)
    B, H, n, r = pq.shape
    dv = V.shape[-1]
    lk, lv = _step_log_gates(gate, B, H, n, dv)
    S = np.zeros((B, H, r, dv)) if S0 is None else _f64(S0).copy()
    z = np.zeros((B, H, r)) if z0 is None else _f64(z0).copy()
    out = np.empty((B, H, n, dv))
    for t0 in range(0, n, block):
        t1 = min(n, t0 + block)
        L = t1 - t0
        mask = np.tril(np.ones((L, L), dtype=bool))
        bk = np.cumsum(lk[:, :, t0:t1], axis=2)                      # [B, H, L, r or 1], from the block start
        dk = np.where(mask[None, None, :, :, None],
                      np.exp(np.minimum(bk[:, :, :, None, :] - bk[:, :, None, :, :], 0.0)), 0.0)
        q_, k_ = pq[:, :, t0:t1], pk[:, :, t0:t1]
        if dk.shape[-1] == 1:
            W = np.matmul(q_, np.swapaxes(k_, -1, -2)) * dk[..., 0]
        else:
            W = np.matmul(dk * k_[:, :, None, :, :], q_[..., None])[..., 0]   # sum over k, per (i, j)
        qs = q_ * np.exp(bk)                                         # the carried state's decay to step i
        v_ = V[:, :, t0:t1]
        if lv is None:
            num = np.matmul(W, v_) + np.matmul(qs, S)
        else:
            bv = np.cumsum(lv[:, :, t0:t1], axis=2)                  # [B, H, L, d_v]
            dvv = np.where(mask[None, None, :, :, None],
                           np.exp(np.minimum(bv[:, :, :, None, :] - bv[:, :, None, :, :], 0.0)), 0.0)
            num = np.einsum("bhij,bhije,bhje->bhie", W, dvv, v_) + np.matmul(qs, S) * np.exp(bv)
        if norm:
            den = W.sum(axis=-1) + np.einsum("bhik,bhk->bhi", qs, z) + eps
            out[:, :, t0:t1] = num / den[..., None]
        else:
            out[:, :, t0:t1] = num
        # carry the state past the block
        ek = np.exp(bk[:, :, -1:] - bk)                              # gates of steps j+1 .. block end
        kd = k_ * ek
        if lv is None:
            S = S * np.exp(bk[:, :, -1])[..., None] + np.matmul(np.swapaxes(kd, -1, -2), v_)
        else:
            ev = np.exp(bv[:, :, -1:] - bv)
            S = (S * np.exp(bk[:, :, -1])[..., None] * np.exp(bv[:, :, -1])[:, :, None, :]
                 + np.matmul(np.swapaxes(kd, -1, -2), v_ * ev))
        z = z * np.exp(bk[:, :, -1]) + kd.sum(axis=2)
    return out, S, z


def decode_step(S, z, q, k, v, fmap="elu1", omega=None, gate=None, eps=1e-6):
    """One step of the recurrence from a given state: returns (o, S', z').

    [LAM-d] "Recurrent Reformulation" (rank-1 update of S, update of z, then
    the read-out); [AFA] "The recurrent form (causal)" (constant cost per
    token). q, k, v (and g for GLA) are [B, H, d] for the single new token;
    ``gate`` is None, ("decay", gamma[H]), ("gla", g[B,H,r], tau),
    ("sel", g[B,H], tau) or ("outer", g[B,H,r], gv[B,H,d_v], tau).
    """
    q4 = _f64(q)[:, :, None, :]
    k4 = _f64(k)[:, :, None, :]
    v4 = _f64(v)[:, :, None, :]
    g4 = gate
    if gate is not None and gate[0] == "gla":
        g4 = ("gla", _f64(gate[1])[:, :, None, :], gate[2])
    if gate is not None and gate[0] == "sel":
        g4 = ("sel", _f64(gate[1])[:, :, None], gate[2])
    if gate is not None and gate[0] == "outer":
        g4 = ("outer", _f64(gate[1])[:, :, None, :], _f64(gate[2])[:, :, None, :], gate[3])
    o, S1, z1 = causal_recurrent(q4, k4, v4, fmap, omega, g4, eps, S0=S, z0=z)
    return o[:, :, 0, :], S1, z1


# ---------------------------------------------------------------------------
# Softmax attention (what the method replaces) -- used by the FAVOR+ pins
# ---------------------------------------------------------------------------

def softmax_score_matrix_bytes(n, bytes_per_entry):
    """Bytes to hold one n x n score matrix.

    [LAM-d] "Standard Self-Attention: The Quadratic Baseline" quotes the size of
    this matrix at n = 16384 in float16.
    """
    return int(n) * int(n) * int(bytes_per_entry)
