"""Plain fp64 softmax attention: the quadratic baseline that linear attention replaces.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle/``): the GPU tests, the
smoke check and the benchmark's CPU-baseline leg may use it; the HIP library
never does. It shares no code with the HIP kernels.

[LAM-d] "Standard Self-Attention: The Quadratic Baseline" ("Linear Attention
Mechanisms", dileepadev.github.io): every query scores every key, the n x n
score matrix is normalised row by row with a softmax, and the rows weight the
values; [LAM-s] "Why attention is quadratic" (sadullah.online) gives the same
form with the 1/sqrt(d) temperature. The causal form keeps keys j <= i (the
mask of the recurrent, autoregressive use on the same pages).
"""
from __future__ import annotations

import numpy as np


def scores(Q, K, scale):
    """S_ij = scale * q_i . k_j, shape [B, H, n, n] (the quadratic object itself)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    return scale * np.matmul(Q, np.swapaxes(K, -1, -2))


def softmax_attention(Q, K, V, causal=True, scale=None):
    """o_i = sum_j softmax_j(S_ij) v_j, the row softmax taken over the keys each
    query may see (all of them, or j <= i when causal). ``scale`` defaults to
    1/sqrt(d). Each row is shifted by its own maximum before exp (a shift that
    cancels in the ratio, so the value is the textbook definition's)."""
    V = np.asarray(V, dtype=np.float64)
    d = np.shape(Q)[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    S = scores(Q, K, scale)
    n = S.shape[-1]
    if causal:
        S = np.where(np.tril(np.ones((n, n), dtype=bool)), S, -np.inf)
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P = P / P.sum(axis=-1, keepdims=True)
    return np.matmul(P, V)


def softmax_attention_rows(Q, K, V, rows, causal=True, scale=None):
    """The same outputs for selected query rows only (any n, O(len(rows) n d)
    memory): o_i for i in ``rows`` of every (b, h)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = Q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else float(scale)
    out = np.empty(Q.shape[:2] + (len(rows), V.shape[-1]))
    for r, i in enumerate(rows):
        hi = i + 1 if causal else K.shape[2]
        s = scale * np.einsum("bhd,bhjd->bhj", Q[:, :, i], K[:, :, :hi])
        s = s - s.max(axis=-1, keepdims=True)
        p = np.exp(s)
        out[:, :, r] = np.einsum("bhj,bhje->bhe", p / p.sum(axis=-1, keepdims=True), V[:, :, :hi])
    return out
