"""Pins of the fp64 softmax-attention oracle (oracle/softmax.py) against a
library routine and closed forms, so that a slip in it (a transposed operand,
a missing temperature, a strict or missing mask, a softmax over the wrong
axis) fails here before a kernel is ever compared with it."""
import numpy as np
import pytest
import torch

from oracle import softmax as osm


def _qkv(seed, B=2, H=3, n=37, d=16, dv=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, n, d)), rng.standard_normal((B, H, n, d)),
            rng.standard_normal((B, H, n, dv)))


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("scale", [None, 0.3])
def test_matches_torch_sdpa_fp64(causal, scale):
    Q, K, V = _qkv(1)
    got = osm.softmax_attention(Q, K, V, causal=causal, scale=scale)
    t = lambda a: torch.from_numpy(a)
    ref = torch.nn.functional.scaled_dot_product_attention(t(Q), t(K), t(V), is_causal=causal, scale=scale).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12


def test_zero_keys_give_prefix_means():
    """All scores equal: the causal output is the mean of the values seen so far."""
    Q, K, V = _qkv(2)
    got = osm.softmax_attention(Q, np.zeros_like(K), V, causal=True)
    ref = np.cumsum(V, axis=2) / np.arange(1, V.shape[2] + 1)[None, None, :, None]
    assert np.max(np.abs(got - ref)) < 1e-13
    full = osm.softmax_attention(Q, np.zeros_like(K), V, causal=False)
    assert np.max(np.abs(full - V.mean(axis=2, keepdims=True))) < 1e-13


def test_shift_of_every_key_cancels():
    """Adding one vector c to every key adds scale q_i . c to a whole row of scores."""
    Q, K, V = _qkv(3)
    c = np.random.default_rng(4).standard_normal(K.shape[-1])
    a = osm.softmax_attention(Q, K, V, causal=True)
    b = osm.softmax_attention(Q, K + c, V, causal=True)
    assert np.max(np.abs(a - b)) < 1e-12


def test_dominant_key_selects_its_value():
    """A query aligned with one key far more than with any other returns that key's value."""
    Q, K, V = _qkv(5, n=20, d=16)
    K = K * 0.01
    K[:, :, 7] = 0.0
    K[:, :, 7, 0] = 1.0
    Q = np.zeros_like(Q)
    Q[..., 0] = 4000.0  # scale 1/4: score 1000 for key 7, |score| < 0.5 for the rest
    got = osm.softmax_attention(Q, K, V, causal=False)
    assert np.max(np.abs(got - V[:, :, 7:8])) < 1e-12
    # causal: rows before 7 cannot see key 7; row 7 and later select it
    gc = osm.softmax_attention(Q, K, V, causal=True)
    assert np.max(np.abs(gc[:, :, 7:] - V[:, :, 7:8])) < 1e-12
    assert np.max(np.abs(gc[:, :, 0] - V[:, :, 0])) < 1e-12  # row 0 sees only key 0


def test_noncausal_is_permutation_invariant():
    Q, K, V = _qkv(6)
    perm = np.random.default_rng(7).permutation(K.shape[2])
    a = osm.softmax_attention(Q, K, V, causal=False)
    b = osm.softmax_attention(Q, K[:, :, perm], V[:, :, perm], causal=False)
    assert np.max(np.abs(a - b)) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_selected_rows_equal_the_full_form(causal):
    Q, K, V = _qkv(8, n=50)
    rows = [0, 1, 17, 49]
    full = osm.softmax_attention(Q, K, V, causal=causal)
    part = osm.softmax_attention_rows(Q, K, V, rows, causal=causal)
    assert np.max(np.abs(part - full[:, :, rows])) < 1e-13


def test_score_matrix_is_n_by_n():
    Q, K, _ = _qkv(9, n=33)
    assert osm.scores(Q, K, 1.0).shape == (2, 3, 33, 33)
