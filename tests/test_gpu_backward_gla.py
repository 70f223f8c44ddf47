"""GPU parity of the causal backward pass with the diagonal GLA gate
(la_backward with dg) against the fp64 gradient oracle
(oracle.la_backward.backward_gla) on the same seeded inputs.

The metric is the one of test_gpu_backward.py: the entrywise error over the
sum of the magnitudes of the terms each gradient entry sums, here with the
per-feature decay factors inside the sums. d log alpha_u is the sum of the
terms of the pairs (query i >= u, key j < u) whose weight alpha_u decays, plus
the carried-in state's terms of the queries i >= u; dg_u is that times
sigmoid(-g_u) / tau, and its scale is the magnitude sum of those terms. Where
no pair crosses u (u = 0 without a carried state) the exact value is zero and
the scale is the bound of what the kernel's suffix sum leaves over (see
gla_scales). The oracle's explicit form holds an [n, n, r] decay tensor per
head, so the oracle runs head by head on sampled heads.
"""
import numpy as np
import pytest
import torch

from oracle import la_backward as obwd
from oracle.la_oracle import feature_map
from workloads import WORKLOADS, make_inputs, to_f64, incoming_gradient
from _helpers import dev, gpu_gate

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _head(inp, dO, head, S0=None, z0=None):
    b, h = head
    sl = lambda x: None if x is None else to_f64(x)[b:b + 1, h:h + 1]
    return (sl(inp["Q"]), sl(inp["K"]), sl(inp["V"]), sl(dO), sl(inp["g"]), sl(S0), sl(z0))


def gla_scales(Q, K, V, dO, g, tau, eps, S0=None, z0=None):
    """Magnitude sums of the terms behind dQ, dK, dV and dg (one head)."""
    pq = feature_map(Q, "elu1")
    pk = feature_map(K, "elu1")
    n = Q.shape[2]
    la = -np.logaddexp(0.0, -g) / tau
    Bc = np.cumsum(la, axis=2)
    mask = np.tril(np.ones((n, n), dtype=bool))
    D = np.where(mask[None, None, :, :, None],
                 np.exp(np.minimum(Bc[:, :, :, None, :] - Bc[:, :, None, :, :], 0.0)), 0.0)
    W = np.einsum("bhik,bhjk,bhijk->bhij", pq, pk, D)
    num = W @ V
    den = W.sum(axis=-1) + eps
    c = np.exp(Bc)
    if S0 is not None:
        num = num + (pq * c) @ S0
        den = den + np.einsum("bhik,bhk->bhi", pq * c, z0)
    o = num / den[..., None]
    gg = dO / den[..., None]
    hh = -np.sum(dO * o, axis=-1) / den
    T = (np.abs(gg) @ np.abs(np.swapaxes(V, -1, -2)) + np.abs(hh)[..., None]) * mask
    sq = np.einsum("bhij,bhjk,bhijk->bhik", T, pk, D)
    if S0 is not None:
        sq = sq + c * (np.abs(gg) @ np.abs(np.swapaxes(S0, -1, -2)) + np.abs(hh)[..., None] * z0[:, :, None, :])
    sk = np.einsum("bhij,bhik,bhijk->bhjk", T, pq, D)
    sv = np.einsum("bhij,bhie->bhje", W, np.abs(gg))
    # d log alpha_u sums the terms of the pairs (i >= u, j < u) that alpha_u
    # decays, and the carried-in state's terms of every query i >= u
    M = T[..., None] * pq[:, :, :, None, :] * pk[:, :, None, :, :] * D          # [b, h, i, j, k]
    P = np.cumsum(M, axis=3) - M                                                 # sum over j < u, at [i, u]
    i = np.arange(n)[:, None]
    P = np.where((i >= i.T)[None, None, :, :, None], P, 0.0)
    cross = P.sum(axis=2)                                                        # [b, h, u, k]
    if S0 is not None:
        st = c * pq * (np.abs(gg) @ np.abs(np.swapaxes(S0, -1, -2)) + np.abs(hh)[..., None] * z0[:, :, None, :])
        cross = cross + np.flip(np.cumsum(np.flip(st, axis=2), axis=2), axis=2)
    # where no pair crosses (u = 0 without a carried state) d log alpha_u is
    # exactly zero; the kernel sums dB_t over the whole suffix, whose pair
    # terms cancel up to one bf16 rounding of the state each side reads them
    # through: 2^-8 of the suffix's magnitude sum bounds what is left
    suffix = np.flip(np.cumsum(np.flip(sq * pq + sk * pk, axis=2), axis=2), axis=2)
    sdg = np.where(cross > 0, cross, suffix * 2.0 ** -8) / (1.0 + np.exp(g)) / tau
    dphi = lambda x: np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    return sq * dphi(Q), sk * dphi(K), sv, sdg


def run_backward_gla(inp, dO, S0=None, z0=None):
    import kernelized_sequence_mixing_amd as ksm
    res = ksm.backward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(dO), fmap="elu1", gate=gpu_gate(inp),
                       eps=inp["eps"], S0=dev(S0), z0=dev(z0))
    torch.cuda.synchronize()
    assert len(res) == 4
    return tuple(x.cpu() for x in res)


def check_heads(got, inp, dO, heads, what, S0=None, z0=None):
    for head in heads:
        b, h = head
        Q, K, V, d, g, s0, z = _head(inp, dO, head, S0, z0)
        z = None if z is None else z
        ref = obwd.backward_gla(Q, K, V, d, g, inp["tau"], "elu1", None, inp["eps"], s0, z)
        scales = gla_scales(Q, K, V, d, g, inp["tau"], inp["eps"], s0, z)
        errs = []
        for x, r, sc in zip(got, ref, scales):
            xg = to_f64(x[b:b + 1, h:h + 1])
            assert np.isfinite(xg).all()
            errs.append(float(np.max(np.abs(xg - r) / (sc + 1e-30))))
        dgh = float(np.max(np.abs(to_f64(got[3][b:b + 1, h:h + 1]) - ref[3])) / (np.max(np.abs(ref[3])) + 1e-30))
        print(f"  {what} head {head}: term-relative dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e} "
              f"dg {errs[3]:.2e}; dg of the head max {dgh:.2e}", flush=True)
        for nm, e in zip(("dQ", "dK", "dV", "dg"), errs):
            assert e < TOL_GRAD, (what, head, nm, e)


def _case(d, dv, B, H, n, seed=3):
    wl = WORKLOADS["gla_gate"].resized(d_k=d, d_v=dv, r=d)
    inp = make_inputs(wl, seed=seed, B=B, H=H, n=n)
    dO = incoming_gradient((B, H, n, dv), seed + 100)
    return wl, inp, dO


CASES = [(64, 64, 2, 4, 777), (64, 64, 4, 16, 1285), (128, 64, 2, 4, 300), (64, 128, 2, 4, 300),
         (64, 64, 2, 4, 200), (64, 64, 1, 1, 1), (64, 64, 2, 1, 65)]


@pytest.mark.parametrize("d,dv,B,H,n", CASES)
def test_backward_gla_parity(d, dv, B, H, n):
    """Many one-chunk segments with a ragged tail (n 777), segments of three
    chunks (n 1285), one segment (n 200, 300), tiny n, each built shape."""
    wl, inp, dO = _case(d, dv, B, H, n)
    got = run_backward_gla(inp, dO)
    heads = sorted({(0, 0), (B - 1, H - 1)} | ({(B // 2, H // 2)} if n < 1000 else set()))
    check_heads(got, inp, dO, heads, f"gla d{d}x{dv} B{B} H{H} n{n}")


def test_backward_gla_with_carried_state():
    """The carried-in state enters dQ~ with the weight e^{B_t}, hence dg."""
    wl, inp, dO = _case(64, 64, 4, 16, 700, seed=9)
    rng = np.random.default_rng(77)
    S0 = torch.from_numpy((rng.standard_normal((4, 16, 64, 64)) * 2.0).astype(np.float32))
    z0 = torch.from_numpy((20.0 + 2.0 * np.abs(rng.standard_normal((4, 16, 64)))).astype(np.float32))
    got = run_backward_gla(inp, dO, S0, z0)
    check_heads(got, inp, dO, [(0, 0), (3, 15)], "gla carried state", S0, z0)


def test_backward_gla_deterministic():
    wl, inp, dO = _case(64, 64, 4, 16, 1285, seed=4)
    a = run_backward_gla(inp, dO)
    b = run_backward_gla(inp, dO)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
