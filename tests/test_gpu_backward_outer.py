"""GPU parity of the causal backward pass with the outer-product gate
G_t = alpha_t beta_t^T (la_backward with dg and dgv) against the fp64
gradient oracle (oracle.la_backward.backward_outer, pinned by finite
differences of the recurrent forward) on the same seeded inputs.

The metric is the one of the GLA backward test: each entry's error over the
sum of the magnitudes of the terms it sums, with both the per-feature and
the per-column decay factors inside those sums. d log beta_u sums, per value
column, the terms g_ie W_ij v_je of the pairs (i >= u, j < u) that beta_u
decays plus the carried-in state's terms of the queries i >= u. The kernel
sums dC_t = dO_t o_t - dV_t v_t from u to the end of u's segment and takes
the pairs that cross the segment's end from the states there, so the pair
terms inside that range cancel up to the bf16 roundings of the operands that
give o and dV: 2^-8 of the magnitude sum of everything it adds (all dC_t
terms from u on, a bound on the segment's) is added to the scale. The oracle
holds [n, n, r] and [n, n, d_v] decay tensors per head, so it runs head by
head on sampled heads.
"""
import numpy as np
import pytest
import torch

from oracle import la_backward as obwd
from oracle.la_oracle import causal_recurrent, feature_map
from workloads import WORKLOADS, make_inputs, strong_gate_input, to_f64, incoming_gradient
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
    return (sl(inp["Q"]), sl(inp["K"]), sl(inp["V"]), sl(dO), sl(inp["g"]), sl(inp["gv"]), sl(S0), sl(z0))


def _suffix(x):
    return np.flip(np.cumsum(np.flip(x, axis=2), axis=2), axis=2)


def outer_scales(Q, K, V, dO, g, gv, tau, eps, S0=None, z0=None, fmap="elu1"):
    """Magnitude sums of the terms behind dQ, dK, dV, dg and dgv (one head)."""
    norm = fmap != "identity"
    fq, fk = feature_map(Q, fmap), feature_map(K, fmap)
    pq, pk = np.abs(fq), np.abs(fk)
    n = Q.shape[2]
    la = -np.logaddexp(0.0, -g) / tau
    lb = -np.logaddexp(0.0, -gv) / tau
    Ac, Cc = np.cumsum(la, axis=2), np.cumsum(lb, axis=2)
    mask = np.tril(np.ones((n, n), dtype=bool))
    Dk = np.where(mask[None, None, :, :, None], np.exp(np.minimum(Ac[:, :, :, None, :] - Ac[:, :, None, :, :], 0.0)),
                  0.0)
    Dv = np.where(mask[None, None, :, :, None], np.exp(np.minimum(Cc[:, :, :, None, :] - Cc[:, :, None, :, :], 0.0)),
                  0.0)
    ca, cb = np.exp(Ac), np.exp(Cc)
    # signed forward quantities for g and h
    Ws = np.einsum("bhik,bhjk,bhijk->bhij", fq, fk, Dk)
    num = np.einsum("bhij,bhije,bhje->bhie", Ws, Dv, V)
    den = Ws.sum(axis=-1) + eps
    if S0 is not None:
        num = num + cb * ((fq * ca) @ S0)
        den = den + np.einsum("bhik,bhk->bhi", fq * ca, z0)
    if not norm:
        den = np.ones_like(den)
    o = num / den[..., None]
    gg = np.abs(dO / den[..., None])
    hh = np.abs(np.sum(dO * o, axis=-1) / den) if norm else np.zeros(den.shape)
    aV = np.abs(V)
    # magnitudes from here on
    W = np.einsum("bhik,bhjk,bhijk->bhij", pq, pk, Dk)
    T = (np.einsum("bhie,bhije,bhje->bhij", gg, Dv, aV) + hh[..., None]) * mask
    st = None
    if S0 is not None:
        st = ca * ((gg * cb) @ np.abs(np.swapaxes(S0, -1, -2)) + hh[..., None] * np.abs(z0)[:, :, None, :])
    sq = np.einsum("bhij,bhjk,bhijk->bhik", T, pk, Dk) + (st if st is not None else 0.0)
    sk = np.einsum("bhij,bhik,bhijk->bhjk", T, pq, Dk)
    sv = np.einsum("bhij,bhije,bhie->bhje", W, Dv, gg)
    # d log alpha (the GLA test's bound): the crossing pairs and the carried state's terms,
    # plus 2^-8 of the in-chunk suffix of |dB| and the terms crossing the chunk's end
    M = T[..., None] * pq[:, :, :, None, :] * pk[:, :, None, :, :] * Dk
    P = np.cumsum(M, axis=3) - M
    i = np.arange(n)[:, None]
    P = np.where((i >= i.T)[None, None, :, :, None], P, 0.0)
    cross = P.sum(axis=2)
    if st is not None:
        cross = cross + _suffix(st * pq)
    mag = sq * pq + sk * pk
    floor = np.zeros_like(mag)
    for c0 in range(0, n, 64):
        c1 = min(n, c0 + 64)
        floor[:, :, c0:c1] = _suffix(mag[:, :, c0:c1]) + (cross[:, :, c1:c1 + 1] if c1 < n else 0.0)
    sdg = (cross + floor * 2.0 ** -8) / (1.0 + np.exp(g)) / tau
    # d log beta: the crossing pairs (i >= u > j) and the carried state's terms, per column
    Mv = gg[:, :, :, None, :] * W[..., None] * aV[:, :, None, :, :] * Dv          # [b, h, i, j, e]
    Pv = np.cumsum(Mv, axis=3) - Mv
    Pv = np.where((i >= i.T)[None, None, :, :, None], Pv, 0.0)
    crossv = Pv.sum(axis=2)
    numabs = np.einsum("bhij,bhije,bhje->bhie", W, Dv, aV)
    if S0 is not None:
        sts = gg * cb * ((pq * ca) @ np.abs(S0))
        crossv = crossv + _suffix(sts)
        numabs = numabs + cb * ((pq * ca) @ np.abs(S0))
    magv = gg * numabs + sv * aV
    sdgv = (crossv + _suffix(magv) * 2.0 ** -8) / (1.0 + np.exp(gv)) / tau
    if not norm:
        return sq, sk, sv, sdg, sdgv
    dphi = lambda x: np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    return sq * dphi(Q), sk * dphi(K), sv, sdg, sdgv


def run_backward_outer(inp, dO, S0=None, z0=None, fmap="elu1"):
    import kernelized_sequence_mixing_amd as ksm
    res = ksm.backward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(dO), fmap=fmap, gate=gpu_gate(inp),
                       eps=inp["eps"], S0=dev(S0), z0=dev(z0))
    torch.cuda.synchronize()
    assert len(res) == 5
    return tuple(x.cpu() for x in res)


NAMES = ("dQ", "dK", "dV", "dg", "dgv")


def check_heads(got, inp, dO, heads, what, S0=None, z0=None, fmap="elu1"):
    for head in heads:
        b, h = head
        Q, K, V, d, g, gv, s0, z = _head(inp, dO, head, S0, z0)
        ref = obwd.backward_outer(Q, K, V, d, g, gv, inp["tau"], fmap, None, inp["eps"], s0, z)
        scales = outer_scales(Q, K, V, d, g, gv, inp["tau"], inp["eps"], s0, z, fmap)
        errs, hm = [], []
        for x, r, sc in zip(got, ref, scales):
            xg = to_f64(x[b:b + 1, h:h + 1])
            assert np.isfinite(xg).all()
            errs.append(float(np.max(np.abs(xg - r) / (sc + 1e-30))))
            hm.append(float(np.max(np.abs(xg - r)) / (np.max(np.abs(r)) + 1e-30)))
        print(f"  {what} head {head}: term-relative " + " ".join(f"{nm} {e:.2e}" for nm, e in zip(NAMES, errs)) +
              "; of the head max " + " ".join(f"{nm} {e:.2e}" for nm, e in zip(NAMES, hm)), flush=True)
        for nm, e in zip(NAMES, errs):
            assert e < TOL_GRAD, (what, head, nm, e)


def _case(d, dv, B, H, n, seed=3):
    wl = WORKLOADS["outer_gate"].resized(d_k=d, d_v=dv, r=d, qk_scale=d ** -0.5, v_scale=d ** -0.5)
    inp = make_inputs(wl, seed=seed, B=B, H=H, n=n)
    dO = incoming_gradient((B, H, n, dv), seed + 100)
    return wl, inp, dO


CASES = [(64, 64, 2, 4, 777), (64, 64, 4, 16, 1285), (128, 64, 2, 4, 300), (64, 128, 2, 4, 300),
         (64, 64, 1, 1, 1), (64, 64, 2, 1, 65), (128, 128, 2, 4, 300)]


@pytest.mark.parametrize("d,dv,B,H,n", CASES)
def test_backward_outer_parity(d, dv, B, H, n):
    """Several segments with a ragged tail, one chunk, tiny n, every built
    (d_k, d_v); 128 x 128 runs as two value-column halves (each with its own
    columns of gv and dgv)."""
    wl, inp, dO = _case(d, dv, B, H, n)
    got = run_backward_outer(inp, dO)
    check_heads(got, inp, dO, [(0, 0), (B - 1, H - 1)], f"outer d{d} dv{dv} B{B} H{H} n{n}")


@pytest.mark.parametrize("d", [64, 128])
def test_backward_outer_carried_state(d):
    """A carried-in state; at 128 x 128 each value-column half takes its own
    columns of S0 (z0 is shared)."""
    wl, inp, dO = _case(d, d, 2, 4, 400, seed=5)
    rng = np.random.default_rng(81)
    S0 = torch.from_numpy((rng.standard_normal((2, 4, d, d)) * 2.0).astype(np.float32))
    z0 = torch.from_numpy((20.0 + 2.0 * np.abs(rng.standard_normal((2, 4, d)))).astype(np.float32))
    got = run_backward_outer(inp, dO, S0, z0)
    check_heads(got, inp, dO, [(0, 0), (1, 3)], f"outer carried state d{d}", S0, z0)


def test_backward_outer_state_space():
    """Identity features with the unnormalised read-out (h = 0)."""
    wl = WORKLOADS["outer_gate"].resized(d_k=64, d_v=64, r=64, fmap="identity", qk_scale=0.125, v_scale=0.125)
    inp = make_inputs(wl, seed=7, B=2, H=2, n=500)
    dO = incoming_gradient((2, 2, 500, 64), 107)
    got = run_backward_outer(inp, dO, fmap="identity")
    check_heads(got, inp, dO, [(0, 0), (1, 1)], "outer state-space", fmap="identity")


@pytest.mark.parametrize("side", ["key", "value"])
def test_backward_outer_at_the_domain_edge(side):
    """A summed log-gate of about -75 per 64-token chunk on one side, every
    other chunk (crossing chunk and segment boundaries): the backward passes
    reuse the forward's chunk-start factors on both sides."""
    wl, inp, dO = _case(64, 64, 2, 4, 700, seed=9)
    if side == "key":
        inp["g"] = strong_gate_input((2, 4, 700, 64), 70)
    else:
        inp["gv"] = strong_gate_input((2, 4, 700, 64), 71)
    got = run_backward_outer(inp, dO)
    check_heads(got, inp, dO, [(0, 0), (1, 3)], f"outer backward edge ({side})")


def test_backward_outer_workload_full_size_tail():
    """The outer-product gate's workload (B2 H16 n16384 d_k = d_v = 128: two
    value-column halves, several segments) in one la_backward call. Every
    gradient of a token depends only on that token, the later ones and the
    forward state entering it, so on two sampled heads the last 320 tokens'
    gradients are checked against the oracle run on those tokens from the
    state the recurrent oracle carries into them; every entry is finite."""
    wl = WORKLOADS["outer_gate"]
    inp = make_inputs(wl, seed=0)
    dO = incoming_gradient((wl.B, wl.H, wl.n, wl.d_v), 1)
    print(f"  outer backward at B={wl.B} H={wl.H} n={wl.n} d_k={wl.d_k} d_v={wl.d_v}", flush=True)
    got = run_backward_outer(inp, dO)
    for x in got:
        assert torch.isfinite(x).all()
    m = 320
    n0 = wl.n - m
    for b, h in [(0, 0), (wl.B - 1, wl.H - 1)]:
        sl = lambda x: to_f64(x[b:b + 1, h:h + 1])
        Q, K, V, d, g, gv = (sl(inp["Q"]), sl(inp["K"]), sl(inp["V"]), sl(dO), sl(inp["g"]), sl(inp["gv"]))
        pre = lambda x: x[:, :, :n0]
        _, S0, z0 = causal_recurrent(pre(Q), pre(K), pre(V), "elu1", None, ("outer", pre(g), pre(gv), inp["tau"]),
                                     inp["eps"])
        tail = lambda x: x[:, :, n0:]
        args = (tail(Q), tail(K), tail(V), tail(d), tail(g), tail(gv), inp["tau"])
        ref = obwd.backward_outer(*args, "elu1", None, inp["eps"], S0, z0)
        scales = outer_scales(*args, inp["eps"], S0, z0)
        errs = []
        for x, r, sc in zip(got, ref, scales):
            xg = to_f64(x[b:b + 1, h:h + 1, n0:])
            errs.append(float(np.max(np.abs(xg - r) / (sc + 1e-30))))
        print(f"  full-size head ({b}, {h}), last {m} tokens: term-relative " +
              " ".join(f"{nm} {e:.2e}" for nm, e in zip(NAMES, errs)), flush=True)
        for nm, e in zip(NAMES, errs):
            assert e < TOL_GRAD, ("full size", (b, h), nm, e)


def test_backward_outer_deterministic():
    wl, inp, dO = _case(64, 64, 2, 4, 777, seed=6)
    a, b = run_backward_outer(inp, dO), run_backward_outer(inp, dO)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
