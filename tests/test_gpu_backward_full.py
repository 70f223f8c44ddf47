"""Full-size parity of the gated backward pass, in the launch configurations
the benchmark times (B2 H16 n16384 at d64 and at the GLA workload's own
d128, which runs as two value-column halves): sampled gradient entries of two heads
against the fp64 oracle's per-row form (oracle.la_backward.backward_gla_rows,
pinned against the explicit form), for the GLA gate with elu+1, and the
state-space form under the GLA and the selective scalar gate.

Rows 0, 1, n/2 and n-1 of dQ, dK, dV, and dg over the last chunk (the
suffix sums there run over the whole chunk). The metric is the term-relative
one of test_gpu_backward_gla.py: each entry's error over the magnitude sum
of the terms it sums (computed here with the same per-row loops on
magnitudes); for dg the crossing pairs' magnitudes plus the 2^-8 floor of the
in-chunk suffix.
"""
import numpy as np
import pytest
import torch

from oracle import la_backward as obwd
from oracle.la_oracle import feature_map
from workloads import WORKLOADS, make_inputs, to_f64, incoming_gradient
from _helpers import dev

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def sampled_scales(Q, K, V, dO, G, tau, fmap, den, o, rows, tail):
    """Magnitude sums of the terms behind dQ, dK, dV at `rows` and dg over the
    last `tail` steps (one head, no carried state)."""
    pq, pk = np.abs(feature_map(Q, fmap)), np.abs(feature_map(K, fmap))
    n = Q.shape[0]
    la = -np.logaddexp(0.0, -G) / tau
    Bc = np.cumsum(la, axis=0)
    norm = fmap != "identity"
    gg = np.abs(dO) / den[:, None]
    hh = np.abs(np.sum(dO * o, axis=1)) / den if norm else np.zeros(n)
    aV = np.abs(V)
    dphi = (lambda x: np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))) if norm else (lambda x: np.ones_like(x))

    def sq(i):
        D = np.exp(Bc[i] - Bc[:i + 1])
        return ((aV[:i + 1] @ gg[i] + hh[i])[:, None] * pk[:i + 1] * D).sum(axis=0)

    def sk(j):
        D = np.exp(Bc[j:] - Bc[j])
        return ((gg[j:] @ aV[j] + hh[j:])[:, None] * pq[j:] * D).sum(axis=0), ((pq[j:] * D) @ pk[j]) @ gg[j:]

    s_q = np.array([sq(i) * dphi(Q[i]) for i in rows])
    s_k = np.array([sk(j)[0] * dphi(K[j]) for j in rows])
    s_v = np.array([sk(j)[1] for j in rows])
    u0 = n - tail
    cross = np.zeros((tail, pq.shape[1]))
    for i in range(u0, n):
        D = np.exp(Bc[i] - Bc[:i + 1])
        M = (aV[:i + 1] @ gg[i] + hh[i])[:, None] * pk[:i + 1] * D     # terms of pairs (i, j <= i)
        C = np.cumsum(M, axis=0) - M                                      # sum over j < u, at row u
        cross[:i - u0 + 1] += pq[i] * C[u0:i + 1]
    mag = np.array([sq(t) * pq[t] + sk(t)[0] * pk[t] for t in range(u0, n)])
    floor = np.flip(np.cumsum(np.flip(mag, axis=0), axis=0), axis=0) * 2.0 ** -8
    s_g = (cross + floor) / (1.0 + np.exp(G[u0:])) / tau
    return s_q, s_k, s_v, s_g


CASES = [("gla_gate_d64", "elu1", "gla"), ("ssm_selective", "identity", "gla"), ("ssm_scalar", "identity", "sel"),
         ("gla_gate", "elu1", "gla")]


@pytest.mark.parametrize("name,fmap,gate", CASES)
def test_backward_full_size_sampled(name, fmap, gate):
    import kernelized_sequence_mixing_amd as ksm
    if name == "gla_gate_d64":
        wl = WORKLOADS["gla_gate"].resized(name="gla_gate_d64", d_k=64, d_v=64, r=64, qk_scale=64 ** -0.5,
                                          v_scale=64 ** -0.5)
    else:
        wl = WORKLOADS[name]
    inp = make_inputs(wl, seed=0)
    dO = incoming_gradient((wl.B, wl.H, wl.n, wl.d_v), 1)
    res = ksm.backward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(dO), fmap=fmap,
                       gate=(gate, dev(inp["g"]), wl.tau), eps=wl.eps)
    torch.cuda.synchronize()
    got = tuple(x.cpu() for x in res)
    n, tail = wl.n, 64
    rows = [0, 1, n // 2, n - 1]
    for b, h in [(0, 0), (wl.B - 1, wl.H - 1)]:
        Q, K, V, d = (to_f64(x)[b, h] for x in (inp["Q"], inp["K"], inp["V"], dO))
        g = to_f64(inp["g"])[b, h]
        G = g if gate == "gla" else np.repeat(g[:, None], Q.shape[1], axis=1)
        ref = obwd.backward_gla_rows(Q, K, V, d, G, wl.tau, fmap, wl.eps, rows=rows, tail=tail, return_forward=True)
        den, o = ref[4], ref[5]
        ref = ref[:4] if gate == "gla" else obwd.backward_sel_rows(Q, K, V, d, g, wl.tau, fmap, wl.eps, rows, tail)
        s_q, s_k, s_v, s_g = sampled_scales(Q, K, V, d, G, wl.tau, fmap, den, o, rows, tail)
        if gate == "sel":
            s_g = s_g.sum(axis=1)
        errs = []
        for x, r_, sc, sel in zip(got, ref, (s_q, s_k, s_v, s_g), (rows, rows, rows, slice(n - tail, n))):
            xg = to_f64(x[b, h])[sel]
            assert np.isfinite(xg).all()
            errs.append(float(np.max(np.abs(xg - r_) / (sc + 1e-30))))
        print(f"  {name} backward full size head {(b, h)}: term-relative dQ {errs[0]:.2e} dK {errs[1]:.2e} "
              f"dV {errs[2]:.2e} dg {errs[3]:.2e}", flush=True)
        for nm, e in zip(("dQ", "dK", "dV", "dg"), errs):
            assert e < TOL_GRAD, (name, (b, h), nm, e)
