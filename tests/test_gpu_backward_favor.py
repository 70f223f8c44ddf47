"""GPU parity of the FAVOR+ backward pass (la_backward with the FAVOR+ feature
map) against the fp64 gradient oracle (oracle.la_backward.backward, whose
feature-map step is pinned by finite differences).

The library materialises phi(Q), phi(K) in bf16, runs the chunked backward on
them as precomputed features, and takes d phi back through the map:
dx = sum_m dphi_m phi_m (w_m - x). The metric is term-relative as for the
other feature maps: each entry's error over the magnitude sum of its terms,
here sum_m s_m phi_m (|w_m| + |x|) with s_m the magnitude sum behind dphi_m.
Each term then carries the elementwise backward's roundings plus the bf16
feature and d phi, about six 2^-9; the tolerance is 2e-2 as for the others.
"""
import numpy as np
import pytest
import torch

from oracle import la_backward as obwd
from oracle.la_oracle import feature_map
from workloads import WORKLOADS, make_inputs, to_f64, incoming_gradient
from _helpers import dev, gpu_gate, oracle_gate

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _case(d, r, dv, B, H, n, gate="none", seed=3):
    wl = WORKLOADS["favor_causal"].resized(d_k=d, r=r, d_v=dv, gate=gate, qk_scale=d ** -0.25, v_scale=1.0)
    inp = make_inputs(wl, seed=seed, B=B, H=H, n=n)
    dO = incoming_gradient((B, H, n, dv), seed + 100)
    return wl, inp, dO


def _scales(inp, dO, S0=None, z0=None):
    """Magnitude sums of the terms behind dQ, dK (through the feature map) and dV."""
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    om = to_f64(inp["omega"])
    d = to_f64(dO)
    gate = oracle_gate(inp)
    pq, pk, D, c, W, num, den, o = obwd.forward_terms(Q, K, V, "favor", om, True, gate, inp["eps"],
                                                      None if S0 is None else to_f64(S0),
                                                      None if z0 is None else to_f64(z0))
    g = d / den[..., None]
    hh = -np.sum(d * o, axis=-1) / den
    T = (np.einsum("bhie,bhje->bhij", np.abs(g), np.abs(V)) + np.abs(hh)[..., None]) * D[None]
    sq = np.einsum("bhij,bhjf->bhif", T, pk)
    if S0 is not None:
        sq = sq + c[None, :, :, None] * (np.einsum("bhre,bhie->bhir", np.abs(to_f64(S0)), np.abs(g)) +
                                         np.abs(hh)[..., None] * np.abs(to_f64(z0))[:, :, None, :])
    sk = np.einsum("bhij,bhif->bhjf", T, pq)
    sv = np.einsum("bhij,bhie->bhje", W, np.abs(g))

    def through(x, s, ph):  # sum_m s_m phi_m (|w_m| + |x|)
        u = s * ph
        return np.einsum("bhnm,md->bhnd", u, np.abs(om)) + np.abs(x) * u.sum(axis=-1, keepdims=True)
    return through(Q, sq, pq), through(K, sk, pk), sv


def _run(inp, dO, S0=None, z0=None):
    import kernelized_sequence_mixing_amd as ksm
    res = ksm.backward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(dO), fmap="favor", omega=dev(inp["omega"]),
                       gate=gpu_gate(inp), eps=inp["eps"], S0=dev(S0), z0=dev(z0))
    torch.cuda.synchronize()
    return tuple(x.cpu() for x in res)


def _check(got, inp, dO, what, S0=None, z0=None):
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    ref = obwd.backward(Q, K, V, to_f64(dO), "favor", to_f64(inp["omega"]), True, oracle_gate(inp), inp["eps"],
                        None if S0 is None else to_f64(S0), None if z0 is None else to_f64(z0))
    scales = _scales(inp, dO, S0, z0)
    errs = []
    for x, r_, sc in zip(got, ref, scales):
        xg = to_f64(x)
        assert np.isfinite(xg).all()
        errs.append(float(np.max(np.abs(xg - r_) / (sc + 1e-30))))
    head = [float(np.max(np.abs(to_f64(x) - r_)) / np.max(np.abs(r_))) for x, r_ in zip(got, ref)]
    print(f"  {what}: term-relative dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}; of the largest entry "
          f"dQ {head[0]:.2e} dK {head[1]:.2e} dV {head[2]:.2e}", flush=True)
    for nm, e in zip(("dQ", "dK", "dV"), errs):
        assert e < TOL_GRAD, (what, nm, e)


CASES = [(64, 128, 64, 2, 4, 777, "none"), (64, 64, 64, 2, 4, 300, "none"), (32, 64, 128, 2, 2, 300, "none"),
         (128, 128, 128, 2, 2, 300, "none"), (64, 128, 64, 2, 4, 500, "decay"), (64, 128, 64, 2, 1, 65, "none"),
         (64, 128, 64, 1, 1, 1, "none")]


@pytest.mark.parametrize("d,r,dv,B,H,n,gate", CASES)
def test_backward_favor_parity(d, r, dv, B, H, n, gate):
    """Several segments with a ragged tail, one segment, tiny n, every built
    (r, d_v) with d_k 32 to 128, the RetNet decay; 128 x 128 runs as two
    value-column halves."""
    wl, inp, dO = _case(d, r, dv, B, H, n, gate)
    got = _run(inp, dO)
    _check(got, inp, dO, f"favor d{d} r{r} dv{dv} B{B} H{H} n{n} {gate}")


def test_backward_favor_carried_state():
    wl, inp, dO = _case(64, 128, 64, 2, 4, 400, seed=5)
    rng = np.random.default_rng(79)
    S0 = torch.from_numpy((rng.standard_normal((2, 4, 128, 64)) * 2.0).astype(np.float32))
    z0 = torch.from_numpy((20.0 + 2.0 * np.abs(rng.standard_normal((2, 4, 128)))).astype(np.float32))
    got = _run(inp, dO, S0, z0)
    _check(got, inp, dO, "favor carried state", S0, z0)


def test_backward_favor_deterministic():
    wl, inp, dO = _case(64, 128, 64, 2, 4, 777, seed=6)
    a, b = _run(inp, dO), _run(inp, dO)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
