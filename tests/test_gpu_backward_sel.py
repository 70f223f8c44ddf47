"""GPU parity of the causal backward pass under the selective scalar gate (one
decay a_t = sigmoid(g_t)^(1/tau) per step and head, g [B, H, n]) against the
fp64 gradient oracle (oracle.la_backward.backward_sel), for elu+1 and the
state-space form's identity features.

The metric is the term-relative one of test_gpu_backward_gla.py: the gate is
the diagonal gate with the same alpha on every feature, so the scales of dQ,
dK, dV are gla_scales' for g repeated over features, and dg_t, the sum of the
per-feature gate gradients, gets the sum of their scales.
"""
import numpy as np
import pytest
import torch

from oracle import la_backward as obwd
from workloads import WORKLOADS, make_inputs, to_f64, incoming_gradient
from _helpers import dev
import test_gpu_backward_gla as tg

pytestmark = pytest.mark.gpu

TOL_GRAD = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _case(fmap, d, dv, B, H, n, seed=5):
    if fmap == "identity":
        wl = WORKLOADS["ssm_scalar"].resized(d_k=d, d_v=dv, r=d, qk_scale=d ** -0.5)
    else:
        wl = WORKLOADS["gla_gate"].resized(d_k=d, d_v=dv, r=d, gate="sel")
    inp = make_inputs(wl, seed=seed, B=B, H=H, n=n)
    assert tuple(inp["g"].shape) == (B, H, n)
    dO = incoming_gradient((B, H, n, dv), seed + 100)
    return wl, inp, dO


def run(inp, dO, fmap, S0=None, z0=None):
    import kernelized_sequence_mixing_amd as ksm
    res = ksm.backward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(dO), fmap=fmap,
                       gate=("sel", dev(inp["g"]), inp["tau"]), eps=inp["eps"], S0=dev(S0), z0=dev(z0))
    torch.cuda.synchronize()
    assert len(res) == 4 and tuple(res[3].shape) == tuple(inp["g"].shape)
    return tuple(x.cpu() for x in res)


def check_heads(got, inp, dO, heads, what, fmap, S0=None, z0=None):
    for b, h in heads:
        sl = lambda x: None if x is None else to_f64(x)[b:b + 1, h:h + 1]
        Q, K, V, d, g, s0, z = sl(inp["Q"]), sl(inp["K"]), sl(inp["V"]), sl(dO), sl(inp["g"]), sl(S0), sl(z0)
        ref = obwd.backward_sel(Q, K, V, d, g, inp["tau"], fmap, None, inp["eps"], s0, z)
        r = Q.shape[-1]
        sq, sk, sv, sdg = tg.gla_scales(Q, K, V, d, np.repeat(g[..., None], r, axis=-1), inp["tau"], inp["eps"],
                                        s0, z, fmap)
        errs = []
        for x, rf, sc in zip(got, ref, (sq, sk, sv, sdg.sum(axis=-1))):
            xg = to_f64(x[b:b + 1, h:h + 1])
            assert np.isfinite(xg).all()
            errs.append(float(np.max(np.abs(xg - rf) / (sc + 1e-30))))
        dgh = float(np.max(np.abs(to_f64(got[3][b:b + 1, h:h + 1]) - ref[3])) / (np.max(np.abs(ref[3])) + 1e-30))
        print(f"  {what} head {(b, h)}: term-relative dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e} "
              f"dg {errs[3]:.2e}; dg of the head max {dgh:.2e}", flush=True)
        for nm, e in zip(("dQ", "dK", "dV", "dg"), errs):
            assert e < TOL_GRAD, (what, (b, h), nm, e)


CASES = [(f, d, dv, B, H, n) for f in ("elu1", "identity")
         for (d, dv, B, H, n) in ((64, 64, 2, 4, 777), (64, 64, 2, 4, 1285), (128, 64, 2, 2, 300),
                                  (64, 128, 2, 2, 300), (64, 64, 2, 1, 65), (128, 128, 2, 2, 300))]


@pytest.mark.parametrize("fmap,d,dv,B,H,n", CASES)
def test_backward_sel_parity(fmap, d, dv, B, H, n):
    """One-chunk and three-chunk segments with ragged tails, one segment, n 65,
    each built shape, both elementwise feature maps."""
    wl, inp, dO = _case(fmap, d, dv, B, H, n)
    got = run(inp, dO, fmap)
    heads = sorted({(0, 0), (B - 1, H - 1)})
    check_heads(got, inp, dO, heads, f"sel {fmap} d{d}x{dv} B{B} H{H} n{n}", fmap)


def test_backward_sel_with_carried_state():
    wl, inp, dO = _case("elu1", 64, 64, 2, 4, 700, seed=9)
    rng = np.random.default_rng(79)
    S0 = torch.from_numpy((rng.standard_normal((2, 4, 64, 64)) * 2.0).astype(np.float32))
    z0 = torch.from_numpy((20.0 + 2.0 * np.abs(rng.standard_normal((2, 4, 64)))).astype(np.float32))
    got = run(inp, dO, "elu1", S0, z0)
    check_heads(got, inp, dO, [(0, 0), (1, 3)], "sel carried state", "elu1", S0, z0)


def test_backward_sel_deterministic():
    wl, inp, dO = _case("elu1", 64, 64, 2, 8, 1285, seed=4)
    a = run(inp, dO, "elu1")
    b = run(inp, dO, "elu1")
    for x, y in zip(a, b):
        assert torch.equal(x, y)
