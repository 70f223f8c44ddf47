"""GPU parity of the backward pass of the state-space form (identity
features, unnormalised read-out y = C^T h: g = dO, h = 0, phi' = 1) against
the fp64 gradient oracle, under no gate, the RetNet decay and the GLA gate
(with the gate's gradient dg). The metrics are those of test_gpu_backward.py
and test_gpu_backward_gla.py, with the features taken in magnitude.
"""
import numpy as np
import pytest
import torch

from workloads import WORKLOADS, make_inputs, incoming_gradient
import test_gpu_backward as tb
import test_gpu_backward_gla as tg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _case(gate, d, dv, B, H, n, seed=3):
    wl = WORKLOADS["ssm_selective"].resized(d_k=d, d_v=dv, r=d, gate=gate, qk_scale=d ** -0.5)
    inp = make_inputs(wl, seed=seed, B=B, H=H, n=n)
    dO = incoming_gradient((B, H, n, dv), seed + 100)
    return wl, inp, dO


CASES = [(g, d, dv, B, H, n) for g in ("none", "decay")
         for (d, dv, B, H, n) in ((64, 64, 2, 4, 777), (64, 128, 2, 4, 300), (128, 64, 2, 4, 300),
                                  (64, 64, 4, 16, 1285), (64, 64, 2, 1, 65), (128, 128, 2, 4, 777))]


@pytest.mark.parametrize("gate,d,dv,B,H,n", CASES)
def test_ssm_backward_parity(gate, d, dv, B, H, n):
    wl, inp, dO = _case(gate, d, dv, B, H, n)
    got = tb.run_backward(inp, dO, fmap="identity")
    ref = tb.oracle_backward(inp, dO, fmap="identity")
    tb.check_grads(got, ref, tb.term_scales(inp, dO, fmap="identity"), f"ssm {gate} d{d}x{dv} B{B} H{H} n{n}")


def test_ssm_backward_carried_state():
    wl, inp, dO = _case("decay", 64, 64, 4, 16, 700, seed=9)
    rng = np.random.default_rng(77)
    S0 = torch.from_numpy(rng.standard_normal((4, 16, 64, 64)).astype(np.float32))
    z0 = torch.from_numpy((1.0 + rng.random((4, 16, 64))).astype(np.float32))
    got = tb.run_backward(inp, dO, S0, z0, fmap="identity")
    ref = tb.oracle_backward(inp, dO, S0, z0, fmap="identity")
    tb.check_grads(got, ref, tb.term_scales(inp, dO, S0, z0, fmap="identity"), "ssm carried state")


GLA_CASES = [(64, 64, 2, 4, 777), (64, 64, 4, 16, 1285), (128, 64, 2, 4, 300), (64, 128, 2, 4, 300),
             (64, 64, 2, 1, 65), (128, 128, 2, 4, 300)]


@pytest.mark.parametrize("d,dv,B,H,n", GLA_CASES)
def test_ssm_backward_gla_parity(d, dv, B, H, n):
    """The selective recurrence with the per-feature gate: dQ, dK, dV and dg."""
    wl, inp, dO = _case("gla", d, dv, B, H, n)
    got = tg.run_backward_gla(inp, dO, fmap="identity")
    heads = sorted({(0, 0), (B - 1, H - 1)} | ({(B // 2, H // 2)} if n < 1000 else set()))
    tg.check_heads(got, inp, dO, heads, f"ssm gla d{d}x{dv} B{B} H{H} n{n}", fmap="identity")


def test_ssm_backward_gla_carried_state():
    wl, inp, dO = _case("gla", 64, 64, 4, 16, 700, seed=9)
    rng = np.random.default_rng(78)
    S0 = torch.from_numpy(rng.standard_normal((4, 16, 64, 64)).astype(np.float32))
    z0 = torch.from_numpy((1.0 + rng.random((4, 16, 64))).astype(np.float32))
    got = tg.run_backward_gla(inp, dO, S0, z0, fmap="identity")
    tg.check_heads(got, inp, dO, [(0, 0), (3, 15)], "ssm gla carried state", S0, z0, fmap="identity")
