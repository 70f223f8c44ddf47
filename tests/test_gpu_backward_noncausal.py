"""GPU parity of the non-causal backward pass (elu+1, fp32 vector-ALU kernels)
against the fp64 gradient oracle (oracle.la_backward.backward with causal=False,
pinned by finite differences of the non-causal forward oracle).

The gradients are computed in fp32 throughout, so with fp32 inputs the bound is
the fp32 paths' 1e-4; with bf16 inputs and outputs the bf16 rounding of the
outputs sets it, 1e-2. Each entry's error is taken relative to the magnitude
sum of the terms it sums (dq_i sums (g_i . v_j + h_i) phi(k_j) over all j,
which cancel: the output does not change with the scale of phi(q_i) but for
eps, so dq can be far smaller than its terms, e.g. exactly ~0 for n = 1).
"""
import numpy as np
import pytest
import torch

from oracle import la_backward as obwd
from workloads import WORKLOADS, make_inputs, to_f64, incoming_gradient
from _helpers import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


CASES = [("f32", 32, 32, 1, 1, 256), ("f32", 64, 128, 2, 4, 1000), ("f32", 128, 64, 1, 2, 77),
         ("f32", 32, 64, 2, 1, 1), ("bf16", 64, 64, 2, 3, 513), ("bf16", 128, 128, 1, 2, 300)]


@pytest.mark.parametrize("dt,d,dv,B,H,n", CASES)
def test_noncausal_backward_parity(dt, d, dv, B, H, n):
    """The non-causal workload's shape (B1 H1 n256 d32 fp32), several splits
    with ragged tails, n = 1, each dtype and built width."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["noncausal_elu1_f32"].resized(d_k=d, d_v=dv, r=d, dtype=dt, qk_scale=d ** -0.5,
                                               v_scale=dv ** -0.5)
    inp = make_inputs(wl, seed=11, B=B, H=H, n=n)
    dO = incoming_gradient((B, H, n, dv), 12, dtype=dt)
    got = ksm.backward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(dO), causal=False, eps=wl.eps)
    torch.cuda.synchronize()
    ref = obwd.backward(to_f64(inp["Q"]), to_f64(inp["K"]), to_f64(inp["V"]), to_f64(dO), "elu1", None, False,
                        None, wl.eps)
    tol = 1e-4 if dt == "f32" else 1e-2
    pq, pk, _, _, W, _, den, o = obwd.forward_terms(to_f64(inp["Q"]), to_f64(inp["K"]), to_f64(inp["V"]), "elu1",
                                                    None, False, None, wl.eps)
    dd, V = to_f64(dO), np.abs(to_f64(inp["V"]))
    ag = np.abs(dd) / den[..., None]
    ah = np.abs(np.sum(dd * o, axis=-1)) / den
    T = ag @ np.swapaxes(V, -1, -2) + ah[..., None]                        # |terms| of dW_ij
    dphi = lambda phi: np.minimum(phi, 1.0)
    scales = (np.einsum("bhij,bhjr->bhir", T, pk) * dphi(pq), np.einsum("bhij,bhir->bhjr", T, pq) * dphi(pk),
              np.einsum("bhij,bhie->bhje", np.abs(W), ag))
    for nm, x, r, sc in zip(("dQ", "dK", "dV"), got, ref, scales):
        assert x.dtype == inp["Q"].dtype
        e = float(np.max(np.abs(to_f64(x.cpu()) - r) / (sc + 1e-30)))
        print(f"  noncausal {dt} d{d}x{dv} B{B} H{H} n{n}: {nm} term-relative err {e:.2e}", flush=True)
        assert e < tol, (nm, e)


def test_noncausal_backward_deterministic():
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["noncausal_elu1_f32"].resized(d_k=64, d_v=64, r=64)
    inp = make_inputs(wl, seed=3, B=2, H=4, n=3000)
    dO = incoming_gradient((2, 4, 3000, 64), 4, dtype="f32")
    a = ksm.backward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(dO), causal=False)
    b = ksm.backward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), dev(dO), causal=False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
