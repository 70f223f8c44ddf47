"""Causal d_v = 32 against the fp64 oracle: la_forward runs the 64-column
chunk kernels on zero-padded copies of V (and gv) in its workspace and copies
the 32 real columns of the output and the final state back. Every feature map
and gate, several segments with a ragged tail, tiny n, a carried-in state, the
final state, and la_forward_noalloc."""
import numpy as np
import pytest
import torch

from workloads import WORKLOADS, make_inputs, to_f64
from _helpers import TOL_BF16, check_close, dev, gpu_gate, oracle_forward, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _wl(name, d):
    wl = WORKLOADS[name].resized(d_v=32)
    if wl.fmap != "favor":
        wl = wl.resized(d_k=d, r=d, qk_scale=d ** -0.5, v_scale=32 ** -0.5)
    return wl


CASES = [("causal_elu1", 64, 4, 16, 1285), ("causal_elu1", 32, 1, 2, 200), ("retnet_decay", 128, 2, 8, 1285),
         ("gla_gate", 64, 2, 8, 1285), ("gla_gate", 128, 1, 1, 65), ("favor_causal", 64, 2, 2, 777),
         ("outer_gate", 64, 2, 4, 777), ("ssm_selective", 64, 2, 4, 777), ("causal_elu1", 64, 1, 1, 1)]


@pytest.mark.parametrize("name,d,B,H,n", CASES)
def test_dv32_parity(name, d, B, H, n):
    inp = make_inputs(_wl(name, d), seed=2, B=B, H=H, n=n)
    out, S, z = run_forward(inp, return_state=True)
    assert out.shape[-1] == 32 and S.shape[-1] == 32
    ref, Sr, zr = oracle_forward(inp)
    # bit for bit the first 32 columns of the same problem at d_v = 64 with V (and gv) zero-padded
    pad = dict(inp)
    for key in ("V", "gv"):
        if isinstance(inp.get(key), torch.Tensor):
            x = inp[key]
            pad[key] = torch.cat([x, torch.zeros_like(x)], dim=-1).contiguous()
    out64, S64, z64 = run_forward(pad, return_state=True)
    assert torch.equal(out, out64[..., :32]) and torch.equal(S, S64[..., :32]) and torch.equal(z, z64)
    if inp["fmap"] == "identity":  # the state-space read-out is checked term-relative in its own file
        return
    check_close(out, ref, TOL_BF16, f"{name} d{d} d_v 32 B{B} H{H} n{n}")
    scale = np.max(np.abs(Sr)) + 1e-30
    assert np.max(np.abs(to_f64(S) - Sr)) / scale < 2e-2
    np.testing.assert_allclose(to_f64(z), zr, rtol=2e-2)


@pytest.mark.parametrize("name", ["causal_elu1", "gla_gate"])
def test_dv32_carried_state(name):
    """Resume from a carried-in state [B H r 32]: equals the oracle run from it."""
    inp = make_inputs(_wl(name, 64), seed=4, B=2, H=4, n=900)
    rng = np.random.default_rng(17)
    S0 = torch.from_numpy((rng.standard_normal((2, 4, 64, 32)) * 2.0).astype(np.float32))
    z0 = torch.from_numpy((20.0 + 2.0 * np.abs(rng.standard_normal((2, 4, 64)))).astype(np.float32))
    out, S, z = run_forward(inp, return_state=True, S0=S0, z0=z0)
    ref, Sr, zr = oracle_forward(inp, S0=to_f64(S0), z0=to_f64(z0))
    check_close(out, ref, TOL_BF16, f"{name} d_v 32 carried state")
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 2e-2


def test_dv32_noalloc_bit_equal():
    """The allocation-free entry point (its scratch array holds the padded copies too)."""
    import kernelized_sequence_mixing_amd as ksm
    inp = make_inputs(_wl("gla_gate", 64), seed=6, B=2, H=8, n=2000)
    Q, K, V = dev(inp["Q"]), dev(inp["K"]), dev(inp["V"])
    gate = gpu_gate(inp)
    ref, Sr, zr = ksm.forward(Q, K, V, gate=gate, eps=inp["eps"], return_state=True)
    out = torch.full_like(ref, float("nan"))
    S = torch.full_like(Sr, float("nan"))
    z = torch.full_like(zr, float("nan"))
    ksm.forward_noalloc(Q, K, V, gate=gate, eps=inp["eps"], out=out, S_final=S, z_final=z)
    torch.cuda.synchronize()
    for a, b, nm in ((ref, out, "out"), (Sr, S, "S"), (zr, z, "z")):
        assert torch.equal(a.cpu(), b.cpu()), nm
