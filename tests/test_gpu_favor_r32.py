"""FAVOR+ with r = 32 random features on every path, against the fp64 oracle.

The vector-ALU paths (non-causal, decode step, feature map) take r = 32
directly; the causal chunk kernels work in 64-feature blocks, so la_forward
runs them on omega zero-padded to 64 rows with the features past 32 masked to
zero (and the 1/sqrt(r) of the map at r = 32), the states padded alike: the
result equals the r = 32 map's. Also with d_v = 32 (both paddings at once), the
RetNet decay, a carried-in and a final state, and against an r = 64 map whose
extra features are cancelled exactly (not expressible): instead, against the
oracle only."""
import numpy as np
import pytest
import torch

import oracle as orc
from workloads import WORKLOADS, make_inputs, to_f64
from _helpers import TOL_BF16, TOL_F32, check_close, dev, gpu_gate, oracle_forward, run_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


@pytest.mark.parametrize("d,dv,B,H,n,gate", [(64, 64, 2, 4, 1285, "none"), (32, 128, 1, 2, 777, "none"),
                                             (128, 64, 2, 2, 300, "none"), (64, 32, 2, 4, 777, "none"),
                                             (64, 64, 2, 4, 777, "decay"), (64, 64, 1, 1, 1, "none"),
                                             (64, 64, 2, 1, 65, "none")])
def test_causal_r32(d, dv, B, H, n, gate):
    wl = WORKLOADS["favor_causal"].resized(d_k=d, d_v=dv, r=32, gate=gate, qk_scale=d ** -0.25, v_scale=1.0)
    inp = make_inputs(wl, seed=7, B=B, H=H, n=n)
    out, S, z = run_forward(inp, return_state=True)
    assert S.shape[-2:] == (32, dv) and z.shape[-1] == 32
    ref, Sr, zr = oracle_forward(inp)
    check_close(out, ref, TOL_BF16, f"favor r32 d{d} dv{dv} B{B} H{H} n{n} {gate}")
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 2e-2
    np.testing.assert_allclose(to_f64(z), zr, rtol=2e-2)


def test_causal_r32_carried_state():
    wl = WORKLOADS["favor_causal"].resized(r=32, qk_scale=64 ** -0.25, v_scale=1.0)
    inp = make_inputs(wl, seed=9, B=2, H=3, n=700)
    rng = np.random.default_rng(23)
    S0 = torch.from_numpy((rng.standard_normal((2, 3, 32, 64)) * 0.5).astype(np.float32))
    z0 = torch.from_numpy((5.0 + np.abs(rng.standard_normal((2, 3, 32)))).astype(np.float32))
    out, S, z = run_forward(inp, return_state=True, S0=S0, z0=z0)
    ref, Sr, zr = oracle_forward(inp, S0=to_f64(S0), z0=to_f64(z0))
    check_close(out, ref, TOL_BF16, "favor r32 carried state")
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 2e-2


@pytest.mark.parametrize("dtype,d,dv", [("f32", 64, 64), ("bf16", 32, 32), ("f32", 128, 128)])
def test_noncausal_r32(dtype, d, dv):
    wl = WORKLOADS["noncausal_elu1_f32"].resized(d_k=d, d_v=dv, r=32, fmap="favor", dtype=dtype,
                                                 qk_scale=d ** -0.25, v_scale=1.0)
    inp = make_inputs(wl, seed=3, B=2, H=3, n=500)
    out = run_forward(inp, out_dtype=torch.float32)
    ref, _, _ = oracle_forward(inp)
    check_close(out, ref, TOL_F32, f"noncausal favor r32 {dtype} d{d} dv{dv}")


@pytest.mark.parametrize("gate,dtype", [("none", "f32"), ("gla", "bf16"), ("decay", "f32")])
def test_decode_r32(gate, dtype):
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["gla_decode"].resized(fmap="favor", gate=gate, dtype=dtype, d_k=64, d_v=64, r=32,
                                         qk_scale=64 ** -0.25)
    inp = make_inputs(wl, seed=8, B=3, H=5)
    om = inp["omega"]
    g_gpu = None if gate == "none" else (("decay", dev(inp["gamma"])) if gate == "decay" else ("gla", dev(inp["g"]), wl.tau))
    g_orc = None if gate == "none" else (("decay", to_f64(inp["gamma"])) if gate == "decay" else ("gla", to_f64(inp["g"]), wl.tau))
    S, z = dev(inp["S0"]), dev(inp["z0"])
    out = ksm.decode_step(S, z, dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), fmap="favor", omega=dev(om), gate=g_gpu,
                          eps=wl.eps)
    torch.cuda.synchronize()
    o, S1, z1 = orc.decode_step(to_f64(inp["S0"]), to_f64(inp["z0"]), to_f64(inp["q"]), to_f64(inp["k"]),
                                to_f64(inp["v"]), "favor", to_f64(om), g_orc, wl.eps)
    check_close(out.cpu(), o, TOL_F32, f"decode favor r32 {gate} {dtype}")
    np.testing.assert_allclose(to_f64(S), S1, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_feature_map_r32(dtype, d):
    import kernelized_sequence_mixing_amd as ksm
    rng = np.random.default_rng(12)
    X = torch.from_numpy(rng.standard_normal((3, 77, d), dtype=np.float32) * d ** -0.25)
    X = X.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    om = torch.from_numpy(rng.standard_normal((32, d), dtype=np.float32)).to(X.dtype)
    phi = ksm.feature_map(dev(X), fmap="favor", omega=dev(om)).cpu()
    assert phi.shape[-1] == 32
    check_close(phi, orc.feature_map(to_f64(X), "favor", to_f64(om)), TOL_F32, f"phi favor r32 {dtype}")
