"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Small shapes span several chunks, several segments and a ragged tail and are
compared element by element on every head; the full-size workloads run in the
launch configuration the benchmark times and are compared on sampled heads
(each head is an independent problem the oracle computes in full), plus
properties that hold at any size on every output.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from workloads import WORKLOADS, make_inputs, to_f64
from _helpers import (TOL_BF16, TOL_F32, check_close, dev, gpu_gate, oracle_forward, run_forward, tol_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    import kernelized_sequence_mixing_amd as ksm
    from kernelized_sequence_mixing_amd import _native
    _native.lib()  # raise loudly if the library is missing
    return ksm


# ------------------------------------------------------------------ non-causal

def test_noncausal_f32_workload_full():
    """B=1 H=1 n=256 d=32 fp32, eps 1e-6: reassociated oracle and the explicit
    256 x 256 kernel matrix, at 1e-4."""
    inp = make_inputs("noncausal_elu1_f32")
    out, S, z = run_forward(inp, return_state=True)
    ref, _, _ = oracle_forward(inp)
    check_close(out, ref, TOL_F32, "noncausal f32 vs reassociated")
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    check_close(out, orc.brute(Q, K, V, causal=False, eps=1e-6), TOL_F32, "noncausal f32 vs 256x256 matrix")
    pk = orc.phi_elu1(K)
    np.testing.assert_allclose(to_f64(S), np.einsum("bhjr,bhje->bhre", pk, V), rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(to_f64(z), pk.sum(axis=2), rtol=1e-5)


@pytest.mark.parametrize("fmap,dtype,d,dv,r,n", [
    ("elu1", "f32", 64, 32, 64, 1000), ("elu1", "bf16", 128, 128, 128, 517), ("favor", "f32", 64, 64, 256, 300),
    ("favor", "bf16", 32, 128, 128, 129), ("elu1", "f32", 32, 64, 32, 1)])
def test_noncausal_shapes(fmap, dtype, d, dv, r, n):
    wl = WORKLOADS["noncausal_elu1_f32"].resized(d_k=d, d_v=dv, r=r, fmap=fmap, dtype=dtype,
                                                 qk_scale=d ** -0.25 if fmap == "favor" else 1.0, v_scale=1.0)
    inp = make_inputs(wl, seed=3, B=2, H=3, n=n)
    out = run_forward(inp, out_dtype=torch.float32)
    ref, _, _ = oracle_forward(inp)
    check_close(out, ref, TOL_F32, f"noncausal {fmap} {dtype} n={n}")


# ------------------------------------------------------------------ causal, small shapes on every head

CAUSAL = ["causal_elu1", "retnet_decay", "gla_gate", "favor_causal"]


@pytest.mark.parametrize("name", CAUSAL)
@pytest.mark.parametrize("B,H,n", [(4, 16, 1285), (1, 2, 200), (8, 64, 100), (1, 1, 1), (2, 1, 63), (2, 1, 65)])
def test_causal_parity_small(name, B, H, n):
    """Multi-chunk segments with a ragged last one (B4 H16 n1285), one chunk
    per segment (B1 H2 n200), a single segment (B8 H64 n100) and tiny n."""
    wl = WORKLOADS[name]
    if name == "retnet_decay":
        H = min(H, 8) if H > 1 else H
    inp = make_inputs(wl, seed=1, B=B, H=H, n=n)
    out, S, z = run_forward(inp, return_state=True)
    ref, Sr, zr = oracle_forward(inp)
    check_close(out, ref, TOL_BF16, f"{name} B{B} H{H} n{n}")
    # the carried state leaves the kernel in fp32; bf16 operands bound its error
    scale = np.max(np.abs(Sr)) + 1e-30
    assert np.max(np.abs(to_f64(S) - Sr)) / scale < 2e-2
    np.testing.assert_allclose(to_f64(z), zr, rtol=2e-2)


@pytest.mark.parametrize("name", CAUSAL)
def test_causal_stress_unscaled(name):
    """Unscaled N(0,1) inputs make the features vary strongly (the workloads'
    scaling keeps elu+1 features near 1, which would hide feature-map slips)."""
    wl = WORKLOADS[name]
    qk = 0.5 if name == "favor_causal" else 1.0
    inp = make_inputs(wl, seed=5, B=2, H=4 if name != "retnet_decay" else 4, n=777, qk_scale=qk, v_scale=1.0)
    out = run_forward(inp)
    ref, _, _ = oracle_forward(inp)
    check_close(out, ref, TOL_BF16, f"{name} unscaled")


# ------------------------------------------------------------------ full-size workloads, sampled heads

@pytest.mark.parametrize("name", CAUSAL)
def test_causal_workload_full_size(name):
    wl = WORKLOADS[name]
    inp = make_inputs(wl, seed=0)
    print(f"  {name}: B={wl.B} H={wl.H} n={wl.n} d_k={wl.d_k} d_v={wl.d_v} r={wl.r}", flush=True)
    out = run_forward(inp)
    o = to_f64(out)
    assert np.all(np.isfinite(o))
    # outputs are shrunk convex combinations of the values they mix
    vmax = np.max(np.abs(to_f64(inp["V"])), axis=(2, 3), keepdims=True)
    assert np.all(np.abs(o) <= vmax * (1 + 1e-2) + 1e-6)
    for head in [(0, 0), (wl.B - 1, wl.H - 1)]:
        ref, _, _ = oracle_forward(inp, head=head)
        check_close(out[head[0]:head[0] + 1, head[1]:head[1] + 1], ref, TOL_BF16, f"{name} head {head}")


# ------------------------------------------------------------------ exact structure (bit-exact)

@pytest.mark.parametrize("name", ["causal_elu1", "retnet_decay", "gla_gate", "favor_causal", "outer_gate"])
def test_exact_zero_probe(name):
    """V = 0 except a single 1 at (p, c): every output before p is exactly
    0.0, no other column is ever nonzero, and o_p[c] > 0. Sweeps p over chunk
    and segment boundaries, one (b, h) slice per p."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS[name]
    B, H, n = 4, 16, 1285
    if name == "retnet_decay":
        B, H = 8, 8
    inp = make_inputs(wl, seed=2, B=B, H=H, n=n)
    P, L = ksm.segments(B, H, n, wl.d_k, wl.d_v, fmap=wl.fmap, r=wl.r, gate_kind=wl.gate)
    ps = sorted({0, 1, 63, 64, 65, 127, 128, L - 1, L, L + 1, 2 * L - 1, 2 * L, (P - 1) * L, n - 2, n - 1} - {-1})
    ps = [p for p in ps if 0 <= p < n][:B * H]
    V = torch.zeros_like(inp["V"])
    col = 5
    for i, p in enumerate(ps):
        V[i // H, i % H, p, col] = 1.0
    inp["V"] = V
    out = to_f64(run_forward(inp))
    for i, p in enumerate(ps):
        o = out[i // H, i % H]
        assert np.all(o[:p] == 0.0), f"future leak before p={p}"
        assert o[p, col] > 0, f"o_p missing at p={p}"
        assert np.all(np.delete(o, col, axis=1) == 0.0)
    unused = out.reshape(B * H, n, -1)[len(ps):]
    assert np.all(unused == 0.0)


def test_integer_exact_probe():
    """Q = K = 0 makes every elu+1 feature exactly 1, so scores are exactly d and
    the denominators exactly (i+1) d. Integer values whose running sums stay
    small keep every partial sum exact in bf16/fp32; with eps = 0 each output
    must equal fl(num * fl(1 / den)) in IEEE fp32 (one correctly rounded
    reciprocal per row, then a product) rounded to bf16, bit for bit, across
    chunk and segment boundaries and the ragged tail."""
    wl = WORKLOADS["causal_elu1"]
    B, H, n = 4, 16, 1285
    inp = make_inputs(wl, seed=0, B=B, H=H, n=n)
    inp["Q"] = torch.zeros_like(inp["Q"])
    inp["K"] = torch.zeros_like(inp["K"])
    t = np.arange(n)[:, None]
    e = np.arange(wl.d_v)[None, :]
    bh = np.arange(B * H).reshape(B, H, 1, 1)
    Vint = (((t + e + bh) % 3) - 1) * (1 + (e % 4))           # period-3 zero-sum pattern: bounded prefix sums
    inp["V"] = torch.from_numpy(Vint.astype(np.float32)).to(torch.bfloat16)
    out = run_forward(inp, eps=0.0)
    num = np.cumsum(np.broadcast_to(Vint, (B, H, n, wl.d_v)).astype(np.float64), axis=2) * wl.d_k
    den = (np.arange(1, n + 1, dtype=np.float64) * wl.d_k)[None, None, :, None]
    assert np.all(np.abs(num) < 2 ** 24) and np.all(np.abs(num / wl.d_k) <= 256)
    inv = (np.float32(1.0) / den.astype(np.float32)).astype(np.float32)
    q32 = (num.astype(np.float32) * inv).astype(np.float32)
    want = torch.from_numpy(q32).to(torch.bfloat16)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("name", CAUSAL)
def test_deterministic(name):
    inp = make_inputs(WORKLOADS[name], seed=4, B=2, H=8, n=1000)
    a = run_forward(inp)
    b = run_forward(inp)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------------------------------ state handoff and decode

@pytest.mark.parametrize("name", CAUSAL)
def test_initial_state_resumes(name):
    """forward(second half, S0/z0 = oracle state after the first half) equals
    the oracle over the whole sequence (the state is the whole history)."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl, seed=6, B=2, H=4, n=600)
    m = 257
    full, _, _ = oracle_forward(inp)
    first = {k: (v[:, :, :m] if isinstance(v, torch.Tensor) and v.dim() == 4 and k != "omega" else v)
             for k, v in inp.items()}
    _, S1, z1 = oracle_forward(first)
    second = {k: (v[:, :, m:].contiguous() if isinstance(v, torch.Tensor) and v.dim() == 4 and k != "omega" else v)
              for k, v in inp.items()}
    second["n"] = 600 - m
    out = run_forward(second, S0=torch.from_numpy(S1.astype(np.float32)), z0=torch.from_numpy(z1.astype(np.float32)))
    check_close(out, full[:, :, m:], TOL_BF16, f"{name} resumed")


@pytest.mark.parametrize("gate,d,dv,B,H,n", [("decay", 64, 64, 4, 16, 700), ("gla", 64, 64, 4, 16, 700),
                                              ("gla", 32, 64, 2, 16, 1100), ("decay", 32, 64, 2, 16, 1100)])
def test_small_state_gates_resume(gate, d, dv, B, H, n):
    """Gated forms with small states over several segments with a ragged last
    one, resumed from a carried-in state, against the oracle over the whole
    history (outputs and final state)."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["causal_elu1"].resized(d_k=d, d_v=dv, r=d, gate=gate)
    P, L = ksm.segments(B, H, n, d, dv, fmap="elu1", r=d, gate_kind=gate)
    assert P > 1 and n % L != 0, (P, L)
    m = 130
    inp = make_inputs(wl, seed=11, B=B, H=H, n=m + n)
    full, Sr, zr = oracle_forward(inp)
    first = {k: (v[:, :, :m] if isinstance(v, torch.Tensor) and v.dim() == 4 else v) for k, v in inp.items()}
    _, S1, z1 = oracle_forward(first)
    second = {k: (v[:, :, m:].contiguous() if isinstance(v, torch.Tensor) and v.dim() == 4 else v)
              for k, v in inp.items()}
    second["n"] = n
    out, S, z = run_forward(second, return_state=True, S0=torch.from_numpy(S1.astype(np.float32)),
                            z0=torch.from_numpy(z1.astype(np.float32)))
    check_close(out, full[:, :, m:], TOL_BF16, f"{gate} d{d}x{dv} resumed")
    scale = np.max(np.abs(Sr)) + 1e-30
    assert np.max(np.abs(to_f64(S) - Sr)) / scale < 2e-2
    np.testing.assert_allclose(to_f64(z), zr, rtol=2e-2)


def test_decode_workload_full():
    """Decode step at batch 256 x 16 heads with 128 x 128 fp32 states (GLA)."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["gla_decode"]
    inp = make_inputs(wl, seed=0)
    S, z = dev(inp["S0"]), dev(inp["z0"])
    out = ksm.decode_step(S, z, dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), gate=("gla", dev(inp["g"]), wl.tau),
                          eps=wl.eps)
    torch.cuda.synchronize()
    o, S1, z1 = orc.decode_step(to_f64(inp["S0"]), to_f64(inp["z0"]), to_f64(inp["q"]), to_f64(inp["k"]),
                                to_f64(inp["v"]), gate=("gla", to_f64(inp["g"]), wl.tau), eps=wl.eps)
    check_close(out.cpu(), o, TOL_F32, "decode out")
    np.testing.assert_allclose(to_f64(S), S1, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(to_f64(z), z1, rtol=1e-6)


@pytest.mark.parametrize("fmap,gate,dtype", [("elu1", "none", "f32"), ("elu1", "decay", "bf16"),
                                             ("favor", "gla", "f32"), ("favor", "decay", "bf16"),
                                             ("elu1", "gla", "bf16")])
def test_decode_variants(fmap, gate, dtype):
    import kernelized_sequence_mixing_amd as ksm
    d, dv, r = (64, 64, 256) if fmap == "favor" else (128, 64, 128)
    wl = WORKLOADS["gla_decode"].resized(fmap=fmap, gate=gate, dtype=dtype, d_k=d, d_v=dv, r=r,
                                         qk_scale=d ** -0.25 if fmap == "favor" else 1.0)
    inp = make_inputs(wl, seed=8, B=3, H=5)
    om = inp.get("omega")
    g_gpu = None if gate == "none" else (("decay", dev(inp["gamma"])) if gate == "decay" else ("gla", dev(inp["g"]), wl.tau))
    g_orc = None if gate == "none" else (("decay", to_f64(inp["gamma"])) if gate == "decay" else ("gla", to_f64(inp["g"]), wl.tau))
    S, z = dev(inp["S0"]), dev(inp["z0"])
    out = ksm.decode_step(S, z, dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), fmap=fmap, omega=dev(om), gate=g_gpu,
                          eps=wl.eps)
    torch.cuda.synchronize()
    o, S1, z1 = orc.decode_step(to_f64(inp["S0"]), to_f64(inp["z0"]), to_f64(inp["q"]), to_f64(inp["k"]),
                                to_f64(inp["v"]), fmap, None if om is None else to_f64(om), g_orc, wl.eps)
    check_close(out.cpu(), o, TOL_F32, f"decode {fmap} {gate} {dtype}")
    np.testing.assert_allclose(to_f64(S), S1, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("name", ["causal_elu1", "gla_gate", "retnet_decay", "favor_causal"])
def test_prefill_then_decode_matches_forward(name):
    """forward(n - m) -> (S, z) -> m decode steps == forward(n) on the GPU, and
    both match the oracle: the parallel/recurrent duality end to end."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS[name]
    B, H, n, m = 2, 4, 300, 5
    inp = make_inputs(wl, seed=9, B=B, H=H, n=n)
    ref, _, _ = oracle_forward(inp)
    pre = {k: (v[:, :, :n - m].contiguous() if isinstance(v, torch.Tensor) and v.dim() == 4 else v)
           for k, v in inp.items()}
    pre["n"] = n - m
    _, S, z = run_forward(pre, return_state=True)
    S, z = S.cuda(), z.cuda()
    om = dev(inp.get("omega"))
    for t in range(n - m, n):
        sl = lambda x: dev(x[:, :, t].contiguous())  # noqa: E731
        if wl.gate == "gla":
            gg = ("gla", sl(inp["g"]), wl.tau)
        elif wl.gate == "decay":
            gg = ("decay", dev(inp["gamma"]))
        else:
            gg = None
        o = ksm.decode_step(S, z, sl(inp["Q"]), sl(inp["K"]), sl(inp["V"]), fmap=wl.fmap, omega=om, gate=gg,
                            eps=wl.eps)
        check_close(o.cpu()[:, :, None, :], ref[:, :, t:t + 1], TOL_BF16, f"{name} decode t={t}")


# ------------------------------------------------------------------ feature map alone

@pytest.mark.parametrize("fmap,dtype,d,r", [("elu1", "f32", 64, 64), ("elu1", "bf16", 128, 128),
                                            ("favor", "f32", 64, 256), ("favor", "bf16", 32, 64)])
def test_feature_map(fmap, dtype, d, r):
    import kernelized_sequence_mixing_amd as ksm
    rng = np.random.default_rng(12)
    X = torch.from_numpy(rng.standard_normal((3, 77, d), dtype=np.float32) * (d ** -0.25 if fmap == "favor" else 2.0))
    X = X.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    om = None
    if fmap == "favor":
        om = torch.from_numpy(rng.standard_normal((r, d), dtype=np.float32)).to(X.dtype)
    phi = ksm.feature_map(dev(X), fmap=fmap, omega=dev(om)).cpu()
    ref = orc.feature_map(to_f64(X), fmap, None if om is None else to_f64(om))
    check_close(phi, ref, TOL_F32, f"phi {fmap} {dtype}")


# ------------------------------------------------------------------ prepared calls

@pytest.mark.parametrize("name", ["causal_elu1", "gla_gate", "favor_causal"])
def test_prepared_forward_matches_forward(name):
    """PreparedForward launches the same la_forward call: bitwise the output of
    forward(), on every repeat, and after the inputs are overwritten in place."""
    import kernelized_sequence_mixing_amd as ksm
    inp = make_inputs(WORKLOADS[name], seed=12, B=2, H=4, n=777)
    Q, K, V = dev(inp["Q"]), dev(inp["K"]), dev(inp["V"])
    kw = dict(fmap=inp["fmap"], omega=dev(inp.get("omega")), causal=True, gate=gpu_gate(inp), eps=inp["eps"])
    ref = ksm.forward(Q, K, V, **kw)
    call = ksm.PreparedForward(Q, K, V, **kw)
    for _ in range(3):
        got = call()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    Q.mul_(0.5)
    ref2 = ksm.forward(Q, K, V, **kw)
    got2 = call()
    torch.cuda.synchronize()
    assert torch.equal(got2.view(torch.int16), ref2.view(torch.int16))


def test_prepared_decode_matches_decode_step():
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["gla_decode"]
    inp = make_inputs(wl, seed=13, B=4, H=3)
    q, k, v, g = (dev(inp[x]) for x in ("q", "k", "v", "g"))
    S1, z1 = dev(inp["S0"]), dev(inp["z0"])
    S2, z2 = S1.clone(), z1.clone()
    call = ksm.PreparedDecode(S2, z2, q, k, v, gate=("gla", g, wl.tau), eps=wl.eps)
    for _ in range(2):  # two steps: the state advances in place both ways
        ref = ksm.decode_step(S1, z1, q, k, v, gate=("gla", g, wl.tau), eps=wl.eps)
        got = call()
        torch.cuda.synchronize()
        assert torch.equal(got, ref) and torch.equal(S2, S1) and torch.equal(z2, z1)
