"""GPU parity at the edge of the gate domain.

The chunked kernels form the GLA and outer-product gate factors e^{+b}, e^{-b}
against the start of each 64-token chunk, which the header states as a
precondition: within every chunk the summed log-gate of each feature (and, for
the outer-product gate, of each value column) stays at or above -80. Inputs
drawn N(0, 1) stay near -3 per chunk, far from it. Here the strong chunks (every
other chunk, or all of them) carry a gate input near -18.75 at tau 16: a
per-step log-gate near -1.17 and a chunk sum near -75, checked on the oracle's
own gate values before each run. The strong and ordinary chunks alternate, so
chunk and segment boundaries meet both. The selective scalar gate and the
decode step have no such limit and are driven far beyond it, down to gates
that are exactly zero in fp32 ("Gating and Selective State Updates",
dileepadev page: G_t = 0 overwrites the state).
"""
import numpy as np
import pytest
import torch

import oracle as orc
from oracle import la_backward as obwd
from workloads import WORKLOADS, make_inputs, strong_gate_input, to_f64, incoming_gradient
from _helpers import TOL_BF16, check_close, dev, gpu_gate, oracle_forward, run_forward

pytestmark = pytest.mark.gpu

TOL_TERMS = 2e-2
EDGE_LO, EDGE_HI = -80.0, -70.0


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def chunk_log_sums(g, tau, n):
    """Per-chunk sums of log alpha (the oracle's gate) over the 64-token chunks: [.., chunks, features]."""
    la = np.log(orc.gla_alpha(to_f64(g), tau))
    nc = -(-n // 64)
    pad = nc * 64 - n
    if pad:
        la = np.concatenate([la, np.zeros(la.shape[:2] + (pad,) + la.shape[3:])], axis=2)
    return la.reshape(la.shape[:2] + (nc, 64) + la.shape[3:]).sum(axis=3)


def assert_at_edge(g, tau, n, period):
    """The strong chunks that are whole (64 steps) sum to within [-80, -70] on every feature."""
    s = chunk_log_sums(g, tau, n)
    full = s[:, :, [c for c in range(0, n // 64, period)]]
    print(f"  per-chunk summed log-gate of the strong chunks: min {full.min():.2f} max {full.max():.2f}",
          flush=True)
    assert full.min() >= EDGE_LO and full.max() <= EDGE_HI, (full.min(), full.max())


def gla_case(d, dv, B, H, n, period, seed, fmap="elu1"):
    wl = WORKLOADS["gla_gate"].resized(d_k=d, d_v=dv, r=d, fmap=fmap,
                                       v_scale=1.0 if fmap == "identity" else d ** -0.5)
    inp = make_inputs(wl, seed=seed, B=B, H=H, n=n)
    inp["g"] = strong_gate_input((B, H, n, d), seed + 50, period=period)
    return wl, inp


# ------------------------------------------------------------------ GLA forward

@pytest.mark.parametrize("d,dv,B,H,n,period", [(128, 128, 4, 16, 1285, 2), (64, 64, 4, 16, 1285, 2),
                                               (128, 64, 2, 4, 777, 1), (64, 128, 2, 2, 200, 1),
                                               (64, 64, 2, 3, 130, 3)])
def test_gla_forward_at_the_domain_edge(d, dv, B, H, n, period):
    """Segments of several chunks with a ragged tail (n 1285: segment
    boundaries fall on strong chunks), every chunk strong, tiny n."""
    wl, inp = gla_case(d, dv, B, H, n, period, seed=11)
    assert_at_edge(inp["g"], wl.tau, n, period)
    out, S, z = run_forward(inp, return_state=True)
    assert np.isfinite(to_f64(out)).all()
    ref, Sr, zr = oracle_forward(inp)
    check_close(out, ref, TOL_BF16, f"GLA edge d{d}x{dv} B{B} H{H} n{n} period {period}")
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 2e-2
    np.testing.assert_allclose(to_f64(z), zr, rtol=2e-2, atol=1e-6 * np.max(zr))


def test_gla_state_space_at_the_domain_edge():
    """The identity feature map (the selective state-space form) under strong
    GLA gates, term-relative like every state-space check."""
    wl, inp = gla_case(64, 64, 4, 16, 1285, 2, seed=12, fmap="identity")
    assert_at_edge(inp["g"], wl.tau, 1285, 2)
    out = run_forward(inp)
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    gate = ("gla", to_f64(inp["g"]), wl.tau)
    o = orc.causal_recurrent(Q, K, V, "identity", None, gate)[0]
    sc = orc.causal_recurrent(np.abs(Q), np.abs(K), np.abs(V), "identity", None, gate)[0]
    e = float(np.max(np.abs(to_f64(out) - o) / (sc + 1e-30)))
    print(f"  state-space GLA edge: term-relative {e:.2e}", flush=True)
    assert e < TOL_TERMS


def test_gla_serving_batch_at_the_domain_edge():
    """Ragged sequences through la_forward_batch (chunks counted from each
    sequence's own start), each against the oracle on it alone."""
    import kernelized_sequence_mixing_amd as ksm
    lens = np.array([1, 64, 65, 300, 130, 0, 257], dtype=np.int32)
    T = int(lens.sum()) + 10
    wl, inp = gla_case(128, 128, 1, 4, T, 1, seed=13)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = ksm.forward_batch(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), cu_seqlens=dev(torch.from_numpy(cu)),
                            max_seqlen=int(lens.max()), gate=gpu_gate(inp), eps=wl.eps)
    torch.cuda.synchronize()
    out = out.cpu()
    for b in range(len(lens)):
        if lens[b] == 0:
            continue
        sl = slice(int(cu[b]), int(cu[b + 1]))
        part = {k: (v[:, :, sl].contiguous() if k in ("Q", "K", "V", "g") else v) for k, v in inp.items()}
        ref, _, _ = oracle_forward(part)
        check_close(out[:, :, sl], ref, TOL_BF16, f"batch edge seq {b} len {lens[b]}")


# ------------------------------------------------------------------ outer-product gate

@pytest.mark.parametrize("side", ["key", "value", "both"])
@pytest.mark.parametrize("d,dv,B,H,n", [(128, 128, 4, 16, 1285), (64, 64, 2, 4, 300)])
def test_outer_gate_at_the_domain_edge(side, d, dv, B, H, n):
    wl = WORKLOADS["outer_gate"].resized(d_k=d, d_v=dv, r=d, qk_scale=d ** -0.5, v_scale=d ** -0.5)
    inp = make_inputs(wl, seed=14, B=B, H=H, n=n)
    if side in ("key", "both"):
        inp["g"] = strong_gate_input((B, H, n, d), 60)
        assert_at_edge(inp["g"], wl.tau, n, 2)
    if side in ("value", "both"):
        inp["gv"] = strong_gate_input((B, H, n, dv), 61)
        assert_at_edge(inp["gv"], wl.tau, n, 2)
    out, S, z = run_forward(inp, return_state=True)
    ref, Sr, zr = oracle_forward(inp)
    check_close(out, ref, TOL_BF16, f"outer edge ({side} side) d{d}x{dv} n{n}")
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 2e-2


# ------------------------------------------------------------------ selective scalar gate: no limit

@pytest.mark.parametrize("fmap", ["elu1", "identity"])
def test_selective_gate_far_beyond_the_edge(fmap):
    """Chunk sums near -1000 (g near -250 at tau 16) and isolated gates that
    are exactly zero in fp32 (g = -30000: log a = -1875), at chunk starts,
    chunk ends and inside chunks."""
    wl = WORKLOADS["ssm_scalar"].resized(fmap=fmap, qk_scale=64 ** -0.5, v_scale=1.0 if fmap == "identity" else 0.125)
    B, H, n = 4, 16, 1285
    inp = make_inputs(wl, seed=15, B=B, H=H, n=n)
    g = strong_gate_input((B, H, n), 62, mean=-250.0, std=20.0, period=2)
    g[:, :, [64, 127, 300, 555, 1000]] = -30000.0
    inp["g"] = g
    out = run_forward(inp)
    assert np.isfinite(to_f64(out)).all()
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    gate = ("sel", to_f64(g), wl.tau)
    ref = orc.causal_recurrent(Q, K, V, fmap, None, gate, eps=wl.eps)[0]
    if fmap == "elu1":
        check_close(out, ref, TOL_BF16, "selective gate, strong chunks and zero gates")
    else:
        sc = orc.causal_recurrent(np.abs(Q), np.abs(K), np.abs(V), "identity", None, gate)[0]
        e = float(np.max(np.abs(to_f64(out) - ref) / (sc + 1e-30)))
        print(f"  state-space selective edge: term-relative {e:.2e}", flush=True)
        assert e < TOL_TERMS


# ------------------------------------------------------------------ decode step: no limit

@pytest.mark.parametrize("gate", ["gla", "sel", "outer"])
def test_decode_step_with_zero_gates(gate):
    """Gates of exactly zero overwrite the state: S' = phi(k) v^T, z' = phi(k)
    wherever the gate is zero; the other heads draw N(0, 1) gates."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["gla_decode"].resized(B=8, H=4, gate=gate)
    inp = make_inputs(wl, seed=16)
    g = inp["g"].clone()
    g[::2] = -30000.0
    gv = inp["gv"].clone() if gate == "outer" else None
    if gate == "outer":
        gv[::2] = -30000.0
    S, z = dev(inp["S0"]), dev(inp["z0"])
    gg = (gate, dev(g), wl.tau) if gate != "outer" else ("outer", dev(g), dev(gv), wl.tau)
    out = ksm.decode_step(S, z, dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), gate=gg, eps=wl.eps)
    torch.cuda.synchronize()
    og = (gate, to_f64(g), wl.tau) if gate != "outer" else ("outer", to_f64(g), to_f64(gv), wl.tau)
    o, S1, z1 = orc.decode_step(to_f64(inp["S0"]), to_f64(inp["z0"]), to_f64(inp["q"]), to_f64(inp["k"]),
                                to_f64(inp["v"]), "elu1", None, og, eps=wl.eps)
    e = float(np.max(np.abs(to_f64(out.cpu()) - o)) / np.max(np.abs(o)))
    print(f"  decode {gate} with zero gates: err {e:.2e}", flush=True)
    assert e < 1e-4
    np.testing.assert_allclose(to_f64(S), S1, rtol=1e-5, atol=1e-4)
    pk = orc.phi_elu1(to_f64(inp["k"]))
    np.testing.assert_allclose(to_f64(z)[::2], pk[::2], rtol=1e-6)


# ------------------------------------------------------------------ GLA backward (dg included)

def test_gla_backward_at_the_domain_edge():
    """The backward passes reuse the forward's chunk-start factors, dg included."""
    from test_gpu_backward_gla import check_heads, run_backward_gla
    B, H, n = 4, 16, 1285
    wl, inp = gla_case(64, 64, B, H, n, 2, seed=17)
    assert_at_edge(inp["g"], wl.tau, n, 2)
    dO = incoming_gradient((B, H, n, 64), 117)
    got = run_backward_gla(inp, dO)
    for x in got:
        assert np.isfinite(to_f64(x)).all()
    check_heads(got, inp, dO, [(0, 0), (3, 15)], "GLA backward edge")


def test_gla_backward_state_space_at_the_domain_edge():
    from test_gpu_backward_gla import check_heads, run_backward_gla
    B, H, n = 2, 4, 777
    wl, inp = gla_case(64, 64, B, H, n, 1, seed=18, fmap="identity")
    assert_at_edge(inp["g"], wl.tau, n, 1)
    dO = incoming_gradient((B, H, n, 64), 118)
    got = run_backward_gla(inp, dO, fmap="identity")
    check_heads(got, inp, dO, [(0, 0), (1, 3)], "GLA backward edge, state-space", fmap="identity")


# ------------------------------------------------------------------ RetNet decay with a small gamma

# gamma^-15 overflows fp32 below about 0.0027; a factor above the diagonal must
# never meet a product (0 * inf = NaN)
SMALL_GAMMAS = [1e-3, 1e-5, 1e-12, 0.0025]


@pytest.mark.parametrize("name,d,dv", [("retnet_decay", 128, 128), ("retnet_decay", 64, 64),
                                       ("favor_causal", 64, 64)])
def test_decay_with_small_gamma(name, d, dv):
    """Several segments with a ragged tail chunk (n 1285) at gammas down to 1e-12."""
    r = 256 if name == "favor_causal" else d
    wl = WORKLOADS[name].resized(gate="decay", d_k=d, d_v=dv, r=r)
    inp = make_inputs(wl, seed=19, B=2, H=4, n=1285)
    inp["gamma"] = torch.tensor(SMALL_GAMMAS, dtype=torch.float32)
    out, S, z = run_forward(inp, return_state=True)
    assert np.isfinite(to_f64(out)).all() and np.isfinite(to_f64(S)).all()
    ref, Sr, zr = oracle_forward(inp)
    check_close(out, ref, TOL_BF16, f"{name} small gamma d{d}x{dv}")
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 2e-2


def test_decay_backward_with_small_gamma():
    from test_gpu_backward import _case, check_grads, oracle_backward, run_backward, term_scales
    wl, inp, dO = _case("decay", 64, 64, 2, 4, 777)
    inp["gamma"] = torch.tensor(SMALL_GAMMAS, dtype=torch.float32)
    got = run_backward(inp, dO)
    for x in got:
        assert np.isfinite(to_f64(x)).all()
    check_grads(got, oracle_backward(inp, dO), term_scales(inp, dO), "decay backward, small gamma")
