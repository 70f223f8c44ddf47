"""GPU parity of the state-space form (identity features, unnormalised
read-out y_t = C_t^T h_t) against the fp64 oracle.

The read-out is a plain sum of signed terms q_ik k_jk D_ijk v_je (D the gate
products), so the error is measured entrywise against the sum of the terms'
magnitudes, which the oracle's own recurrence gives when it runs on |q|, |k|,
|v| (and |S0|): each term carries at most four bf16 roundings (q e^b, k e^-b,
the rounded score or the state's bf16 image, and the output), about 4 * 2^-9
of its size, and the tolerance is 2e-2, the derivation of the backward pass's
gradients. A row-relative measure would be meaningless here: outputs are
random walks over the keys, far smaller than their terms.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from workloads import WORKLOADS, make_inputs, to_f64
from _helpers import dev, gpu_gate

pytestmark = pytest.mark.gpu

TOL_TERMS = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _gate64(inp, head=None):
    if inp["gate"] == "decay":
        gam = to_f64(inp["gamma"])
        return ("decay", gam if head is None else gam[head[1]:head[1] + 1])
    if inp["gate"] in ("gla", "sel"):
        g = to_f64(inp["g"])
        if head is not None:
            g = g[head[0]:head[0] + 1, head[1]:head[1] + 1]
        return (inp["gate"], g, inp["tau"])
    return None


def oracle_ssm(inp, head=None, S0=None, z0=None):
    """(o, scale, S, z): the oracle's read-out and the magnitude sum of its terms."""
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    if head is not None:
        b, h = head
        Q, K, V = (x[b:b + 1, h:h + 1] for x in (Q, K, V))
    gate = _gate64(inp, head)
    o, S, z = orc.causal_recurrent(Q, K, V, "identity", None, gate, eps=inp["eps"], S0=S0, z0=z0)
    sc = orc.causal_recurrent(np.abs(Q), np.abs(K), np.abs(V), "identity", None, gate,
                              S0=None if S0 is None else np.abs(S0), z0=z0)[0]
    return o, sc, S, z


def term_err(got, ref, scale):
    return float(np.max(np.abs(to_f64(got) - ref) / (scale + 1e-30)))


def run(inp, S0=None, z0=None, return_state=False):
    import kernelized_sequence_mixing_amd as ksm
    res = ksm.forward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), fmap="identity", causal=True,
                      gate=gpu_gate(inp), eps=inp["eps"], S0=dev(S0), z0=dev(z0), return_state=return_state)
    torch.cuda.synchronize()
    return tuple(x.cpu() for x in res) if return_state else res.cpu()


def _case(gate, d, dv, B, H, n, seed=2):
    wl = WORKLOADS["ssm_selective"].resized(d_k=d, d_v=dv, r=d, gate=gate, qk_scale=d ** -0.5)
    return wl, make_inputs(wl, seed=seed, B=B, H=H, n=n)


CASES = [(g, d, dv, B, H, n) for g in ("none", "decay", "gla", "sel")
         for (d, dv, B, H, n) in ((64, 64, 2, 4, 777), (64, 128, 2, 4, 300), (128, 64, 2, 3, 300),
                                  (32, 64, 2, 2, 129), (128, 128, 1, 2, 200), (64, 64, 4, 16, 1285))]


@pytest.mark.parametrize("gate,d,dv,B,H,n", CASES)
def test_ssm_parity(gate, d, dv, B, H, n):
    """Every built shape and gate: multi-chunk segments with a ragged tail (n
    777, 1285), one segment (n 129 .. 300), every head."""
    wl, inp = _case(gate, d, dv, B, H, n)
    got = run(inp)
    o, sc, _, _ = oracle_ssm(inp)
    e = term_err(got, o, sc)
    print(f"  ssm {gate} d{d}x{dv} B{B} H{H} n{n}: term-relative err {e:.2e}", flush=True)
    assert e < TOL_TERMS


@pytest.mark.parametrize("gate", ["none", "gla", "sel"])
def test_ssm_resumes_from_state(gate):
    """A carried-in state (the oracle's state after a 150-token prefix) and the
    final state: the continuation equals one pass over the whole sequence."""
    wl, inp = _case(gate, 64, 64, 2, 4, 700, seed=6)
    m = 150
    seq = ("Q", "K", "V", "g")  # the per-token inputs (the selective gate's g is [B, H, n])
    first = {k: (v[:, :, :m].contiguous() if k in seq else v) for k, v in inp.items()}
    second = {k: (v[:, :, m:].contiguous() if k in seq else v) for k, v in inp.items()}
    _, _, S1, z1 = oracle_ssm(first)
    o, sc, Sr, zr = oracle_ssm(second, S0=S1, z0=z1)
    got, S, z = run(second, torch.from_numpy(S1.astype(np.float32)), torch.from_numpy(z1.astype(np.float32)),
                    return_state=True)
    e = term_err(got, o, sc)
    print(f"  ssm {gate} resumed: term-relative err {e:.2e}", flush=True)
    assert e < TOL_TERMS
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 2e-2


@pytest.mark.parametrize("name", ["ssm_selective", "ssm_scalar"])
def test_ssm_full_size_sampled_heads(name):
    """The benchmark's shapes (B2 H16 n16384 d64 under the GLA and the
    selective gate, several segments), two heads against the oracle's recurrence."""
    wl = WORKLOADS[name]
    inp = make_inputs(wl, seed=0)
    got = run(inp)
    assert torch.isfinite(got.float()).all()
    for head in [(0, 0), (wl.B - 1, wl.H - 1)]:
        o, sc, _, _ = oracle_ssm(inp, head=head)
        b, h = head
        e = term_err(got[b:b + 1, h:h + 1], o, sc)
        print(f"  {name} full size head {head}: term-relative err {e:.2e}", flush=True)
        assert e < TOL_TERMS


@pytest.mark.parametrize("gate", ["none", "decay", "gla", "sel"])
def test_ssm_decode_step(gate):
    """The recurrent step with identity features (fp32 arithmetic): one step
    from a carried state equals the oracle's step."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["gla_decode"].resized(fmap="identity", gate=gate, B=8, H=4)
    inp = make_inputs(wl, seed=3)
    S, z = dev(inp["S0"]), dev(inp["z0"])
    g = None
    if gate == "decay":
        g = ("decay", dev(inp["gamma"]))
    elif gate in ("gla", "sel"):
        g = (gate, dev(inp["g"]), wl.tau)
    out = ksm.decode_step(S, z, dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), fmap="identity", gate=g, eps=wl.eps)
    torch.cuda.synchronize()
    og = None
    if gate == "decay":
        og = ("decay", to_f64(inp["gamma"]))
    elif gate in ("gla", "sel"):
        og = (gate, to_f64(inp["g"]), wl.tau)
    o, S1, z1 = orc.decode_step(to_f64(inp["S0"]), to_f64(inp["z0"]), to_f64(inp["q"]), to_f64(inp["k"]),
                                to_f64(inp["v"]), "identity", None, og, eps=wl.eps)
    sc, _, _ = orc.decode_step(np.abs(to_f64(inp["S0"])), to_f64(inp["z0"]), np.abs(to_f64(inp["q"])),
                               np.abs(to_f64(inp["k"])), np.abs(to_f64(inp["v"])), "identity", None, og, eps=wl.eps)
    e = term_err(out.cpu(), o, sc)
    print(f"  ssm decode {gate}: term-relative err {e:.2e}", flush=True)
    assert e < 1e-5  # fp32 arithmetic throughout
    np.testing.assert_allclose(to_f64(S), S1, rtol=1e-5, atol=1e-5)


def test_ssm_serving_batch():
    """A ragged prefill and a 4-token step through la_forward_batch with
    identity features, against the oracle on each whole sequence."""
    import kernelized_sequence_mixing_amd as ksm
    wl, _ = _case("gla", 64, 64, 1, 1, 1)
    H, m = 4, 4
    lens = [90, 1, 300, 64]
    full = [make_inputs(wl, seed=60 + b, B=1, H=H, n=L + m) for b, L in enumerate(lens)]
    pre = {k: torch.cat([f[k][:, :, :L] for f, L in zip(full, lens)], dim=2).contiguous() for k in ("Q", "K", "V", "g")}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    ids = torch.tensor([2, 0, 3, 1], dtype=torch.int32, device="cuda")
    S = torch.zeros((4, H, 64, 64), dtype=torch.float32, device="cuda")
    z = torch.zeros((4, H, 64), dtype=torch.float32, device="cuda")
    o1 = ksm.forward_batch(dev(pre["Q"]), dev(pre["K"]), dev(pre["V"]), cu_seqlens=cu, max_seqlen=max(lens),
                           state=(S, z), slot_ids=ids, write=True, fmap="identity",
                           gate=("gla", dev(pre["g"]), wl.tau), eps=wl.eps).cpu()
    step = {k: torch.cat([f[k][:, :, L:L + m] for f, L in zip(full, lens)], dim=0).contiguous()
            for k in ("Q", "K", "V", "g")}
    o2 = ksm.forward_batch(dev(step["Q"]), dev(step["K"]), dev(step["V"]), state=(S, z), slot_ids=ids, read=True,
                           write=True, fmap="identity", gate=("gla", dev(step["g"]), wl.tau), eps=wl.eps).cpu()
    torch.cuda.synchronize()
    off = 0
    for b, L in enumerate(lens):
        o, sc, _, _ = oracle_ssm(full[b])
        e1 = term_err(o1[:, :, off:off + L], o[:, :, :L], sc[:, :, :L])
        e2 = term_err(o2[b:b + 1], o[:, :, L:], sc[:, :, L:])
        print(f"  ssm batch seq {b}: prefill {e1:.2e} step {e2:.2e}", flush=True)
        assert e1 < TOL_TERMS and e2 < TOL_TERMS
        off += L


# ------------------------------------------------ the selective scalar gate, normalised

SEL_CASES = [(64, 64, 2, 4, 777), (64, 128, 2, 4, 300), (128, 64, 2, 3, 300), (32, 64, 2, 2, 129),
             (128, 128, 1, 2, 200), (64, 64, 4, 16, 1285), (64, 64, 2, 1, 1), (64, 64, 2, 1, 65)]


@pytest.mark.parametrize("d,dv,B,H,n", SEL_CASES)
def test_selective_gate_elu1_parity(d, dv, B, H, n):
    """elu+1 attention under the scalar selective gate (the RetNet decay made
    input-dependent), every built shape, several segments with ragged tails and
    tiny n, every head, to the row-wise tolerance of the bf16 paths."""
    from _helpers import TOL_BF16, check_close, oracle_forward, run_forward
    wl = WORKLOADS["causal_elu1"].resized(d_k=d, d_v=dv, r=d, gate="sel", qk_scale=d ** -0.5, v_scale=dv ** -0.5)
    inp = make_inputs(wl, seed=4, B=B, H=H, n=n)
    out = run_forward(inp)
    ref, _, _ = oracle_forward(inp)
    check_close(out, ref, TOL_BF16, f"elu1 sel d{d}x{dv} B{B} H{H} n{n}")


def test_selective_gate_serving_batch():
    """A ragged prefill under the selective gate through la_forward_batch,
    states into slots, then a one-token step (the decode kernel on the slots)."""
    import kernelized_sequence_mixing_amd as ksm
    from _helpers import TOL_BF16, check_close
    wl = WORKLOADS["causal_elu1"].resized(gate="sel")
    H = 4
    lens = [130, 1, 64, 700]
    full = [make_inputs(wl, seed=80 + b, B=1, H=H, n=L + 1) for b, L in enumerate(lens)]
    pre = {k: torch.cat([f[k][:, :, :L] for f, L in zip(full, lens)], dim=2).contiguous() for k in ("Q", "K", "V", "g")}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    ids = torch.tensor([1, 3, 0, 2], dtype=torch.int32, device="cuda")
    S = torch.zeros((4, H, 64, 64), dtype=torch.float32, device="cuda")
    z = torch.zeros((4, H, 64), dtype=torch.float32, device="cuda")
    o1 = ksm.forward_batch(dev(pre["Q"]), dev(pre["K"]), dev(pre["V"]), cu_seqlens=cu, max_seqlen=max(lens),
                           state=(S, z), slot_ids=ids, write=True, gate=("sel", dev(pre["g"]), wl.tau),
                           eps=wl.eps).cpu()
    step = {k: torch.cat([f[k][:, :, L:L + 1] for f, L in zip(full, lens)], dim=0).contiguous()
            for k in ("Q", "K", "V", "g")}
    o2 = ksm.forward_batch(dev(step["Q"]), dev(step["K"]), dev(step["V"]), state=(S, z), slot_ids=ids, read=True,
                           write=True, gate=("sel", dev(step["g"]), wl.tau), eps=wl.eps).cpu()
    torch.cuda.synchronize()
    off = 0
    for b, L in enumerate(lens):
        f = full[b]
        o = orc.causal_recurrent(to_f64(f["Q"]), to_f64(f["K"]), to_f64(f["V"]), "elu1", None,
                                 ("sel", to_f64(f["g"]), wl.tau), eps=wl.eps)[0]
        check_close(o1[:, :, off:off + L], o[:, :, :L], TOL_BF16, f"sel batch prefill seq {b}")
        check_close(o2[b:b + 1], o[:, :, L:], TOL_BF16, f"sel batch step seq {b}")
        off += L
