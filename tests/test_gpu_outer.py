"""GPU parity of the outer-product gate G_t = alpha_t beta_t^T (key side alpha
as the GLA gate, value side beta per value column; z takes the key side
only) against the fp64 oracle: elu+1 attention to the row-wise tolerance of
the bf16 paths, the state-space form to the term-relative tolerance of
test_gpu_ssm.py, the decode step, and the serving batch.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from workloads import WORKLOADS, make_inputs, to_f64
from _helpers import TOL_BF16, check_close, dev, gpu_gate, oracle_forward, run_forward
import test_gpu_ssm as tssm

pytestmark = pytest.mark.gpu

SEQ = ("Q", "K", "V", "g", "gv")  # per-token inputs


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _elu_case(d, dv, B, H, n, seed=4):
    wl = WORKLOADS["causal_elu1"].resized(d_k=d, d_v=dv, r=d, gate="outer", qk_scale=d ** -0.5, v_scale=dv ** -0.5)
    return wl, make_inputs(wl, seed=seed, B=B, H=H, n=n)


def _ssm_case(d, dv, B, H, n, seed=2):
    wl = WORKLOADS["ssm_selective"].resized(d_k=d, d_v=dv, r=d, gate="outer", qk_scale=d ** -0.5)
    return wl, make_inputs(wl, seed=seed, B=B, H=H, n=n)


def _oracle_ssm(inp, S0=None, z0=None):
    """(o, scale, S, z) of the state-space form under the outer-product gate;
    scale is the oracle recurrence on |q|, |k|, |v| (the gate factors are positive)."""
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    gate = ("outer", to_f64(inp["g"]), to_f64(inp["gv"]), inp["tau"])
    o, S, z = orc.causal_recurrent(Q, K, V, "identity", None, gate, eps=inp["eps"], S0=S0, z0=z0)
    sc = orc.causal_recurrent(np.abs(Q), np.abs(K), np.abs(V), "identity", None, gate,
                              S0=None if S0 is None else np.abs(S0), z0=z0)[0]
    return o, sc, S, z


CASES = [(64, 64, 2, 4, 777), (64, 128, 2, 4, 300), (128, 64, 2, 3, 300), (32, 64, 2, 2, 129),
         (128, 128, 1, 2, 200), (64, 64, 4, 16, 1285), (64, 64, 2, 1, 1), (64, 64, 2, 1, 65)]


@pytest.mark.parametrize("d,dv,B,H,n", CASES)
def test_outer_gate_elu1_parity(d, dv, B, H, n):
    """Every built shape, one-chunk and three-chunk segments with ragged tails,
    one segment, n 1 and 65, every head."""
    wl, inp = _elu_case(d, dv, B, H, n)
    out, S, z = run_forward(inp, return_state=True)
    ref, Sr, zr = oracle_forward(inp)
    check_close(out, ref, TOL_BF16, f"elu1 outer d{d}x{dv} B{B} H{H} n{n}")
    # the final state: z takes the key side only, S both
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 1e-2
    assert np.max(np.abs(to_f64(z) - zr) / (np.abs(zr) + 1e-30)) < 1e-2


@pytest.mark.parametrize("d,dv,B,H,n", [c for c in CASES if c[4] > 1])
def test_outer_gate_ssm_parity(d, dv, B, H, n):
    """The state-space form (identity features, no normaliser) under the
    outer-product gate, term-relative."""
    wl, inp = _ssm_case(d, dv, B, H, n)
    got = tssm.run(inp)
    o, sc, _, _ = _oracle_ssm(inp)
    e = tssm.term_err(got, o, sc)
    print(f"  ssm outer d{d}x{dv} B{B} H{H} n{n}: term-relative err {e:.2e}", flush=True)
    assert e < tssm.TOL_TERMS


def test_outer_gate_resumes_from_state():
    """A carried-in state (the oracle's after a 150-token prefix): the
    continuation equals one pass over the whole sequence."""
    wl, inp = _elu_case(64, 64, 2, 4, 700, seed=6)
    m = 150
    first = {k: (v[:, :, :m].contiguous() if k in SEQ else v) for k, v in inp.items()}
    second = {k: (v[:, :, m:].contiguous() if k in SEQ else v) for k, v in inp.items()}
    _, S1, z1 = oracle_forward(first)
    ref, Sr, _ = oracle_forward(second, S0=S1, z0=z1)
    out, S, _ = run_forward(second, return_state=True, S0=torch.from_numpy(S1.astype(np.float32)),
                            z0=torch.from_numpy(z1.astype(np.float32)))
    check_close(out, ref, TOL_BF16, "elu1 outer resumed")
    assert np.max(np.abs(to_f64(S) - Sr)) / (np.max(np.abs(Sr)) + 1e-30) < 1e-2


@pytest.mark.parametrize("fmap", ["elu1", "identity"])
def test_outer_gate_decode_step(fmap):
    """One recurrent step from a carried state (fp32 arithmetic)."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["gla_decode"].resized(fmap=fmap, gate="outer", B=8, H=4)
    inp = make_inputs(wl, seed=3)
    S, z = dev(inp["S0"]), dev(inp["z0"])
    out = ksm.decode_step(S, z, dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), fmap=fmap,
                          gate=("outer", dev(inp["g"]), dev(inp["gv"]), wl.tau), eps=wl.eps)
    torch.cuda.synchronize()
    og = ("outer", to_f64(inp["g"]), to_f64(inp["gv"]), wl.tau)
    o, S1, z1 = orc.decode_step(to_f64(inp["S0"]), to_f64(inp["z0"]), to_f64(inp["q"]), to_f64(inp["k"]),
                                to_f64(inp["v"]), fmap, None, og, eps=wl.eps)
    got = to_f64(out.cpu())
    e = float(np.max(np.abs(got - o)) / np.max(np.abs(o)))
    print(f"  decode outer {fmap}: err {e:.2e}", flush=True)
    assert e < 1e-4
    np.testing.assert_allclose(to_f64(S), S1, rtol=1e-5, atol=1e-4)
    np.testing.assert_allclose(to_f64(z), z1, rtol=1e-5, atol=1e-5)


def test_outer_gate_serving_batch():
    """A ragged prefill through la_forward_batch, states into slots, then a
    one-token step (the decode kernel on the slots)."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["causal_elu1"].resized(gate="outer")
    H = 4
    lens = [130, 1, 64, 700]
    full = [make_inputs(wl, seed=90 + b, B=1, H=H, n=L + 1) for b, L in enumerate(lens)]
    pre = {k: torch.cat([f[k][:, :, :L] for f, L in zip(full, lens)], dim=2).contiguous() for k in SEQ}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    ids = torch.tensor([1, 3, 0, 2], dtype=torch.int32, device="cuda")
    S = torch.zeros((4, H, 64, 64), dtype=torch.float32, device="cuda")
    z = torch.zeros((4, H, 64), dtype=torch.float32, device="cuda")
    o1 = ksm.forward_batch(dev(pre["Q"]), dev(pre["K"]), dev(pre["V"]), cu_seqlens=cu, max_seqlen=max(lens),
                           state=(S, z), slot_ids=ids, write=True,
                           gate=("outer", dev(pre["g"]), dev(pre["gv"]), wl.tau), eps=wl.eps).cpu()
    step = {k: torch.cat([f[k][:, :, L:L + 1] for f, L in zip(full, lens)], dim=0).contiguous() for k in SEQ}
    o2 = ksm.forward_batch(dev(step["Q"]), dev(step["K"]), dev(step["V"]), state=(S, z), slot_ids=ids, read=True,
                           write=True, gate=("outer", dev(step["g"]), dev(step["gv"]), wl.tau), eps=wl.eps).cpu()
    torch.cuda.synchronize()
    off = 0
    for b, L in enumerate(lens):
        f = full[b]
        o = orc.causal_recurrent(to_f64(f["Q"]), to_f64(f["K"]), to_f64(f["V"]), "elu1", None,
                                 ("outer", to_f64(f["g"]), to_f64(f["gv"]), wl.tau), eps=wl.eps)[0]
        check_close(o1[:, :, off:off + L], o[:, :, :L], TOL_BF16, f"outer batch prefill seq {b}")
        check_close(o2[b:b + 1], o[:, :, L:], TOL_BF16, f"outer batch step seq {b}")
        off += L


def test_outer_gate_full_size_sampled_heads():
    """The benchmark's outer-gate shape (B2 H16 n16384 d128, several segments),
    two heads against the oracle's recurrence."""
    wl = WORKLOADS["outer_gate"]
    inp = make_inputs(wl, seed=0)
    out = run_forward(inp)
    assert torch.isfinite(out.float()).all()
    for head in [(0, 0), (wl.B - 1, wl.H - 1)]:
        ref, _, _ = oracle_forward(inp, head=head)
        b, h = head
        check_close(out[b:b + 1, h:h + 1], ref, TOL_BF16, f"outer full size head {head}")


def test_outer_gate_deterministic():
    wl, inp = _elu_case(64, 64, 4, 16, 1285, seed=8)
    a = run_forward(inp, return_state=True)
    b = run_forward(inp, return_state=True)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
