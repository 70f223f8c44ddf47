"""GPU parity of the serving batch (la_forward_batch): ragged prefill packed
along n, per-sequence state slots read and written in place, and multi-token
decode steps, against the fp64 oracle run on each sequence alone
(oracle.causal_recurrent with that sequence's carried-in state), and bit for
bit against la_forward where the two plan the same launches.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from workloads import WORKLOADS, make_inputs, to_f64
from _helpers import TOL_BF16, check_close, dev, gpu_gate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _wl(fmap, gate, d, dv):
    if fmap == "favor":
        return WORKLOADS["favor_causal"].resized(gate=gate)
    base = WORKLOADS["gla_gate"] if gate == "gla" else WORKLOADS["causal_elu1"]
    return base.resized(d_k=d, d_v=dv, r=d, gate=gate, qk_scale=d ** -0.5, v_scale=dv ** -0.5)


def _slice(inp, lo, hi, b=0):
    """One sequence's tokens [lo, hi) of batch row b, as an input dict of its own."""
    out = dict(inp)
    for k in ("Q", "K", "V", "g"):
        if k in inp:
            out[k] = inp[k][b:b + 1, :, lo:hi].contiguous()
    out["B"], out["n"] = 1, hi - lo
    return out


def _oracle(inp, S0=None, z0=None):
    """(o, S, z) of the oracle on one sequence (batch row 0)."""
    gate = None
    if inp["gate"] == "decay":
        gate = ("decay", to_f64(inp["gamma"]))
    elif inp["gate"] == "gla":
        gate = ("gla", to_f64(inp["g"]), inp["tau"])
    om = to_f64(inp["omega"]) if inp["fmap"] == "favor" else None
    if inp["n"] == 0:
        return np.zeros((1, inp["Q"].shape[1], 0, inp["V"].shape[3])), S0, z0
    return orc.causal_recurrent(to_f64(inp["Q"]), to_f64(inp["K"]), to_f64(inp["V"]), inp["fmap"], om, gate,
                                eps=inp["eps"], S0=S0, z0=z0)


def _slot_states(wl, n_slots, H, seed):
    """Carried states of a seeded 37-token history per slot (oracle, fp64)."""
    inp = make_inputs(wl, seed=seed, B=n_slots, H=H, n=37)
    S = np.empty((n_slots, H, wl.r, wl.d_v))
    z = np.empty((n_slots, H, wl.r))
    for s in range(n_slots):
        _, S[s:s + 1], z[s:s + 1] = _oracle(_slice(inp, 0, 37, b=s))
    return S, z


def _gpu_gate(inp):
    return gpu_gate(inp)


def _close_state(S, z, Sr, zr, what):
    scale = np.max(np.abs(Sr)) + 1e-30
    err = np.max(np.abs(to_f64(S) - Sr)) / scale
    print(f"  {what}: state err {err:.2e} of its largest entry", flush=True)
    assert err < 2e-2, (what, err)
    np.testing.assert_allclose(to_f64(z), zr, rtol=2e-2)


CASES = [("elu1", "none", 64, 64), ("elu1", "decay", 64, 64), ("elu1", "gla", 64, 64), ("elu1", "decay", 128, 128),
         ("elu1", "none", 64, 128), ("favor", "none", 64, 64), ("favor", "decay", 64, 64)]
LENS = [0, 1, 63, 64, 65, 130, 517, 1300, 200, 17]


@pytest.mark.parametrize("fmap,gate,d,dv", CASES)
def test_ragged_prefill_with_slots(fmap, gate, d, dv):
    """Ten sequences (lengths 0 .. 1300: one token, chunk edges, several
    segments) packed along n with 50 uncovered tokens after them, each
    continuing from its slot and storing its final state there; two sequences
    with slot ids outside the pool (start from zero, store nothing); slots no
    sequence names stay bit for bit."""
    import kernelized_sequence_mixing_amd as ksm
    wl = _wl(fmap, gate, d, dv)
    H = 4
    T = sum(LENS) + 50
    inp = make_inputs(wl, seed=21, B=1, H=H, n=T)
    cu = np.concatenate([[0], np.cumsum(LENS)]).astype(np.int32)
    n_slots = 14
    slot_ids = np.array([5, 0, 11, 3, 7, -1, 9, 2, 13, 14], dtype=np.int32)  # -1 and 14 are outside the pool
    S_init, z_init = _slot_states(wl, n_slots, H, seed=5)
    S = torch.from_numpy(S_init.astype(np.float32)).to("cuda")
    z = torch.from_numpy(z_init.astype(np.float32)).to("cuda")
    S_before, z_before = S.clone(), z.clone()
    out = torch.full((1, H, T, wl.d_v), 7.0, dtype=torch.bfloat16, device="cuda")
    ksm.forward_batch(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), cu_seqlens=torch.from_numpy(cu).to("cuda"),
                      max_seqlen=max(LENS), state=(S, z), slot_ids=torch.from_numpy(slot_ids).to("cuda"),
                      read=True, write=True, fmap=fmap, omega=dev(inp.get("omega")), gate=_gpu_gate(inp),
                      eps=inp["eps"], out=out)
    torch.cuda.synchronize()
    out, S, z = out.cpu(), S.cpu(), z.cpu()
    for b, (lo, hi) in enumerate(zip(cu[:-1], cu[1:])):
        sl = int(slot_ids[b])
        valid = 0 <= sl < n_slots
        S0 = S_init[sl:sl + 1] if valid else None
        z0 = z_init[sl:sl + 1] if valid else None
        o, Sr, zr = _oracle(_slice(inp, lo, hi), S0, z0)
        if hi > lo:
            check_close(out[:, :, lo:hi], o, TOL_BF16, f"{fmap} {gate} seq {b} len {hi - lo} slot {sl}")
        if valid:
            if hi > lo:
                _close_state(S[sl:sl + 1], z[sl:sl + 1], Sr, zr, f"seq {b} slot {sl}")
            else:  # an empty sequence stores its carried-in state unchanged
                assert torch.equal(S[sl], S_before[sl].cpu()) and torch.equal(z[sl], z_before[sl].cpu())
    for sl in set(range(n_slots)) - set(int(x) for x in slot_ids):
        assert torch.equal(S[sl], S_before[sl].cpu()) and torch.equal(z[sl], z_before[sl].cpu()), sl
    assert torch.all(out[:, :, cu[-1]:] == 7.0), "tokens after the last sequence were written"


@pytest.mark.parametrize("gate", ["none", "gla"])
def test_uniform_batch_matches_forward(gate):
    """Without cu_seqlens the launches are la_forward's: outputs and stored
    states equal la_forward's with S0 gathered from the slots, bit for bit."""
    import kernelized_sequence_mixing_amd as ksm
    wl = _wl("elu1", gate, 64, 64)
    B, H, n = 4, 8, 777
    inp = make_inputs(wl, seed=3, B=B, H=H, n=n)
    rng = np.random.default_rng(1)
    S_pool = torch.from_numpy(rng.standard_normal((5, H, 64, 64)).astype(np.float32)).to("cuda")
    z_pool = torch.from_numpy((20.0 + rng.random((5, H, 64))).astype(np.float32)).to("cuda")
    ids = torch.tensor([2, 0, 4, 1], dtype=torch.int32, device="cuda")
    S0, z0 = S_pool[ids.long()].contiguous(), z_pool[ids.long()].contiguous()
    ref, Sf, zf = ksm.forward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), gate=_gpu_gate(inp), eps=inp["eps"],
                              S0=S0, z0=z0, return_state=True)
    untouched = S_pool[3].clone()
    got = ksm.forward_batch(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), state=(S_pool, z_pool), slot_ids=ids,
                            read=True, write=True, gate=_gpu_gate(inp), eps=inp["eps"])
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(S_pool[ids.long()], Sf) and torch.equal(z_pool[ids.long()], zf)
    assert torch.equal(S_pool[3], untouched)


@pytest.mark.parametrize("gate", ["none", "gla"])
def test_one_token_steps_with_slots(gate):
    """One token per sequence runs the recurrent step kernel on the slots:
    states equal la_decode_step's on the gathered states bit for bit, slots
    of other sequences and the one with an id outside the pool stay as they
    were, and outputs follow the oracle's recurrence."""
    import kernelized_sequence_mixing_amd as ksm
    wl = _wl("elu1", gate, 128, 128)
    B, H = 6, 4
    inp = make_inputs(wl, seed=8, B=B, H=H, n=1)
    S_init, z_init = _slot_states(wl, 9, H, seed=6)
    S = torch.from_numpy(S_init.astype(np.float32)).to("cuda")
    z = torch.from_numpy(z_init.astype(np.float32)).to("cuda")
    ids_np = np.array([4, 0, 8, 2, 11, 6], dtype=np.int32)   # 11 is outside the pool of 9
    ids = torch.from_numpy(ids_np).to("cuda")
    valid = torch.from_numpy(ids_np[ids_np < 9].astype(np.int64)).to("cuda")
    rows = torch.from_numpy(np.nonzero(ids_np < 9)[0]).to("cuda")
    S_ref, z_ref = S[valid].clone(), z[valid].clone()
    before_S, before_z = S.clone(), z.clone()
    out = ksm.forward_batch(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), state=(S, z), slot_ids=ids, read=True,
                            write=True, gate=_gpu_gate(inp), eps=inp["eps"])
    g1 = None
    if gate == "gla":
        g1 = ("gla", dev(inp["g"])[rows, :, 0].contiguous(), wl.tau)
    ksm.decode_step(S_ref, z_ref, dev(inp["Q"])[rows, :, 0].contiguous(), dev(inp["K"])[rows, :, 0].contiguous(),
                    dev(inp["V"])[rows, :, 0].contiguous(), gate=g1, eps=inp["eps"])
    torch.cuda.synchronize()
    assert torch.equal(S[valid], S_ref) and torch.equal(z[valid], z_ref)
    for sl in (1, 3, 5, 7):
        assert torch.equal(S[sl], before_S[sl]) and torch.equal(z[sl], before_z[sl])
    out = out.cpu()
    for b in range(B):
        sl = int(ids_np[b])
        ok = sl < 9
        o, _, _ = _oracle(_slice(inp, 0, 1, b=b), S_init[sl:sl + 1] if ok else None, z_init[sl:sl + 1] if ok else None)
        check_close(out[b:b + 1], o, TOL_BF16, f"{gate} one-token seq {b} slot {sl}")


@pytest.mark.parametrize("gate", ["decay", "gla"])
def test_prefill_then_multi_token_decode(gate):
    """A ragged prefill that stores states, then three steps of four new tokens
    per sequence (uniform batch, read and write in place), equal the oracle on
    each whole sequence; the slots end at the oracle's final states."""
    import kernelized_sequence_mixing_amd as ksm
    wl = _wl("elu1", gate, 64, 64)
    H, m, steps = 4, 4, 3
    lens = [100, 3, 64, 250, 1, 77]
    B = len(lens)
    full = [make_inputs(wl, seed=40 + b, B=1, H=H, n=L + m * steps) for b, L in enumerate(lens)]
    # the prefill tokens packed along n
    pre = {k: torch.cat([f[k][:, :, :L] for f, L in zip(full, lens)], dim=2).contiguous()
           for k in ("Q", "K", "V", "g") if k in full[0]}
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    ids = torch.tensor([3, 1, 6, 0, 5, 2], dtype=torch.int32, device="cuda")
    S = torch.zeros((8, H, 64, 64), dtype=torch.float32, device="cuda")
    z = torch.zeros((8, H, 64), dtype=torch.float32, device="cuda")

    def gate_of(d):
        if gate == "decay":
            return ("decay", dev(full[0]["gamma"]))
        return ("gla", dev(d["g"]), wl.tau)
    out_pre = ksm.forward_batch(dev(pre["Q"]), dev(pre["K"]), dev(pre["V"]), cu_seqlens=cu, max_seqlen=max(lens),
                                state=(S, z), slot_ids=ids, write=True, gate=gate_of(pre), eps=wl.eps).cpu()
    outs = []
    for st in range(steps):
        lo = [L + m * st for L in lens]
        step = {k: torch.cat([f[k][:, :, a:a + m] for f, a in zip(full, lo)], dim=0).contiguous()
                for k in ("Q", "K", "V", "g") if k in full[0]}
        outs.append(ksm.forward_batch(dev(step["Q"]), dev(step["K"]), dev(step["V"]), state=(S, z), slot_ids=ids,
                                      read=True, write=True, gate=gate_of(step), eps=wl.eps).cpu())
    torch.cuda.synchronize()
    off = 0
    for b, L in enumerate(lens):
        o, Sr, zr = _oracle(full[b])
        check_close(out_pre[:, :, off:off + L], o[:, :, :L], TOL_BF16, f"{gate} prefill seq {b}")
        for st in range(steps):
            check_close(outs[st][b:b + 1], o[:, :, L + m * st:L + m * (st + 1)], TOL_BF16,
                        f"{gate} step {st} seq {b}")
        sl = int(ids[b])
        _close_state(S[sl:sl + 1].cpu(), z[sl:sl + 1].cpu(), Sr, zr, f"{gate} seq {b} final")
        off += L


# ------------------------------------------------ the benchmark's serving configurations

def test_serving_prefill_bench_config_sampled():
    """The ragged prefill bench.py times (32 sequences, seeded log-uniform
    lengths 64 .. 8192, H16 d64 elu+1, states into slots): the shortest, the
    longest and the last sequence on two heads against the oracle, with their
    stored states."""
    import kernelized_sequence_mixing_amd as ksm
    from workloads import serving_lengths
    lens = serving_lengths(32, seed=7)
    T, H = int(lens.sum()), 16
    wl = WORKLOADS["causal_elu1"].resized(name="serve_prefill", B=1, H=H, n=T, d_k=64, d_v=64, r=64)
    inp = make_inputs(wl, seed=0)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S = torch.zeros((32, H, 64, 64), dtype=torch.float32, device="cuda")
    z = torch.zeros((32, H, 64), dtype=torch.float32, device="cuda")
    out = ksm.forward_batch(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), cu_seqlens=torch.from_numpy(cu).cuda(),
                            max_seqlen=int(lens.max()), state=(S, z),
                            slot_ids=torch.arange(32, dtype=torch.int32, device="cuda"), write=True,
                            eps=wl.eps).cpu()
    torch.cuda.synchronize()
    Sc, zc = S.cpu(), z.cpu()
    for b in sorted({int(np.argmin(lens)), int(np.argmax(lens)), 31}):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for h in (0, H - 1):
            Q, K, V = (to_f64(inp[k])[:, h:h + 1, lo:hi] for k in ("Q", "K", "V"))
            o, Sr, zr = orc.causal_recurrent(Q, K, V, "elu1", None, None, eps=wl.eps)
            check_close(out[:, h:h + 1, lo:hi], o, TOL_BF16, f"serve prefill seq {b} (len {hi - lo}) head {h}")
            assert np.max(np.abs(to_f64(Sc[b, h]) - Sr[0, 0])) / np.max(np.abs(Sr)) < 1e-2
            assert np.max(np.abs(to_f64(zc[b, h]) - zr[0, 0]) / zr[0, 0]) < 1e-2


@pytest.mark.parametrize("m", [1, 4])
def test_serving_decode_bench_config_sampled(m):
    """The decode steps bench.py times (B256 H16, 128 x 128 GLA states read
    and written in their slots, m tokens per sequence): sampled sequences on
    every head against the oracle's steps from the same states."""
    import kernelized_sequence_mixing_amd as ksm
    dwl = WORKLOADS["gla_decode"]
    B, H = dwl.B, dwl.H
    base = WORKLOADS["gla_gate"].resized(B=B, H=H, n=m)
    inp = make_inputs(base, seed=0)
    dec = make_inputs(dwl, seed=0)
    S, z = dev(dec["S0"]), dev(dec["z0"])
    out = ksm.forward_batch(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), state=(S, z),
                            slot_ids=torch.arange(B, dtype=torch.int32, device="cuda"), read=True, write=True,
                            gate=("gla", dev(inp["g"]), dwl.tau), eps=dwl.eps).cpu()
    torch.cuda.synchronize()
    Sc = S.cpu()
    for b in (0, 97, B - 1):
        sl = lambda x: to_f64(x)[b:b + 1]
        o, Sr, _ = orc.causal_recurrent(sl(inp["Q"]), sl(inp["K"]), sl(inp["V"]), "elu1", None,
                                        ("gla", sl(inp["g"]), dwl.tau), eps=dwl.eps, S0=sl(dec["S0"]),
                                        z0=sl(dec["z0"]))
        check_close(out[b:b + 1], o, TOL_BF16, f"serve decode m{m} seq {b}")
        assert np.max(np.abs(to_f64(Sc[b]) - Sr[0])) / np.max(np.abs(Sr)) < 1e-2


# ------------------------------------------------ short steps on the recurrent step kernel

def _step_wl(fmap, gate, d, dv, r=None):
    if fmap == "favor":
        return WORKLOADS["favor_causal"].resized(gate=gate, d_v=dv, r=r or 256)
    if fmap == "identity":
        return WORKLOADS["ssm_selective"].resized(gate=gate, d_k=d, d_v=dv, r=d)
    base = WORKLOADS["outer_gate"] if gate == "outer" else WORKLOADS["gla_gate"]
    return base.resized(gate=gate, d_k=d, d_v=dv, r=d, qk_scale=d ** -0.5, v_scale=dv ** -0.5)


def _token_gate(inp, t, rows):
    kind = inp["gate"]
    if kind == "decay":
        return ("decay", dev(inp["gamma"]))
    if kind in ("gla", "sel"):
        return (kind, dev(inp["g"])[rows, :, t].contiguous(), inp["tau"])
    if kind == "outer":
        return ("outer", dev(inp["g"])[rows, :, t].contiguous(), dev(inp["gv"])[rows, :, t].contiguous(), inp["tau"])
    return None


def _oracle_gate_row(inp, b):
    kind = inp["gate"]
    if kind == "decay":
        return ("decay", to_f64(inp["gamma"]))
    if kind in ("gla", "sel"):
        return (kind, to_f64(inp["g"])[b:b + 1], inp["tau"])
    if kind == "outer":
        return ("outer", to_f64(inp["g"])[b:b + 1], to_f64(inp["gv"])[b:b + 1], inp["tau"])
    return None


STEP_CASES = [("elu1", "none", 64, 64, None, 2), ("elu1", "decay", 64, 64, None, 5),
              ("elu1", "gla", 128, 128, None, 16), ("elu1", "sel", 64, 64, None, 7),
              ("elu1", "outer", 64, 64, None, 4), ("favor", "none", 64, 64, None, 3),
              ("favor", "decay", 64, 64, 32, 16), ("identity", "gla", 64, 64, None, 6),
              ("elu1", "none", 64, 32, None, 4), ("elu1", "gla", 32, 64, None, 9)]


@pytest.mark.parametrize("fmap,gate,d,dv,r,m", STEP_CASES)
def test_short_steps_equal_successive_decode_steps(fmap, gate, d, dv, r, m):
    """A batch step of m <= 16 tokens per sequence (no cu_seqlens) runs the
    recurrent step kernel over its tokens with the state held in registers:
    outputs and stored states equal m successive la_decode_step calls on the
    gathered states bit for bit, a slot id outside the pool starts from zero
    and stores nothing, other slots stay as they were, and the outputs follow
    the oracle's recurrence. Includes d_v = 32 and FAVOR+ r = 32, which only
    such steps take."""
    import kernelized_sequence_mixing_amd as ksm
    wl = _step_wl(fmap, gate, d, dv, r)
    B, H, n_slots = 5, 3, 7
    inp = make_inputs(wl, seed=60 + m, B=B, H=H, n=m)
    rng = np.random.default_rng(61 + m)
    S_init = rng.standard_normal((n_slots, H, wl.r, wl.d_v)).astype(np.float32)
    z_init = (20.0 + rng.random((n_slots, H, wl.r))).astype(np.float32)
    S, z = torch.from_numpy(S_init).to("cuda"), torch.from_numpy(z_init).to("cuda")
    ids_np = np.array([3, 0, 6, 9, 1], dtype=np.int32)  # 9 is outside the pool
    ids = torch.from_numpy(ids_np).to("cuda")
    before_S, before_z = S.clone(), z.clone()
    om = dev(inp.get("omega"))
    out = ksm.forward_batch(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), state=(S, z), slot_ids=ids, read=True,
                            write=True, fmap=fmap, omega=om, gate=gpu_gate(inp), eps=inp["eps"])
    # the same tokens as m successive decode steps on copies of the states (a zero state for slot 9)
    rows = torch.arange(B, device="cuda")
    S_ref = torch.stack([S_init_t if ok else torch.zeros_like(S_init_t) for S_init_t, ok in
                         zip(before_S[torch.from_numpy(np.minimum(ids_np, n_slots - 1).astype(np.int64)).to("cuda")],
                             ids_np < n_slots)]).contiguous()
    z_ref = torch.stack([z_t if ok else torch.zeros_like(z_t) for z_t, ok in
                         zip(before_z[torch.from_numpy(np.minimum(ids_np, n_slots - 1).astype(np.int64)).to("cuda")],
                             ids_np < n_slots)]).contiguous()
    refs = []
    for t in range(m):
        refs.append(ksm.decode_step(S_ref, z_ref, dev(inp["Q"])[:, :, t].contiguous(),
                                    dev(inp["K"])[:, :, t].contiguous(), dev(inp["V"])[:, :, t].contiguous(),
                                    fmap=fmap, omega=om, gate=_token_gate(inp, t, rows), eps=inp["eps"],
                                    out_dtype=out.dtype))
    torch.cuda.synchronize()
    assert torch.equal(out, torch.stack(refs, dim=2)), f"{fmap} {gate} m{m}: outputs differ from the decode steps"
    for b, sl in enumerate(ids_np):
        if sl < n_slots:
            assert torch.equal(S[sl], S_ref[b]) and torch.equal(z[sl], z_ref[b])
    for sl in (2, 4, 5):
        assert torch.equal(S[sl], before_S[sl]) and torch.equal(z[sl], before_z[sl])
    oc = out.cpu()
    for b in (0, 3):
        sl = int(ids_np[b])
        ok = sl < n_slots
        o, _, _ = orc.causal_recurrent(to_f64(inp["Q"])[b:b + 1], to_f64(inp["K"])[b:b + 1],
                                       to_f64(inp["V"])[b:b + 1], fmap,
                                       to_f64(inp["omega"]) if fmap == "favor" else None, _oracle_gate_row(inp, b),
                                       eps=inp["eps"], S0=S_init[sl:sl + 1] if ok else None,
                                       z0=z_init[sl:sl + 1] if ok else None)
        tol = TOL_BF16 if fmap != "identity" else 2e-2
        check_close(oc[b:b + 1], o, tol, f"{fmap} {gate} d{d} dv{dv} m{m} seq {b} slot {sl}")
