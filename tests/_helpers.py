"""Shared pieces of the GPU tests: moving seeded inputs to the device, calling
the library through its C ABI, and computing the oracle on the same values."""
from __future__ import annotations

import numpy as np
import torch

import oracle as orc
from workloads import to_f64

TOL_F32 = 1e-4   # fp32 inputs, fp32 arithmetic and output
TOL_BF16 = 1e-2  # bf16 inputs, bf16 MFMA operands, fp32 accumulation and state


def dev(t):
    return None if t is None else t.to("cuda").contiguous()


def gpu_gate(inp):
    kind = inp["gate"]
    if kind == "decay":
        return ("decay", dev(inp["gamma"]))
    if kind in ("gla", "sel"):
        return (kind, dev(inp["g"]), inp["tau"])
    if kind == "outer":
        return ("outer", dev(inp["g"]), dev(inp["gv"]), inp["tau"])
    return None


def oracle_gate(inp, heads=None, t_slice=None):
    kind = inp["gate"]
    if kind == "decay":
        gam = to_f64(inp["gamma"])
        return ("decay", gam)
    if kind in ("gla", "sel"):
        g = to_f64(inp["g"])
        if heads is not None:
            g = g[heads[0]:heads[0] + 1, heads[1]:heads[1] + 1]
        if t_slice is not None:
            g = g[:, :, t_slice]
        return (kind, g, inp["tau"])
    if kind == "outer":
        g, gv = to_f64(inp["g"]), to_f64(inp["gv"])
        if heads is not None:
            g, gv = (x[heads[0]:heads[0] + 1, heads[1]:heads[1] + 1] for x in (g, gv))
        if t_slice is not None:
            g, gv = g[:, :, t_slice], gv[:, :, t_slice]
        return ("outer", g, gv, inp["tau"])
    return None


def run_forward(inp, return_state=False, out_dtype=None, S0=None, z0=None, eps=None):
    import kernelized_sequence_mixing_amd as ksm
    res = ksm.forward(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), fmap=inp["fmap"], omega=dev(inp.get("omega")),
                      causal=inp["causal"], gate=gpu_gate(inp), eps=inp["eps"] if eps is None else eps,
                      S0=dev(S0), z0=dev(z0), return_state=return_state, out_dtype=out_dtype)
    torch.cuda.synchronize()
    if return_state:
        return tuple(x.cpu() for x in res)
    return res.cpu()


def oracle_forward(inp, head=None, eps=None, S0=None, z0=None):
    """fp64 oracle output, for every head or for one (b, h) (shape kept 4-D)."""
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    gate = oracle_gate(inp)
    if head is not None:
        b, h = head
        Q, K, V = (x[b:b + 1, h:h + 1] for x in (Q, K, V))
        if gate is not None and gate[0] in ("gla", "sel"):
            gate = (gate[0], gate[1][b:b + 1, h:h + 1], gate[2])
        if gate is not None and gate[0] == "outer":
            gate = ("outer", gate[1][b:b + 1, h:h + 1], gate[2][b:b + 1, h:h + 1], gate[3])
        if gate is not None and gate[0] == "decay":
            gate = ("decay", gate[1][h:h + 1])
    om = to_f64(inp["omega"]) if inp["fmap"] == "favor" else None
    e = inp["eps"] if eps is None else eps
    if not inp["causal"]:
        return orc.noncausal(Q, K, V, inp["fmap"], om, eps=e), None, None
    return orc.causal_recurrent(Q, K, V, inp["fmap"], om, gate, eps=e, S0=S0, z0=z0)


def tol_for(inp):
    return TOL_F32 if inp["dtype"] == "f32" else TOL_BF16


def check_close(got, ref, tol, what=""):
    err = orc.rowwise_rel_err(to_f64(got), ref)
    print(f"  {what}: rowwise rel err {err:.3e} (tol {tol:g})", flush=True)
    assert np.isfinite(err) and err <= tol, f"{what}: {err} > {tol}"
    return err
