"""Python entry points over the C ABI (argument marshalling only).

Torch supplies device memory and the current stream; every step of the
computation runs in the HIP kernels of liblinattn.so. Shapes are read from the
tensors and cross-checked here, because the C ABI receives only pointers and
sizes.
"""
from __future__ import annotations

import ctypes

import torch

from . import _native as N

_DT = {torch.float32: N.LA_F32, torch.bfloat16: N.LA_BF16}
_FMAP = {"elu1": N.LA_FMAP_ELU1, "favor": N.LA_FMAP_FAVOR, "identity": N.LA_FMAP_IDENTITY}


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")
    return _DT[t.dtype]


def _dev(t: torch.Tensor, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor, stream=None):
    s = torch.cuda.current_stream(t.device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _same_dtype(t, in_dtype, name):
    """The C ABI reads g, gv and omega with the element size of the input dtype,
    so a tensor of another dtype would be misread (or read past its end)."""
    if in_dtype is not None and isinstance(t, torch.Tensor) and t.dtype != in_dtype:
        raise TypeError(f"{name} must have the input dtype {in_dtype}, got {t.dtype}")


def _fmap_struct(fmap: str, omega, d_k: int, in_dtype=None):
    if fmap not in _FMAP:
        raise ValueError(f"unknown feature map {fmap!r}")
    if fmap == "favor":
        if omega is None:
            raise ValueError("favor needs omega [r, d_k]")
        _same_dtype(omega, in_dtype, "omega")
        _dev(omega, "omega")
        if omega.dim() != 2 or omega.shape[1] != d_k:
            raise ValueError(f"omega must be [r, {d_k}], got {tuple(omega.shape)}")
        return N.LaFeatureMap(N.LA_FMAP_FAVOR, omega.shape[0], omega.data_ptr()), omega.shape[0]
    if omega is not None:
        raise ValueError(f"{fmap} takes no omega")
    return N.LaFeatureMap(_FMAP[fmap], d_k, None), d_k


def _gate_struct(gate, expect_g_shape, d_v=None, in_dtype=None):
    """gate: None | ("decay", gamma[H] fp32) | ("gla", g, tau) | ("sel", g, tau) |
    ("outer", g, gv, tau); g has shape expect_g_shape for GLA and the outer-product gate,
    and expect_g_shape without its last (feature) axis for the selective scalar gate; gv
    (the outer-product gate's value side) has d_v on that last axis. g and gv must have
    the input dtype in_dtype (checked before anything else)."""
    if gate is None or gate == "none" or (isinstance(gate, tuple) and gate[0] == "none"):
        return N.LaGate(N.LA_GATE_NONE, 1.0, None, None)
    kind = gate[0]
    if kind in ("gla", "sel"):
        _same_dtype(gate[1], in_dtype, "g")
    if kind == "outer":
        _same_dtype(gate[1], in_dtype, "g")
        _same_dtype(gate[2], in_dtype, "gv")
    if kind == "decay":
        gam = _dev(gate[1], "gamma")
        if gam.dtype != torch.float32 or gam.shape != (expect_g_shape[1],):
            raise ValueError("gamma must be float32 [H]")
        return N.LaGate(N.LA_GATE_DECAY, 1.0, gam.data_ptr(), None)
    if kind == "gla":
        g = _dev(gate[1], "g")
        if tuple(g.shape) != tuple(expect_g_shape):
            raise ValueError(f"g must be {tuple(expect_g_shape)}, got {tuple(g.shape)}")
        return N.LaGate(N.LA_GATE_GLA, float(gate[2]), None, g.data_ptr())
    if kind == "sel":
        g = _dev(gate[1], "g")
        if tuple(g.shape) != tuple(expect_g_shape[:-1]):
            raise ValueError(f"g must be {tuple(expect_g_shape[:-1])}, got {tuple(g.shape)}")
        return N.LaGate(N.LA_GATE_SEL, float(gate[2]), None, g.data_ptr())
    if kind == "outer":
        g, gv = _dev(gate[1], "g"), _dev(gate[2], "gv")
        want_v = tuple(expect_g_shape[:-1]) + (d_v,)
        if tuple(g.shape) != tuple(expect_g_shape) or tuple(gv.shape) != want_v:
            raise ValueError(f"g must be {tuple(expect_g_shape)} and gv {want_v}, got {tuple(g.shape)}, "
                             f"{tuple(gv.shape)}")
        if gv.dtype != g.dtype:
            raise TypeError("g and gv must share a dtype")
        return N.LaGate(N.LA_GATE_OUTER, float(gate[3]), None, g.data_ptr(), gv.data_ptr())
    raise ValueError(f"unknown gate {kind!r}")


def _problem(B, H, n, d_k, d_v, in_dt, out_dt, eps):
    return N.LaProblem(B, H, n, d_k, d_v, in_dt, out_dt, float(eps))


def workspace_size(B, H, n, d_k, d_v, *, fmap="elu1", r=None, causal=True, gate_kind="none",
                   dtype=torch.bfloat16, out_dtype=None) -> int:
    """Workspace bytes la_forward needs (host arithmetic only)."""
    r = d_k if r is None else r
    out_dtype = dtype if out_dtype is None else out_dtype
    p = _problem(B, H, n, d_k, d_v, _DT[dtype], _DT[out_dtype], 1e-6)
    f = N.LaFeatureMap(_FMAP[fmap], r, 16 if fmap == "favor" else None)
    gk = {"none": N.LA_GATE_NONE, "decay": N.LA_GATE_DECAY, "gla": N.LA_GATE_GLA, "sel": N.LA_GATE_SEL,
          "outer": N.LA_GATE_OUTER}[gate_kind]
    g = N.LaGate(gk, 16.0, None, None)
    out = ctypes.c_size_t(0)
    N.check(N.lib().la_forward_workspace_size(ctypes.byref(p), ctypes.byref(f), int(causal), ctypes.byref(g),
                                              ctypes.byref(out)), "la_forward_workspace_size")
    return out.value


def segments(B, H, n, d_k, d_v, *, fmap="elu1", r=None, causal=True, gate_kind="none",
             dtype=torch.bfloat16):
    """(segments, segment_len) of the causal sequence split (host arithmetic only)."""
    r = d_k if r is None else r
    p = _problem(B, H, n, d_k, d_v, _DT[dtype], _DT[dtype], 1e-6)
    f = N.LaFeatureMap(_FMAP[fmap], r, 16 if fmap == "favor" else None)
    gk = {"none": N.LA_GATE_NONE, "decay": N.LA_GATE_DECAY, "gla": N.LA_GATE_GLA, "sel": N.LA_GATE_SEL,
          "outer": N.LA_GATE_OUTER}[gate_kind]
    g = N.LaGate(gk, 16.0, None, None)
    P, L = ctypes.c_int32(0), ctypes.c_int32(0)
    N.check(N.lib().la_forward_segments(ctypes.byref(p), ctypes.byref(f), int(causal), ctypes.byref(g),
                                        ctypes.byref(P), ctypes.byref(L)), "la_forward_segments")
    return P.value, L.value


def _forward_args(Q, K, V, fmap, omega, causal, gate, eps, S0, z0, return_state, out_dtype, out, workspace, stream,
                  noalloc=False):
    """Validate and marshal one la_forward call: (ctypes argument tuple, keep-alive objects, out, S_final, z_final).
    noalloc: the arguments of la_forward_noalloc instead (no workspace)."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, nm)
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError(f"shapes Q{tuple(Q.shape)} K{tuple(K.shape)} V{tuple(V.shape)} do not match")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K, V must share a dtype")
    B, H, n, d_k = Q.shape
    d_v = V.shape[3]
    in_dt = _dt(Q)
    out_dtype = Q.dtype if out_dtype is None else out_dtype
    f, r = _fmap_struct(fmap, omega, d_k, Q.dtype)
    g = _gate_struct(gate, (B, H, n, r), d_v, Q.dtype)
    p = _problem(B, H, n, d_k, d_v, in_dt, _DT[out_dtype], eps)
    if out is None:
        out = torch.empty((B, H, n, d_v), dtype=out_dtype, device=Q.device)
    else:
        _dev(out, "out")
        if tuple(out.shape) != (B, H, n, d_v) or out.dtype != out_dtype:
            raise ValueError("out has the wrong shape or dtype")
    for t, nm, shp in ((S0, "S0", (B, H, r, d_v)), (z0, "z0", (B, H, r))):
        if t is not None:
            _dev(t, nm)
            if tuple(t.shape) != shp or t.dtype != torch.float32:
                raise ValueError(f"{nm} must be float32 {shp}")
    Sf = zf = None
    if return_state:
        Sf = torch.empty((B, H, r, d_v), dtype=torch.float32, device=Q.device)
        zf = torch.empty((B, H, r), dtype=torch.float32, device=Q.device)
    if noalloc:
        args = (ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(f), int(bool(causal)), ctypes.byref(g),
                _ptr(S0), _ptr(z0), _ptr(Sf), _ptr(zf), _ptr(out), _stream(Q, stream))
        return args, (p, f, g, Q, K, V, omega, gate, S0, z0), out, Sf, zf
    ws_bytes = ctypes.c_size_t(0)
    N.check(N.lib().la_forward_workspace_size(ctypes.byref(p), ctypes.byref(f), int(bool(causal)), ctypes.byref(g),
                                              ctypes.byref(ws_bytes)), "la_forward_workspace_size")
    need = ws_bytes.value
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    args = (ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(f), int(bool(causal)), ctypes.byref(g),
            _ptr(S0), _ptr(z0), _ptr(Sf), _ptr(zf), _ptr(out), _ptr(workspace) if need else None, need,
            _stream(Q, stream))
    keep = (p, f, g, Q, K, V, omega, gate, S0, z0, workspace)
    return args, keep, out, Sf, zf


def forward(Q, K, V, *, fmap="elu1", omega=None, causal=True, gate=None, eps=1e-6, S0=None, z0=None,
            return_state=False, out_dtype=None, out=None, workspace=None, stream=None):
    """o = phi(Q) S / (phi(Q) z + eps) through la_forward.

    Q, K [B, H, n, d_k]; V [B, H, n, d_v]; gate None | ("decay", gamma[H]) |
    ("gla", g[B, H, n, r], tau). Returns out, or (out, S_final, z_final).
    """
    args, _keep, out, Sf, zf = _forward_args(Q, K, V, fmap, omega, causal, gate, eps, S0, z0, return_state,
                                             out_dtype, out, workspace, stream)
    N.check(N.lib().la_forward(*args), "la_forward")
    return (out, Sf, zf) if return_state else out


def forward_noalloc(Q, K, V, *, fmap="elu1", omega=None, causal=True, gate=None, eps=1e-6, S0=None, z0=None,
                    out=None, S_final=None, z_final=None, stream=None):
    """forward() through la_forward_noalloc: the library's own fixed scratch
    array instead of a workspace. `out` (and S_final, z_final, to receive the
    final state) must be given: this call allocates nothing."""
    if out is None:
        raise ValueError("forward_noalloc allocates nothing: pass out")
    if (S_final is None) != (z_final is None):
        raise ValueError("S_final and z_final go together")
    args, _keep, out, _, _ = _forward_args(Q, K, V, fmap, omega, causal, gate, eps, S0, z0, False, out.dtype, out,
                                           None, stream, noalloc=True)
    if S_final is not None:
        args = args[:9] + (_ptr(S_final), _ptr(z_final)) + args[11:]
    N.check(N.lib().la_forward_noalloc(*args), "la_forward_noalloc")
    return out


class PreparedForward:
    """One la_forward call validated and marshalled once (same arguments as
    forward). Calling the object launches it again on the same buffers and
    stream, with no per-call Python work beyond the foreign call: for loops
    that repeat a call, such as timing runs. The tensors passed in must stay
    alive and unchanged in shape while the object is used."""

    def __init__(self, Q, K, V, *, fmap="elu1", omega=None, causal=True, gate=None, eps=1e-6, S0=None, z0=None,
                 return_state=False, out_dtype=None, out=None, workspace=None, stream=None):
        self._args, self._keep, self.out, self.S_final, self.z_final = _forward_args(
            Q, K, V, fmap, omega, causal, gate, eps, S0, z0, return_state, out_dtype, out, workspace, stream)
        self._fn = N.lib().la_forward

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            N.check(st, "la_forward")
        return self.out


def _batch_args(Q, K, V, cu_seqlens, max_seqlen, state, slot_ids, read, write, fmap, omega, gate, eps, out,
                workspace, stream):
    """Validate and marshal one la_forward_batch call: (ctypes arguments, keep-alive objects, out)."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, nm)
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3]:
        raise ValueError(f"shapes Q{tuple(Q.shape)} K{tuple(K.shape)} V{tuple(V.shape)} do not match")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K, V must share a dtype")
    B, H, n, d_k = Q.shape
    d_v = V.shape[3]
    f, r = _fmap_struct(fmap, omega, d_k, Q.dtype)
    g = _gate_struct(gate, (B, H, n, r), d_v, Q.dtype)
    p = _problem(B, H, n, d_k, d_v, _dt(Q), _dt(Q), eps)
    if cu_seqlens is not None:
        _dev(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor")
        num_seqs = cu_seqlens.numel() - 1
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens (a host-side bound)")
    else:
        num_seqs, max_seqlen = B, n
    flags = (N.LA_SLOT_READ if read else 0) | (N.LA_SLOT_WRITE if write else 0)
    S = z = None
    num_slots = 0
    if flags:
        if state is None or slot_ids is None:
            raise ValueError("reading or writing slots needs state=(S, z) and slot_ids")
        S, z = state
        _dev(S, "S")
        _dev(z, "z")
        _dev(slot_ids, "slot_ids")
        num_slots = S.shape[0]
        if (S.dtype != torch.float32 or tuple(S.shape) != (num_slots, H, r, d_v) or z.dtype != torch.float32
                or tuple(z.shape) != (num_slots, H, r)):
            raise ValueError(f"state must be float32 S[slots, {H}, {r}, {d_v}] and z[slots, {H}, {r}]")
        if slot_ids.dtype != torch.int32 or slot_ids.numel() != num_seqs:
            raise ValueError("slot_ids must be int32 with one entry per sequence")
    addr = lambda t: None if t is None else t.data_ptr()
    batch = N.LaBatch(addr(cu_seqlens), num_seqs, int(max_seqlen), addr(S), addr(z), addr(slot_ids), num_slots,
                      flags)
    if out is None:
        out = torch.empty((B, H, n, d_v), dtype=Q.dtype, device=Q.device)
    ws_bytes = ctypes.c_size_t(0)
    N.check(N.lib().la_forward_batch_workspace_size(ctypes.byref(p), ctypes.byref(batch), ctypes.byref(f),
                                                    ctypes.byref(g), ctypes.byref(ws_bytes)),
            "la_forward_batch_workspace_size")
    need = ws_bytes.value
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    args = (ctypes.byref(p), ctypes.byref(batch), _ptr(Q), _ptr(K), _ptr(V), ctypes.byref(f), ctypes.byref(g),
            _ptr(out), _ptr(workspace) if need else None, need, _stream(Q, stream))
    keep = (p, batch, f, g, Q, K, V, omega, gate, cu_seqlens, S, z, slot_ids, workspace)
    return args, keep, out


def forward_batch(Q, K, V, *, cu_seqlens=None, max_seqlen=None, state=None, slot_ids=None, read=False,
                  write=False, fmap="elu1", omega=None, gate=None, eps=1e-6, out=None, workspace=None, stream=None):
    """Causal forward over a serving batch through la_forward_batch.

    Without cu_seqlens: B sequences of n tokens (Q [B, H, n, d_k]), e.g. a step
    of n new tokens for each of B running sequences. With cu_seqlens (int32
    [num_seqs + 1] on the device) and max_seqlen (host int): the sequences lie
    back to back along n of [1, H, n, d_k] tensors. state = (S, z), float32
    [slots, H, r, d_v] and [slots, H, r], updated in place; slot_ids int32
    [num_seqs]; read: start from the slots' states; write: store the final
    states. Returns out."""
    args, _keep, out = _batch_args(Q, K, V, cu_seqlens, max_seqlen, state, slot_ids, read, write, fmap, omega,
                                   gate, eps, out, workspace, stream)
    N.check(N.lib().la_forward_batch(*args), "la_forward_batch")
    return out


class PreparedForwardBatch:
    """One la_forward_batch call marshalled once (same arguments as
    forward_batch); calling the object launches it again on the same buffers."""

    def __init__(self, Q, K, V, **kw):
        keys = ("cu_seqlens", "max_seqlen", "state", "slot_ids", "read", "write", "fmap", "omega", "gate", "eps",
                "out", "workspace", "stream")
        d = dict(cu_seqlens=None, max_seqlen=None, state=None, slot_ids=None, read=False, write=False, fmap="elu1",
                 omega=None, gate=None, eps=1e-6, out=None, workspace=None, stream=None)
        d.update(kw)
        self._args, self._keep, self.out = _batch_args(Q, K, V, *(d[k] for k in keys))
        self._fn = N.lib().la_forward_batch

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            N.check(st, "la_forward_batch")
        return self.out


def _backward_args(Q, K, V, dO, fmap, gate, eps, S0, z0, grads, workspace, stream, causal=True, omega=None):
    """Validate and marshal one la_backward call: (ctypes arguments, keep-alive objects, gradients), the
    gradients being (dQ, dK, dV), plus dg with a gate input (GLA, selective, outer-product) and dgv with
    the outer-product gate's value side."""
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V"), (dO, "dO")):
        _dev(t, nm)
    if Q.dim() != 4 or K.shape != Q.shape or V.dim() != 4 or V.shape[:3] != Q.shape[:3] or dO.shape != V.shape:
        raise ValueError(f"shapes Q{tuple(Q.shape)} K{tuple(K.shape)} V{tuple(V.shape)} dO{tuple(dO.shape)} "
                         "do not match")
    if K.dtype != Q.dtype or V.dtype != Q.dtype or dO.dtype != Q.dtype:
        raise TypeError("Q, K, V, dO must share a dtype")
    B, H, n, d_k = Q.shape
    d_v = V.shape[3]
    f, r = _fmap_struct(fmap, omega, d_k, Q.dtype)
    g = _gate_struct(gate, (B, H, n, r), d_v, Q.dtype)
    p = _problem(B, H, n, d_k, d_v, _dt(Q), _dt(Q), eps)
    for t, nm, shp in ((S0, "S0", (B, H, r, d_v)), (z0, "z0", (B, H, r))):
        if t is not None:
            _dev(t, nm)
            if tuple(t.shape) != shp or t.dtype != torch.float32:
                raise ValueError(f"{nm} must be float32 {shp}")
    # gates with an input, whose gradient dg is returned; the outer-product gate adds dgv
    gla = g.kind in (N.LA_GATE_GLA, N.LA_GATE_SEL, N.LA_GATE_OUTER)
    outer = g.kind == N.LA_GATE_OUTER
    if grads is None:
        grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
        if gla:
            grads = grads + (torch.empty_like(gate[1]),)
        if outer:
            grads = grads + (torch.empty_like(gate[2]),)
    if len(grads) != 3 + int(gla) + int(outer):
        raise ValueError("grads must be (dQ, dK, dV)" + (" plus dg with a gate input" if gla else "") +
                         (" and dgv" if outer else ""))
    dQ, dK, dV = grads[:3]
    dg = grads[3] if gla else None
    dgv = grads[4] if outer else None
    checks = ((dQ, Q, "dQ"), (dK, K, "dK"), (dV, V, "dV")) + (((dg, gate[1], "dg"),) if gla else ()) + \
        (((dgv, gate[2], "dgv"),) if outer else ())
    for t, ref, nm in checks:
        _dev(t, nm)
        if t.shape != ref.shape or t.dtype != ref.dtype:
            raise ValueError(f"{nm} has the wrong shape or dtype")
    ws_bytes = ctypes.c_size_t(0)
    N.check(N.lib().la_backward_workspace_size(ctypes.byref(p), ctypes.byref(f), int(bool(causal)), ctypes.byref(g),
                                               ctypes.byref(ws_bytes)), "la_backward_workspace_size")
    need = ws_bytes.value
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    args = (ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), _ptr(dO), ctypes.byref(f), int(bool(causal)), ctypes.byref(g),
            _ptr(S0),
            _ptr(z0), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dg), _ptr(dgv), _ptr(workspace), need, _stream(Q, stream))
    keep = (p, f, g, Q, K, V, dO, gate, S0, z0, workspace, omega)
    return args, keep, tuple(grads)


def backward(Q, K, V, dO, *, fmap="elu1", omega=None, gate=None, eps=1e-6, S0=None, z0=None, grads=None,
             workspace=None, stream=None, causal=True):
    """(dQ, dK, dV) of the causal forward for an incoming gradient dO, through la_backward;
    (dQ, dK, dV, dg) with the GLA or the selective gate, dg the gradient of its raw input g;
    (dQ, dK, dV, dg, dgv) with the outer-product gate, dgv the gradient of its value-side input gv.

    Q, K [B, H, n, d_k]; V, dO [B, H, n, d_v] (bf16); gate None | ("decay", gamma[H]) |
    ("gla", g[B, H, n, d_k] bf16, tau) | ("sel", g[B, H, n] bf16, tau) |
    ("outer", g[B, H, n, d_k], gv[B, H, n, d_v] bf16, tau); S0, z0: the forward's
    carried-in state, if any. fmap="favor" with omega [r, d_k] (r 64 or 128; no gate or the
    decay). causal=False: the non-causal form (elu+1, no gate, no state; fp32 or bf16,
    gradients in the input dtype)."""
    args, _keep, grads = _backward_args(Q, K, V, dO, fmap, gate, eps, S0, z0, grads, workspace, stream, causal,
                                        omega)
    N.check(N.lib().la_backward(*args), "la_backward")
    return grads


class PreparedBackward:
    """One la_backward call marshalled once (same arguments as backward);
    calling the object launches it again on the same buffers and stream."""

    def __init__(self, Q, K, V, dO, *, fmap="elu1", omega=None, gate=None, eps=1e-6, S0=None, z0=None, grads=None,
                 workspace=None, stream=None, causal=True):
        self._args, self._keep, self.grads = _backward_args(Q, K, V, dO, fmap, gate, eps, S0, z0, grads, workspace,
                                                            stream, causal, omega)
        self._fn = N.lib().la_backward

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            N.check(st, "la_backward")
        return self.grads


def _decode_args(S, z, q, k, v, fmap, omega, gate, eps, out_dtype, out, stream):
    for t, nm in ((S, "S"), (z, "z"), (q, "q"), (k, "k"), (v, "v")):
        _dev(t, nm)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [B, H, d_k] and v [B, H, d_v]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    B, H, d_k = q.shape
    d_v = v.shape[2]
    f, r = _fmap_struct(fmap, omega, d_k, q.dtype)
    if tuple(S.shape) != (B, H, r, d_v) or S.dtype != torch.float32:
        raise ValueError(f"S must be float32 {(B, H, r, d_v)}")
    if tuple(z.shape) != (B, H, r) or z.dtype != torch.float32:
        raise ValueError(f"z must be float32 {(B, H, r)}")
    g = _gate_struct(gate, (B, H, r), d_v, q.dtype)
    p = _problem(B, H, 1, d_k, d_v, _dt(q), _DT[out_dtype], eps)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=out_dtype, device=q.device)
    args = (ctypes.byref(p), _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(f), ctypes.byref(g),
            _ptr(out), _stream(q, stream))
    return args, (p, f, g, S, z, q, k, v, omega, gate), out


def decode_step(S, z, q, k, v, *, fmap="elu1", omega=None, gate=None, eps=1e-6, out_dtype=torch.float32,
                out=None, stream=None):
    """One recurrent step; S [B, H, r, d_v] and z [B, H, r] (fp32) are updated in place.

    q, k [B, H, d_k]; v [B, H, d_v]; gate None | ("decay", gamma[H]) |
    ("gla", g[B, H, r], tau). Returns out [B, H, d_v].
    """
    args, _keep, out = _decode_args(S, z, q, k, v, fmap, omega, gate, eps, out_dtype, out, stream)
    N.check(N.lib().la_decode_step(*args), "la_decode_step")
    return out


class PreparedDecode:
    """One la_decode_step call validated and marshalled once (same arguments
    as decode_step); calling the object launches it again on the same buffers."""

    def __init__(self, S, z, q, k, v, *, fmap="elu1", omega=None, gate=None, eps=1e-6, out_dtype=torch.float32,
                 out=None, stream=None):
        self._args, self._keep, self.out = _decode_args(S, z, q, k, v, fmap, omega, gate, eps, out_dtype, out,
                                                        stream)
        self._fn = N.lib().la_decode_step

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            N.check(st, "la_decode_step")
        return self.out


def feature_map(X, *, fmap="elu1", omega=None, stream=None):
    """phi(X) over the last axis in fp32 through la_feature_map_apply."""
    _dev(X, "X")
    d_k = X.shape[-1]
    f, r = _fmap_struct(fmap, omega, d_k, X.dtype)
    rows = X.numel() // d_k
    out = torch.empty(X.shape[:-1] + (r,), dtype=torch.float32, device=X.device)
    N.check(N.lib().la_feature_map_apply(ctypes.byref(f), rows, d_k, _dt(X), _ptr(X), _ptr(out),
                                         _stream(X, stream)), "la_feature_map_apply")
    return out


def _softmax_args(Q, K, V, causal, scale, out, stream):
    for t, nm in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, nm)
    if Q.dim() != 4 or K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError(f"Q, K, V must share one [B, H, n, d] shape, got {tuple(Q.shape)} {tuple(K.shape)} "
                         f"{tuple(V.shape)}")
    if K.dtype != Q.dtype or V.dtype != Q.dtype:
        raise TypeError("Q, K, V must share a dtype")
    B, H, n, d = Q.shape
    scale = d ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(V)
    else:
        _dev(out, "out")
        if out.shape != V.shape or out.dtype != V.dtype:
            raise ValueError("out has the wrong shape or dtype")
    p = _problem(B, H, n, d, d, _dt(Q), _dt(out), 0.0)
    args = (ctypes.byref(p), _ptr(Q), _ptr(K), _ptr(V), int(bool(causal)), scale, _ptr(out), _stream(Q, stream))
    return args, (p, Q, K, V), out


def softmax_attention(Q, K, V, *, causal=True, scale=None, out=None, stream=None):
    """Softmax attention (the quadratic baseline) through la_softmax_attention:
    o_i = sum_j softmax_j(scale q_i . k_j) v_j, bf16 [B, H, n, d], d in {64, 128};
    scale defaults to 1/sqrt(d)."""
    args, _keep, out = _softmax_args(Q, K, V, causal, scale, out, stream)
    N.check(N.lib().la_softmax_attention(*args), "la_softmax_attention")
    return out


class PreparedSoftmax:
    """One la_softmax_attention call marshalled once (same arguments as
    softmax_attention); calling the object launches it again."""

    def __init__(self, Q, K, V, *, causal=True, scale=None, out=None, stream=None):
        self._args, self._keep, self.out = _softmax_args(Q, K, V, causal, scale, out, stream)
        self._fn = N.lib().la_softmax_attention

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            N.check(st, "la_softmax_attention")
        return self.out


def launch_times(call, steps, stream, max_launches=8):
    """GPU time of every kernel launch of `steps` calls of `call()` (a prepared
    call on `stream`), through la_timing_begin / la_timing_end: each call runs
    inside its own timing bracket with its own events, back to back. Returns a
    list per call of the milliseconds of each launch, in launch order."""
    L = N.lib()
    evs = []
    for _ in range(steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(max_launches + 1)]
        for e in row:
            e.record(stream)  # creates the event so that it has a handle
        evs.append(row)
    torch.cuda.synchronize()
    handles = [(ctypes.c_void_p * len(row))(*[e.cuda_event for e in row]) for row in evs]
    sp = ctypes.c_void_p(stream.cuda_stream)
    counts = []
    for i in range(steps):
        N.check(L.la_timing_begin(handles[i], len(evs[i])), "la_timing_begin")
        try:
            call()
        finally:
            nl = ctypes.c_int32(0)
            st = L.la_timing_end(sp, ctypes.byref(nl))
        N.check(st, "la_timing_end")
        if nl.value > max_launches:
            raise ValueError(f"{nl.value} launches per call; raise max_launches")
        counts.append(nl.value)
    torch.cuda.synchronize()
    return [[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(counts[i])] for i in range(steps)]
