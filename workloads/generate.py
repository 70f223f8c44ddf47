"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

One ``numpy.random.default_rng(seed)`` per call; draws are fp32
``standard_normal`` in a fixed order (Q, K, V, then g, then the FAVOR+
frequency blocks and their norm vectors, then the decode state), scaled in fp32
and cast to bf16 by round-to-nearest-even (torch's conversion). The GPU and the
oracle both receive exactly these values. This module holds no arithmetic of
the attention method itself; the random frequencies of FAVOR+ are drawn here
because the method takes them as an input.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import WORKLOADS, Workload

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(TORCH_DTYPE[dtype]).contiguous()


def to_f64(t) -> np.ndarray:
    """Exact float64 copy of a (CPU or device) tensor."""
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def orthogonal_gaussian_omega(rng, r: int, d: int) -> np.ndarray:
    """r x d random frequencies: ceil(r/d) blocks of orthonormal rows, rescaled.

    Each d x d block is the Q factor of the QR decomposition of a Gaussian
    matrix, with signs fixed by diag(R); each row is then rescaled by the norm
    of an independent N(0, I_d) draw so that rows are marginally N(0, I_d).
    """
    nblk = -(-r // d)
    blocks = []
    for _ in range(nblk):
        G = rng.standard_normal((d, d), dtype=np.float32).astype(np.float64)
        Qm, Rm = np.linalg.qr(G)
        Qm = Qm * np.sign(np.diag(Rm))[None, :]
        blocks.append(Qm.T)  # rows orthonormal
    W = np.concatenate(blocks, axis=0)[:r]
    norms = np.linalg.norm(rng.standard_normal((r, d), dtype=np.float32).astype(np.float64), axis=1)
    return (W * norms[:, None]).astype(np.float32)


def retnet_gammas(H: int) -> np.ndarray:
    """gamma_h = 1 - 2^(-5-h): per-head fixed decay rates."""
    return np.array([1.0 - 2.0 ** (-5 - h) for h in range(H)], dtype=np.float32)


def make_inputs(wl, seed: int = 0, *, B=None, H=None, n=None, qk_scale=None,
                v_scale=None) -> dict:
    """Inputs for workload ``wl`` (a Workload or its name) as CPU torch tensors.

    Overrides shrink or stretch the shape (same distribution, same draw order)
    for parity tests at sizes the oracle finishes quickly.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    n = wl.n if n is None else n
    qs = wl.qk_scale if qk_scale is None else qk_scale
    vs = wl.v_scale if v_scale is None else v_scale
    rng = np.random.default_rng(seed)
    out = {"B": B, "H": H, "n": n, "d_k": wl.d_k, "d_v": wl.d_v, "r": wl.r,
           "fmap": wl.fmap, "causal": wl.causal, "gate": wl.gate, "dtype": wl.dtype,
           "eps": wl.eps, "tau": wl.tau}
    if wl.decode:
        out.update(_decode_inputs(wl, rng, B, H, qs, vs))
        return out
    f32 = np.float32
    Q = rng.standard_normal((B, H, n, wl.d_k), dtype=f32) * f32(qs)
    K = rng.standard_normal((B, H, n, wl.d_k), dtype=f32) * f32(qs)
    V = rng.standard_normal((B, H, n, wl.d_v), dtype=f32) * f32(vs)
    out["Q"], out["K"], out["V"] = _cast(Q, wl.dtype), _cast(K, wl.dtype), _cast(V, wl.dtype)
    if wl.gate == "gla":
        g = rng.standard_normal((B, H, n, wl.r), dtype=f32)
        out["g"] = _cast(g, wl.dtype)
    if wl.gate == "sel":
        out["g"] = _cast(rng.standard_normal((B, H, n), dtype=f32), wl.dtype)
    if wl.gate == "outer":  # key side as GLA, then the value side per value column
        out["g"] = _cast(rng.standard_normal((B, H, n, wl.r), dtype=f32), wl.dtype)
        out["gv"] = _cast(rng.standard_normal((B, H, n, wl.d_v), dtype=f32), wl.dtype)
    if wl.gate == "decay":
        out["gamma"] = torch.from_numpy(retnet_gammas(H))
    if wl.fmap == "favor":
        out["omega"] = _cast(orthogonal_gaussian_omega(rng, wl.r, wl.d_k), wl.dtype)
    return out


def strong_gate_input(shape, seed: int, dtype: str = "bf16", mean: float = -18.75, std: float = 0.25,
                      period: int = 2, chunk: int = 64) -> torch.Tensor:
    """A raw gate input of ``shape`` (time on axis 2: [B, H, n, r] or [B, H, n])
    whose tokens in the chunk-sized blocks 0, period, 2 period, ... of the time
    axis are N(mean, std^2) and whose other tokens are N(0, 1); period 1 makes
    every block strong. Both draws are taken in full, in that order, from one
    seeded generator, then cast like every other input."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    g = rng.standard_normal(shape, dtype=f32)
    s = rng.standard_normal(shape, dtype=f32) * f32(std) + f32(mean)
    blk = (np.arange(shape[2]) // chunk) % period == 0
    sel = blk.reshape((1, 1, -1) + (1,) * (len(shape) - 3))
    return _cast(np.where(sel, s, g), dtype)


def incoming_gradient(shape, seed: int, dtype: str = "bf16", scale: float = 1.0) -> torch.Tensor:
    """A seeded dL/d(out) for the backward pass: N(0,1) * scale, cast like the inputs."""
    rng = np.random.default_rng(seed)
    g = rng.standard_normal(tuple(shape), dtype=np.float32) * np.float32(scale)
    return _cast(g, dtype)


def _decode_inputs(wl: Workload, rng, B, H, qs, vs) -> dict:
    """A carried state standing in for a short prefill, plus one new token.

    The state is drawn directly (no attention arithmetic): S entries are
    N(0, 16 * v_scale^2), the spread of a sum of 16 value vectors weighted by
    features near 1, and z entries are 16 * (1 + 0.05 * |N(0,1)|) > 0, the size
    of a sum of 16 such features.
    """
    f32 = np.float32
    r, dv = wl.r, wl.d_v
    S0 = rng.standard_normal((B, H, r, dv), dtype=f32) * f32(4.0 * vs)
    z0 = f32(16.0) * (f32(1.0) + f32(0.05) * np.abs(rng.standard_normal((B, H, r), dtype=f32)))
    q = rng.standard_normal((B, H, wl.d_k), dtype=f32) * f32(qs)
    k = rng.standard_normal((B, H, wl.d_k), dtype=f32) * f32(qs)
    v = rng.standard_normal((B, H, dv), dtype=f32) * f32(vs)
    d = {"S0": torch.from_numpy(S0), "z0": torch.from_numpy(z0.astype(f32)),
         "q": _cast(q, wl.dtype), "k": _cast(k, wl.dtype), "v": _cast(v, wl.dtype)}
    if wl.gate == "gla":
        d["g"] = _cast(rng.standard_normal((B, H, r), dtype=f32), wl.dtype)
    if wl.gate == "sel":
        d["g"] = _cast(rng.standard_normal((B, H), dtype=f32), wl.dtype)
    if wl.gate == "outer":
        d["g"] = _cast(rng.standard_normal((B, H, r), dtype=f32), wl.dtype)
        d["gv"] = _cast(rng.standard_normal((B, H, dv), dtype=f32), wl.dtype)
    if wl.gate == "decay":
        d["gamma"] = torch.from_numpy(retnet_gammas(H))
    if wl.fmap == "favor":
        d["omega"] = _cast(orthogonal_gaussian_omega(rng, wl.r, wl.d_k), wl.dtype)
    return d


def serving_lengths(num_seqs: int, seed: int, lo: int = 64, hi: int = 8192) -> np.ndarray:
    """A seeded length mix for a serving batch: log-uniform integers in [lo, hi]
    (many short requests, a few long ones), as int32."""
    rng = np.random.default_rng(seed)
    u = rng.random(num_seqs)
    return np.clip(np.round(np.exp(np.log(lo) + u * (np.log(hi) - np.log(lo)))), lo, hi).astype(np.int32)
