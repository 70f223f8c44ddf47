"""The synthetic workloads, as data.

Each entry fixes shapes, dtypes, value scales and the gate/feature-map choice of
one measured configuration. No arithmetic of the method lives here.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    d_k: int
    d_v: int
    r: int                 # feature dimension (d_k for elu1)
    fmap: str              # "elu1" | "favor" | "identity" (the state-space read-out)
    causal: bool
    gate: str              # "none" | "decay" | "gla" | "sel" (scalar selective) | "outer" (alpha beta^T)
    dtype: str             # input dtype: "f32" | "bf16"
    qk_scale: float        # Q, K ~ N(0,1) * qk_scale
    v_scale: float         # V ~ N(0,1) * v_scale
    eps: float = 1e-6
    tau: float = 16.0      # GLA temperature
    decode: bool = False   # one recurrent step from a carried state

    @property
    def out_dtype(self):
        # forward output takes the input dtype; decode writes fp32
        return "f32" if self.decode else self.dtype

    @property
    def head_tokens(self):
        return self.B * self.H * self.n

    def resized(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "noncausal_elu1_f32": Workload(
        "noncausal_elu1_f32", B=1, H=1, n=256, d_k=32, d_v=32, r=32, fmap="elu1",
        causal=False, gate="none", dtype="f32", qk_scale=32 ** -0.5, v_scale=32 ** -0.5),
    "causal_elu1": Workload(
        "causal_elu1", B=4, H=16, n=4096, d_k=64, d_v=64, r=64, fmap="elu1",
        causal=True, gate="none", dtype="bf16", qk_scale=64 ** -0.5, v_scale=64 ** -0.5),
    "retnet_decay": Workload(
        "retnet_decay", B=2, H=8, n=8192, d_k=128, d_v=128, r=128, fmap="elu1",
        causal=True, gate="decay", dtype="bf16", qk_scale=128 ** -0.5, v_scale=128 ** -0.5),
    "gla_gate": Workload(
        "gla_gate", B=2, H=16, n=16384, d_k=128, d_v=128, r=128, fmap="elu1",
        causal=True, gate="gla", dtype="bf16", qk_scale=128 ** -0.5, v_scale=128 ** -0.5),
    # the GLA workload's shape under the outer-product gate (value-side gate input gv
    # ~ N(0,1) per value column, same tau)
    "outer_gate": Workload(
        "outer_gate", B=2, H=16, n=16384, d_k=128, d_v=128, r=128, fmap="elu1",
        causal=True, gate="outer", dtype="bf16", qk_scale=128 ** -0.5, v_scale=128 ** -0.5),
    "gla_decode": Workload(
        "gla_decode", B=256, H=16, n=1, d_k=128, d_v=128, r=128, fmap="elu1",
        causal=True, gate="gla", dtype="bf16", qk_scale=128 ** -0.5, v_scale=128 ** -0.5,
        decode=True),
    "ssm_selective": Workload(
        "ssm_selective", B=2, H=16, n=16384, d_k=64, d_v=64, r=64, fmap="identity",
        causal=True, gate="gla", dtype="bf16", qk_scale=64 ** -0.5, v_scale=1.0),
    "ssm_scalar": Workload(
        "ssm_scalar", B=2, H=16, n=16384, d_k=64, d_v=64, r=64, fmap="identity",
        causal=True, gate="sel", dtype="bf16", qk_scale=64 ** -0.5, v_scale=1.0),
    "favor_causal": Workload(
        "favor_causal", B=1, H=8, n=32768, d_k=64, d_v=64, r=256, fmap="favor",
        causal=True, gate="none", dtype="bf16", qk_scale=64 ** -0.25, v_scale=1.0),
}

# The measured headline workload: the largest configuration, the GLA-gated
# causal elu+1 forward (B2 H16 n16384 d128, bf16, chunk 64).
HEADLINE = "gla_gate"


def describe(wl: Workload) -> str:
    s = f"B={wl.B} H={wl.H} n={wl.n} d_k={wl.d_k} d_v={wl.d_v}"
    if wl.fmap == "favor":
        s += f" r={wl.r}"
    return f"{wl.name}: {s} {wl.dtype} fmap={wl.fmap} causal={int(wl.causal)} gate={wl.gate}"
