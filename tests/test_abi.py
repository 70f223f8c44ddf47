"""The C ABI on the host: exports, struct layouts, planning and argument checks.

No test here launches a kernel. The validation tests pass fake device pointers
that are only compared and never dereferenced; each case breaks exactly one
rule that the library checks before any HIP call. They are skipped where a GPU
is visible, so a validation bug can never turn into a launch on fake pointers.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

from kernelized_sequence_mixing_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

needs_lib = pytest.mark.skipif(not os.path.exists(N.LIB_PATH), reason="liblinattn.so not built")
no_gpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake-pointer checks run only without a GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(N.EXPORTED)


@needs_lib
def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
    lib = N.lib()
    for name in declared_functions():
        assert hasattr(lib, name)


@needs_lib
def test_version_and_status_strings():
    lib = N.lib()
    assert lib.la_abi_version() == 7
    names = [lib.la_status_str(i).decode() for i in range(6)]
    assert names == ["LA_OK", "LA_ERR_INVALID_ARG", "LA_ERR_UNSUPPORTED", "LA_ERR_WORKSPACE", "LA_ERR_ALIAS",
                     "LA_ERR_HIP"]
    assert lib.la_status_str(99).decode() == "LA_ERR_UNKNOWN"


def test_struct_layouts_match_the_header(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(f"""
#include <stdio.h>
#include <stddef.h>
#include "{HEADER}"
int main(void) {{
  printf("%zu %zu %zu\\n", sizeof(la_problem), offsetof(la_problem, eps), offsetof(la_problem, out_dtype));
  printf("%zu %zu %zu\\n", sizeof(la_feature_map), offsetof(la_feature_map, r), offsetof(la_feature_map, omega));
  printf("%zu %zu %zu %zu %zu\\n", sizeof(la_gate), offsetof(la_gate, tau), offsetof(la_gate, gamma), offsetof(la_gate, g),
         offsetof(la_gate, gv));
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(la_batch), offsetof(la_batch, cu_seqlens),
         offsetof(la_batch, num_seqs), offsetof(la_batch, max_seqlen), offsetof(la_batch, S), offsetof(la_batch, z),
         offsetof(la_batch, slot_ids), offsetof(la_batch, num_slots), offsetof(la_batch, flags));
  return 0;
}}""")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    c = [list(map(int, ln.split())) for ln in lines if ln.strip()]
    assert c[0] == [ctypes.sizeof(N.LaProblem), N.LaProblem.eps.offset, N.LaProblem.out_dtype.offset]
    assert c[1] == [ctypes.sizeof(N.LaFeatureMap), N.LaFeatureMap.r.offset, N.LaFeatureMap.omega.offset]
    assert c[2] == [ctypes.sizeof(N.LaGate), N.LaGate.tau.offset, N.LaGate.gamma.offset, N.LaGate.g.offset,
                    N.LaGate.gv.offset]
    B = N.LaBatch
    assert c[3] == [ctypes.sizeof(B), B.cu_seqlens.offset, B.num_seqs.offset, B.max_seqlen.offset, B.S.offset,
                    B.z.offset, B.slot_ids.offset, B.num_slots.offset, B.flags.offset]


# ------------------------------------------------------------------ planning (host arithmetic)

@needs_lib
@pytest.mark.parametrize("B,H,n,d,dv,fmap,r,gate,expect_P,expect_len", [
    # output-pass LDS 36.8 KB -> 4 workgroups per CU by LDS, capped at 2 -> 512 (head, segment) groups
    (4, 16, 4096, 64, 64, "elu1", 64, "none", 8, 512),        # causal elu+1 workload
    # 128 x 128 states: one output-pass workgroup per CU (registers) -> 256 groups
    (2, 8, 8192, 128, 128, "elu1", 128, "decay", 16, 512),    # RetNet workload
    (2, 16, 16384, 128, 128, "elu1", 128, "gla", 8, 2048),    # GLA workload
    # FAVOR+ r=256: 56.3 KB (64-feature blocks) -> 2 per CU -> 512 groups
    (1, 8, 32768, 64, 64, "favor", 256, "none", 64, 512),     # FAVOR+ workload
    (1, 1, 1, 64, 64, "elu1", 64, "none", 1, 64),
    (1, 1, 65, 64, 64, "elu1", 64, "none", 2, 64),
    (300, 1, 100, 64, 64, "elu1", 64, "none", 2, 64),
    (600, 1, 100, 64, 64, "elu1", 64, "none", 1, 128),
    (800, 1, 100, 64, 64, "elu1", 64, "none", 1, 128),
])
def test_segment_plan(B, H, n, d, dv, fmap, r, gate, expect_P, expect_len):
    from kernelized_sequence_mixing_amd import segments
    P, L = segments(B, H, n, d, dv, fmap=fmap, r=r, gate_kind=gate)
    assert (P, L) == (expect_P, expect_len)
    assert L % 64 == 0 and (P - 1) * L < n <= P * L


@needs_lib
def test_workspace_sizes():
    from kernelized_sequence_mixing_amd import workspace_size
    # one segment: nothing to chain
    assert workspace_size(800, 1, 100, 64, 64) == 0
    # 8 segments x 64 heads of 64x64 fp32 states + normalisers, each region 256-aligned
    assert workspace_size(4, 16, 4096, 64, 64) == 64 * 8 * 64 * 64 * 4 + 64 * 8 * 64 * 4
    gla = workspace_size(2, 16, 16384, 128, 128, gate_kind="gla")
    plain = workspace_size(2, 16, 16384, 128, 128)
    assert gla == plain + 32 * 8 * 128 * 4  # 8 segments: one summed log-gate row per (head, segment)
    # the outer-product gate adds one summed value-side log-gate row (d_v) per (head, segment)
    from kernelized_sequence_mixing_amd import segments
    P, _ = segments(2, 16, 16384, 128, 128, gate_kind="outer")
    outer = workspace_size(2, 16, 16384, 128, 128, gate_kind="outer")
    assert outer == 32 * P * (128 * 128 + 128 + 128 + 128) * 4
    # non-causal partial sums always need workspace
    assert workspace_size(1, 1, 256, 32, 32, causal=False, dtype=torch.float32) > 0


# ------------------------------------------------------------------ validation (no launch)

FAKE = 0x7f0000000000  # a 256-aligned fake device address; never dereferenced
SP = 1 << 32           # spacing of the fake buffers: far apart, so only planted overlaps exist


def _args(**over):
    d = dict(B=2, H=3, n=100, d_k=64, d_v=64, in_dt=N.LA_BF16, out_dt=N.LA_BF16, eps=1e-6,
             fkind=N.LA_FMAP_ELU1, r=64, omega=None, causal=1, gkind=N.LA_GATE_NONE, tau=16.0, gamma=None, g=None,
             gv=None,
             Q=FAKE, K=FAKE + SP, V=FAKE + 2 * SP, S0=None, z0=None, Sf=None, zf=None,
             out=FAKE + 3 * SP, ws=FAKE + 4 * SP, ws_bytes=1 << 30)
    d.update(over)
    return d


def _forward(a):
    p = N.LaProblem(a["B"], a["H"], a["n"], a["d_k"], a["d_v"], a["in_dt"], a["out_dt"], a["eps"])
    f = N.LaFeatureMap(a["fkind"], a["r"], a["omega"])
    g = N.LaGate(a["gkind"], a["tau"], a["gamma"], a["g"], a["gv"])
    return N.lib().la_forward(ctypes.byref(p), a["Q"], a["K"], a["V"], ctypes.byref(f), a["causal"],
                              ctypes.byref(g), a["S0"], a["z0"], a["Sf"], a["zf"], a["out"], a["ws"],
                              a["ws_bytes"], None)


BAD_FORWARD = [
    ("sel favor", dict(gkind=N.LA_GATE_SEL, g=FAKE + 6 * SP, fkind=N.LA_FMAP_FAVOR, r=256, omega=FAKE + 5 * SP),
     N.LA_ERR_UNSUPPORTED),
    ("sel no g", dict(gkind=N.LA_GATE_SEL), N.LA_ERR_INVALID_ARG),
    ("sel tau 0", dict(gkind=N.LA_GATE_SEL, g=FAKE + 6 * SP, tau=0.0), N.LA_ERR_INVALID_ARG),
    ("sel noncausal", dict(gkind=N.LA_GATE_SEL, g=FAKE + 6 * SP, causal=0, in_dt=N.LA_F32, out_dt=N.LA_F32),
     N.LA_ERR_INVALID_ARG),
    ("gate kind 5", dict(gkind=5), N.LA_ERR_INVALID_ARG),
    ("outer no g", dict(gkind=N.LA_GATE_OUTER, gv=FAKE + 7 * SP), N.LA_ERR_INVALID_ARG),
    ("outer no gv", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP), N.LA_ERR_INVALID_ARG),
    ("outer gv misaligned", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP + 8), N.LA_ERR_INVALID_ARG),
    ("gv with gla", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP, gv=FAKE + 7 * SP), N.LA_ERR_INVALID_ARG),
    ("gv without gate", dict(gv=FAKE + 7 * SP), N.LA_ERR_INVALID_ARG),
    ("outer tau 0", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP, tau=0.0), N.LA_ERR_INVALID_ARG),
    ("outer favor", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP, fkind=N.LA_FMAP_FAVOR, r=256,
                         omega=FAKE + 5 * SP), N.LA_ERR_UNSUPPORTED),
    ("outer noncausal", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP, causal=0, in_dt=N.LA_F32,
                             out_dt=N.LA_F32), N.LA_ERR_INVALID_ARG),
    ("outer gv under out", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 3 * SP + 256), N.LA_ERR_ALIAS),
    ("identity noncausal", dict(fkind=N.LA_FMAP_IDENTITY, causal=0, in_dt=N.LA_F32, out_dt=N.LA_F32),
     N.LA_ERR_UNSUPPORTED),
    ("identity r != d_k", dict(fkind=N.LA_FMAP_IDENTITY, r=32), N.LA_ERR_INVALID_ARG),
    ("identity with omega", dict(fkind=N.LA_FMAP_IDENTITY, omega=FAKE + 5 * SP), N.LA_ERR_INVALID_ARG),
    ("fmap kind 3", dict(fkind=3), N.LA_ERR_INVALID_ARG),
    ("B=0", dict(B=0), N.LA_ERR_INVALID_ARG),
    ("n=0", dict(n=0), N.LA_ERR_INVALID_ARG),
    ("d_v<0", dict(d_v=-64), N.LA_ERR_INVALID_ARG),
    ("dtype 7", dict(in_dt=7), N.LA_ERR_INVALID_ARG),
    ("eps<0", dict(eps=-1.0), N.LA_ERR_INVALID_ARG),
    ("eps nan", dict(eps=float("nan")), N.LA_ERR_INVALID_ARG),
    ("fmap kind", dict(fkind=5), N.LA_ERR_INVALID_ARG),
    ("elu r != d_k", dict(r=32), N.LA_ERR_INVALID_ARG),
    ("elu with omega", dict(omega=FAKE + 5 * SP), N.LA_ERR_INVALID_ARG),
    ("favor no omega", dict(fkind=N.LA_FMAP_FAVOR, r=256), N.LA_ERR_INVALID_ARG),
    ("favor odd r", dict(fkind=N.LA_FMAP_FAVOR, r=100, omega=FAKE + 5 * SP), N.LA_ERR_UNSUPPORTED),
    ("favor+gla", dict(fkind=N.LA_FMAP_FAVOR, r=128, omega=FAKE + 5 * SP, gkind=N.LA_GATE_GLA,
                       g=FAKE + 6 * SP), N.LA_ERR_UNSUPPORTED),
    ("gate kind", dict(gkind=9), N.LA_ERR_INVALID_ARG),
    ("tau<=0", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP, tau=0.0), N.LA_ERR_INVALID_ARG),
    ("gla no g", dict(gkind=N.LA_GATE_GLA), N.LA_ERR_INVALID_ARG),
    ("decay no gamma", dict(gkind=N.LA_GATE_DECAY), N.LA_ERR_INVALID_ARG),
    ("noncausal gated", dict(causal=0, gkind=N.LA_GATE_DECAY, gamma=FAKE + 6 * SP), N.LA_ERR_INVALID_ARG),
    ("causal flag 2", dict(causal=2), N.LA_ERR_INVALID_ARG),
    ("d_k 48", dict(d_k=48, r=48), N.LA_ERR_UNSUPPORTED),
    ("causal d_v 96", dict(d_v=96), N.LA_ERR_UNSUPPORTED),
    ("causal d_v 32 ws small", dict(d_v=32, ws_bytes=1 << 16), N.LA_ERR_WORKSPACE),
    ("causal fp32", dict(in_dt=N.LA_F32, out_dt=N.LA_F32), N.LA_ERR_UNSUPPORTED),
    ("causal fp32 out", dict(out_dt=N.LA_F32), N.LA_ERR_UNSUPPORTED),
    ("r*d_v too big", dict(fkind=N.LA_FMAP_FAVOR, r=256, d_v=128, omega=FAKE + 5 * SP), N.LA_ERR_UNSUPPORTED),
    ("BH too big", dict(B=70000, H=1), N.LA_ERR_UNSUPPORTED),
    ("Q null", dict(Q=None), N.LA_ERR_INVALID_ARG),
    ("out null", dict(out=None), N.LA_ERR_INVALID_ARG),
    ("Q misaligned", dict(Q=FAKE + 8), N.LA_ERR_INVALID_ARG),
    ("S0 without z0", dict(S0=FAKE + 7 * SP), N.LA_ERR_INVALID_ARG),
    ("Sf without zf", dict(Sf=FAKE + 7 * SP), N.LA_ERR_INVALID_ARG),
    ("noncausal S0", dict(causal=0, S0=FAKE + 7 * SP, z0=FAKE + 8 * SP), N.LA_ERR_INVALID_ARG),
    ("out aliases V", dict(out=FAKE + 2 * SP + 64), N.LA_ERR_ALIAS),
    ("Sf aliases K", dict(Sf=FAKE + SP, zf=FAKE + 9 * SP), N.LA_ERR_ALIAS),
    ("ws overlaps out", dict(B=4, H=16, n=4096, ws=FAKE + 3 * SP + 256), N.LA_ERR_ALIAS),
    ("ws null", dict(B=4, H=16, n=4096, ws=None), N.LA_ERR_WORKSPACE),
    ("ws small", dict(B=4, H=16, n=4096, ws_bytes=1024), N.LA_ERR_WORKSPACE),
    ("ws misaligned", dict(B=4, H=16, n=4096, ws=FAKE + 4 * SP + 16), N.LA_ERR_WORKSPACE),
]


@needs_lib
@no_gpu
@pytest.mark.parametrize("name,over,want", BAD_FORWARD, ids=[b[0] for b in BAD_FORWARD])
def test_forward_rejects(name, over, want):
    assert _forward(_args(**over)) == want


@needs_lib
@no_gpu
def test_decode_rejects():
    lib = N.lib()

    def call(n=1, S=FAKE, z=FAKE + 0x1000000, q=FAKE + 0x2000000, out=FAKE + 0x3000000, d_v=128, gk=0, tau=16.0):
        p = N.LaProblem(4, 2, n, 128, d_v, N.LA_BF16, N.LA_F32, 1e-6)
        f = N.LaFeatureMap(N.LA_FMAP_ELU1, 128, None)
        g = N.LaGate(gk, tau, None, None)
        return lib.la_decode_step(ctypes.byref(p), S, z, q, FAKE + 0x4000000, FAKE + 5 * SP, ctypes.byref(f),
                                  ctypes.byref(g), out, None)
    assert call(n=2) == N.LA_ERR_INVALID_ARG
    assert call(S=None) == N.LA_ERR_INVALID_ARG
    assert call(q=FAKE + 0x2000000 + 4) == N.LA_ERR_INVALID_ARG
    assert call(d_v=96) == N.LA_ERR_UNSUPPORTED
    assert call(gk=N.LA_GATE_GLA) == N.LA_ERR_INVALID_ARG  # no g pointer
    assert call(gk=N.LA_GATE_GLA, tau=-1.0) == N.LA_ERR_INVALID_ARG
    assert call(out=FAKE + 0x2000000) == N.LA_ERR_ALIAS   # out over q
    assert call(z=FAKE + 0x100) == N.LA_ERR_ALIAS         # z inside S


@needs_lib
@no_gpu
def test_feature_map_rejects():
    lib = N.lib()
    f = N.LaFeatureMap(N.LA_FMAP_ELU1, 64, None)
    assert lib.la_feature_map_apply(ctypes.byref(f), 0, 64, N.LA_BF16, FAKE, FAKE + 0x100000, None) == N.LA_ERR_INVALID_ARG
    assert lib.la_feature_map_apply(ctypes.byref(f), 10, 64, N.LA_BF16, FAKE, FAKE + 64, None) == N.LA_ERR_ALIAS
    f2 = N.LaFeatureMap(N.LA_FMAP_ELU1, 48, None)
    assert lib.la_feature_map_apply(ctypes.byref(f2), 10, 48, N.LA_BF16, FAKE, FAKE + 0x100000, None) == N.LA_ERR_UNSUPPORTED


# ------------------------------------------------------------------ backward (validation, no launch)

def _backward(a, dO=FAKE + 10 * SP, dQ=FAKE + 11 * SP, dK=FAKE + 12 * SP, dV=FAKE + 13 * SP, dg=None, dgv=None):
    p = N.LaProblem(a["B"], a["H"], a["n"], a["d_k"], a["d_v"], a["in_dt"], a["out_dt"], a["eps"])
    f = N.LaFeatureMap(a["fkind"], a["r"], a["omega"])
    g = N.LaGate(a["gkind"], a["tau"], a["gamma"], a["g"], a["gv"])
    return N.lib().la_backward(ctypes.byref(p), a["Q"], a["K"], a["V"], dO, ctypes.byref(f), a["causal"],
                               ctypes.byref(g), a["S0"], a["z0"], dQ, dK, dV, dg, dgv, a["ws"], a["ws_bytes"], None)


BAD_BACKWARD = [
    ("n=0", dict(n=0), {}, N.LA_ERR_INVALID_ARG),
    ("identity sel without dg", dict(fkind=N.LA_FMAP_IDENTITY, gkind=N.LA_GATE_SEL, g=FAKE + 6 * SP), {},
     N.LA_ERR_INVALID_ARG),
    ("sel without dg", dict(gkind=N.LA_GATE_SEL, g=FAKE + 6 * SP), {}, N.LA_ERR_INVALID_ARG),
    ("sel favor", dict(gkind=N.LA_GATE_SEL, g=FAKE + 6 * SP, fkind=N.LA_FMAP_FAVOR, r=256, omega=FAKE + 5 * SP),
     dict(dg=FAKE + 14 * SP), N.LA_ERR_UNSUPPORTED),
    ("outer without dgv", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP), dict(dg=FAKE + 14 * SP),
     N.LA_ERR_INVALID_ARG),
    ("outer without dg", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP), dict(dgv=FAKE + 15 * SP),
     N.LA_ERR_INVALID_ARG),
    ("dgv without outer", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP), dict(dg=FAKE + 14 * SP, dgv=FAKE + 15 * SP),
     N.LA_ERR_INVALID_ARG),
    ("outer no gv", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP), dict(dg=FAKE + 14 * SP, dgv=FAKE + 15 * SP),
     N.LA_ERR_INVALID_ARG),
    ("outer dgv misaligned", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP),
     dict(dg=FAKE + 14 * SP, dgv=FAKE + 15 * SP + 8), N.LA_ERR_INVALID_ARG),
    ("outer dgv aliases gv", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP),
     dict(dg=FAKE + 14 * SP, dgv=FAKE + 7 * SP + 256), N.LA_ERR_ALIAS),
    ("outer dgv aliases dg", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP),
     dict(dg=FAKE + 14 * SP, dgv=FAKE + 14 * SP + 512), N.LA_ERR_ALIAS),
    ("outer dV aliases gv", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP),
     dict(dg=FAKE + 14 * SP, dgv=FAKE + 15 * SP, dV=FAKE + 7 * SP), N.LA_ERR_ALIAS),
    ("outer favor", dict(gkind=N.LA_GATE_OUTER, g=FAKE + 6 * SP, gv=FAKE + 7 * SP, fkind=N.LA_FMAP_FAVOR, r=128,
                         omega=FAKE + 5 * SP), dict(dg=FAKE + 14 * SP, dgv=FAKE + 15 * SP), N.LA_ERR_UNSUPPORTED),
    ("sel dg aliases g", dict(gkind=N.LA_GATE_SEL, g=FAKE + 6 * SP), dict(dg=FAKE + 6 * SP + 1024), N.LA_ERR_ALIAS),
    ("sel dg in workspace", dict(gkind=N.LA_GATE_SEL, g=FAKE + 6 * SP), dict(dg=FAKE + 4 * SP + 4096),
     N.LA_ERR_ALIAS),
    ("noncausal favor", dict(causal=0, fkind=N.LA_FMAP_FAVOR, r=256, omega=FAKE + 5 * SP), {}, N.LA_ERR_UNSUPPORTED),
    ("noncausal identity", dict(causal=0, fkind=N.LA_FMAP_IDENTITY), {}, N.LA_ERR_UNSUPPORTED),
    ("noncausal dtype mix", dict(causal=0, in_dt=N.LA_F32), {}, N.LA_ERR_UNSUPPORTED),
    ("noncausal with S0", dict(causal=0, S0=FAKE + 7 * SP, z0=FAKE + 8 * SP), {}, N.LA_ERR_INVALID_ARG),
    ("noncausal d_v 96", dict(causal=0, d_v=96), {}, N.LA_ERR_UNSUPPORTED),
    ("noncausal gated", dict(causal=0, gkind=N.LA_GATE_DECAY, gamma=FAKE + 6 * SP), {}, N.LA_ERR_INVALID_ARG),
    ("favor r 256", dict(fkind=N.LA_FMAP_FAVOR, r=256, omega=FAKE + 5 * SP), {}, N.LA_ERR_UNSUPPORTED),
    ("favor r 32", dict(fkind=N.LA_FMAP_FAVOR, r=32, omega=FAKE + 5 * SP), {}, N.LA_ERR_UNSUPPORTED),
    ("favor r 128 d_v 32", dict(fkind=N.LA_FMAP_FAVOR, r=128, d_v=32, omega=FAKE + 5 * SP), {},
     N.LA_ERR_UNSUPPORTED),
    ("favor no omega", dict(fkind=N.LA_FMAP_FAVOR, r=128), {}, N.LA_ERR_INVALID_ARG),
    ("gla without dg", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP), {}, N.LA_ERR_INVALID_ARG),
    ("dg without gla", {}, dict(dg=FAKE + 14 * SP), N.LA_ERR_INVALID_ARG),
    ("gla no g", dict(gkind=N.LA_GATE_GLA), dict(dg=FAKE + 14 * SP), N.LA_ERR_INVALID_ARG),
    ("gla tau 0", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP, tau=0.0), dict(dg=FAKE + 14 * SP), N.LA_ERR_INVALID_ARG),
    ("gla dg misaligned", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP), dict(dg=FAKE + 14 * SP + 8),
     N.LA_ERR_INVALID_ARG),
    ("gla dg aliases g", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP), dict(dg=FAKE + 6 * SP + 256), N.LA_ERR_ALIAS),
    ("gla dg aliases dK", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP), dict(dg=FAKE + 12 * SP + 256),
     N.LA_ERR_ALIAS),
    ("gla dg in workspace", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP), dict(dg=FAKE + 4 * SP + 4096),
     N.LA_ERR_ALIAS),
    ("gla dQ aliases g", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP), dict(dQ=FAKE + 6 * SP, dg=FAKE + 14 * SP),
     N.LA_ERR_ALIAS),
    ("gla favor", dict(gkind=N.LA_GATE_GLA, g=FAKE + 6 * SP, fkind=N.LA_FMAP_FAVOR, r=256, omega=FAKE + 5 * SP),
     dict(dg=FAKE + 14 * SP), N.LA_ERR_UNSUPPORTED),
    ("d_v 32", dict(d_v=32), {}, N.LA_ERR_UNSUPPORTED),
    ("d_k 32", dict(d_k=32, r=32), {}, N.LA_ERR_UNSUPPORTED),
    ("fp32", dict(in_dt=N.LA_F32, out_dt=N.LA_F32), {}, N.LA_ERR_UNSUPPORTED),
    ("decay no gamma", dict(gkind=N.LA_GATE_DECAY), {}, N.LA_ERR_INVALID_ARG),
    ("dO null", {}, dict(dO=None), N.LA_ERR_INVALID_ARG),
    ("dK null", {}, dict(dK=None), N.LA_ERR_INVALID_ARG),
    ("dQ misaligned", {}, dict(dQ=FAKE + 11 * SP + 8), N.LA_ERR_INVALID_ARG),
    ("S0 without z0", dict(S0=FAKE + 7 * SP), {}, N.LA_ERR_INVALID_ARG),
    ("dQ aliases K", {}, dict(dQ=FAKE + SP + 256), N.LA_ERR_ALIAS),
    ("dV aliases dO", {}, dict(dV=FAKE + 10 * SP), N.LA_ERR_ALIAS),
    ("dK aliases dQ", {}, dict(dK=FAKE + 11 * SP + 512), N.LA_ERR_ALIAS),
    ("ws null", dict(ws=None), {}, N.LA_ERR_WORKSPACE),
    ("ws small", dict(ws_bytes=1024), {}, N.LA_ERR_WORKSPACE),
    ("ws misaligned", dict(ws=FAKE + 4 * SP + 16), {}, N.LA_ERR_WORKSPACE),
]


@needs_lib
@no_gpu
@pytest.mark.parametrize("name,over,ptrs,want", BAD_BACKWARD, ids=[b[0] for b in BAD_BACKWARD])
def test_backward_rejects(name, over, ptrs, want):
    assert _backward(_args(**over), **ptrs) == want


@needs_lib
def test_backward_workspace_size():
    lib = N.lib()

    def size(B, H, n, d, dv, gk=N.LA_GATE_NONE):
        p = N.LaProblem(B, H, n, d, dv, N.LA_BF16, N.LA_BF16, 1e-6)
        f = N.LaFeatureMap(N.LA_FMAP_ELU1, d, None)
        g = N.LaGate(gk, 16.0, None, None)
        out = ctypes.c_size_t(0)
        assert lib.la_backward_workspace_size(ctypes.byref(p), ctypes.byref(f), 1, ctypes.byref(g),
                                              ctypes.byref(out)) == N.LA_OK
        return out.value
    # headline shape: 8 segments; forward and reverse states, g (bf16) and h per token, 256-aligned regions
    BH, P, n = 64, 8, 4096
    states = BH * P * 64 * 64 * 4
    zs = BH * P * 64 * 4
    assert size(4, 16, n, 64, 64) == 2 * states + 2 * zs + BH * n * 64 * 2 + BH * n * 4
    assert size(4, 16, n, 64, 64, N.LA_GATE_DECAY) == size(4, 16, n, 64, 64)
    # GLA adds dQ~ . Q~ per token and feature (fp32) and the segments' summed log-gates
    assert size(4, 16, n, 64, 64, N.LA_GATE_GLA) == size(4, 16, n, 64, 64) + BH * n * 64 * 4 + zs
    # the selective gate runs the GLA passes with its one input per token: the same regions
    assert size(4, 16, n, 64, 64, N.LA_GATE_SEL) == size(4, 16, n, 64, 64, N.LA_GATE_GLA)
    # the outer-product gate: the GLA regions on its own segment plan, plus dO * o per token and value
    # column (fp32) and the segments' summed value-side log-gates
    p = N.LaProblem(4, 16, n, 64, 64, N.LA_BF16, N.LA_BF16, 1e-6)
    f = N.LaFeatureMap(N.LA_FMAP_ELU1, 64, None)
    g = N.LaGate(N.LA_GATE_OUTER, 16.0, None, None)
    segs, seg_len = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.la_forward_segments(ctypes.byref(p), ctypes.byref(f), 1, ctypes.byref(g), ctypes.byref(segs),
                                   ctypes.byref(seg_len)) == N.LA_OK
    Po = segs.value
    assert Po > 1
    so, zo = BH * Po * 64 * 64 * 4, BH * Po * 64 * 4
    assert size(4, 16, n, 64, 64, N.LA_GATE_OUTER) == (2 * so + 2 * zo + BH * n * 64 * 2 + BH * n * 4 +
                                                       BH * n * 64 * 4 + zo + BH * n * 64 * 4 + BH * Po * 64 * 4)

    def size128(B, H, n, dv, gk=N.LA_GATE_NONE):
        p = N.LaProblem(B, H, n, 128, dv, N.LA_BF16, N.LA_BF16, 1e-6)
        f = N.LaFeatureMap(N.LA_FMAP_ELU1, 128, None)
        g = N.LaGate(gk, 16.0, None, None)
        out = ctypes.c_size_t(0)
        assert lib.la_backward_workspace_size(ctypes.byref(p), ctypes.byref(f), 1, ctypes.byref(g),
                                              ctypes.byref(out)) == N.LA_OK
        return out.value
    # 128 x 128 states run as two (128, 64) halves of the value columns, one after the other, on
    # the halves' workspace, plus one half of a carried-in state (fp32 [BH][128][64])
    for gk in (N.LA_GATE_NONE, N.LA_GATE_GLA):
        assert size128(2, 16, 16384, 128, gk) == size128(2, 16, 16384, 64, gk) + 32 * 128 * 64 * 4

    def size_favor(B, H, n, d, r, dv):
        p = N.LaProblem(B, H, n, d, dv, N.LA_BF16, N.LA_BF16, 1e-6)
        f = N.LaFeatureMap(N.LA_FMAP_FAVOR, r, ctypes.c_void_p(FAKE))
        g = N.LaGate(N.LA_GATE_NONE, 16.0, None, None)
        out = ctypes.c_size_t(0)
        assert lib.la_backward_workspace_size(ctypes.byref(p), ctypes.byref(f), 1, ctypes.byref(g),
                                              ctypes.byref(out)) == N.LA_OK
        return out.value
    # FAVOR+ runs the passes at width r on phi(Q), phi(K) and their gradients (bf16 [BH][n][r] each)
    assert size_favor(1, 8, 32768, 64, 128, 64) == size128(1, 8, 32768, 64) + 4 * 8 * 32768 * 128 * 2
    assert size_favor(2, 2, 300, 128, 128, 128) == size128(2, 2, 300, 128) + 4 * 4 * 300 * 128 * 2
    assert size_favor(1, 1, 65, 32, 64, 64) == size(1, 1, 65, 64, 64) + 4 * 65 * 64 * 2


# ------------------------------------------------------------------ serving batch (validation, no launch)

def _batch_call(a, cu=None, num_seqs=None, max_seqlen=None, S=FAKE + 20 * SP, z=FAKE + 21 * SP,
                slot_ids=FAKE + 22 * SP, num_slots=8, flags=3, out=None):
    p = N.LaProblem(a["B"], a["H"], a["n"], a["d_k"], a["d_v"], a["in_dt"], a["out_dt"], a["eps"])
    f = N.LaFeatureMap(a["fkind"], a["r"], a["omega"])
    g = N.LaGate(a["gkind"], a["tau"], a["gamma"], a["g"], a["gv"])
    b = N.LaBatch(cu, a["B"] if num_seqs is None else num_seqs, a["n"] if max_seqlen is None else max_seqlen, S, z,
                  slot_ids, num_slots, flags)
    return N.lib().la_forward_batch(ctypes.byref(p), ctypes.byref(b), a["Q"], a["K"], a["V"], ctypes.byref(f),
                                    ctypes.byref(g), a["out"] if out is None else out, a["ws"], a["ws_bytes"], None)


BAD_BATCH = [
    ("num_seqs != B", {}, dict(num_seqs=3), N.LA_ERR_INVALID_ARG),
    ("max_seqlen != n", {}, dict(max_seqlen=50), N.LA_ERR_INVALID_ARG),
    ("cu with B 2", {}, dict(cu=FAKE + 23 * SP, num_seqs=4, max_seqlen=50), N.LA_ERR_INVALID_ARG),
    ("cu num_seqs 0", dict(B=1), dict(cu=FAKE + 23 * SP, num_seqs=0, max_seqlen=50), N.LA_ERR_INVALID_ARG),
    ("cu max_seqlen 0", dict(B=1), dict(cu=FAKE + 23 * SP, num_seqs=4, max_seqlen=0), N.LA_ERR_INVALID_ARG),
    ("cu max_seqlen > n", dict(B=1), dict(cu=FAKE + 23 * SP, num_seqs=4, max_seqlen=101), N.LA_ERR_INVALID_ARG),
    ("cu misaligned", dict(B=1), dict(cu=FAKE + 23 * SP + 2, num_seqs=4, max_seqlen=50), N.LA_ERR_INVALID_ARG),
    ("bad flags", {}, dict(flags=4), N.LA_ERR_INVALID_ARG),
    ("no slots", {}, dict(num_slots=0), N.LA_ERR_INVALID_ARG),
    ("S null", {}, dict(S=None), N.LA_ERR_INVALID_ARG),
    ("slot_ids null", {}, dict(slot_ids=None), N.LA_ERR_INVALID_ARG),
    ("S misaligned", {}, dict(S=FAKE + 20 * SP + 8), N.LA_ERR_INVALID_ARG),
    ("noncausal-only dtype", dict(in_dt=N.LA_F32, out_dt=N.LA_F32), {}, N.LA_ERR_UNSUPPORTED),
    ("pool over Q", {}, dict(S=FAKE + 256), N.LA_ERR_ALIAS),
    ("pool over out", {}, dict(z=FAKE + 3 * SP + 256), N.LA_ERR_ALIAS),
    ("out over cu", dict(B=1), dict(cu=FAKE + 3 * SP, num_seqs=4, max_seqlen=50), N.LA_ERR_ALIAS),
    ("pool over slot ids", {}, dict(slot_ids=FAKE + 20 * SP + 64), N.LA_ERR_ALIAS),
    ("ws small", dict(ws_bytes=16), {}, N.LA_ERR_WORKSPACE),
    ("d_v 32 multi-token", dict(d_v=32), {}, N.LA_ERR_UNSUPPORTED),
    ("d_v 32 ragged", dict(B=1, d_v=32), dict(cu=FAKE + 23 * SP, num_seqs=4, max_seqlen=50), N.LA_ERR_UNSUPPORTED),
    ("favor r 32 multi-token", dict(fkind=N.LA_FMAP_FAVOR, r=32, omega=FAKE + 5 * SP), {}, N.LA_ERR_UNSUPPORTED),
]


@needs_lib
@no_gpu
@pytest.mark.parametrize("name,over,kw,want", BAD_BATCH, ids=[b[0] for b in BAD_BATCH])
def test_batch_rejects(name, over, kw, want):
    assert _batch_call(_args(**over), **kw) == want


@needs_lib
def test_batch_workspace_size():
    """Without cu_seqlens a batch needs what la_forward needs. A ragged batch
    is planned from its total and longest lengths: segments of
    ceil((total / 64 + num_seqs) * H / 512) chunks (at most the longest
    sequence's), P of them covering the longest sequence, fp32 segment states
    for num_seqs * H * P (0 when P is 1)."""
    lib = N.lib()

    def size(B, n, cu, num_seqs, max_seqlen, flags=0):
        p = N.LaProblem(B, 16, n, 64, 64, N.LA_BF16, N.LA_BF16, 1e-6)
        f = N.LaFeatureMap(N.LA_FMAP_ELU1, 64, None)
        g = N.LaGate(N.LA_GATE_NONE, 16.0, None, None)
        b = N.LaBatch(cu, num_seqs, max_seqlen, None, None, None, 1, flags)
        out = ctypes.c_size_t(0)
        assert lib.la_forward_batch_workspace_size(ctypes.byref(p), ctypes.byref(b), ctypes.byref(f),
                                                   ctypes.byref(g), ctypes.byref(out)) == N.LA_OK
        return out.value

    def fwd(B, n):
        p = N.LaProblem(B, 16, n, 64, 64, N.LA_BF16, N.LA_BF16, 1e-6)
        f = N.LaFeatureMap(N.LA_FMAP_ELU1, 64, None)
        g = N.LaGate(N.LA_GATE_NONE, 16.0, None, None)
        out = ctypes.c_size_t(0)
        assert lib.la_forward_workspace_size(ctypes.byref(p), ctypes.byref(f), 1, ctypes.byref(g),
                                             ctypes.byref(out)) == N.LA_OK
        return out.value
    assert size(4, 4096, None, 4, 4096) == fwd(4, 4096)

    def ragged(total, nseq, max_len, H=16, r=64, dv=64):
        seg = min(max(-(-((-(-total // 64) + nseq) * H) // 512), 1), -(-max_len // 64))
        P = -(-(-(-max_len // 64)) // seg)
        return 0 if P <= 1 else nseq * H * P * (r * dv + r) * 4
    assert size(1, 40000, FAKE, 10, 4096) == ragged(40000, 10, 4096) == 10 * 16 * 4 * (64 * 64 + 64) * 4
    assert size(1, 8192, FAKE, 64, 4096) == ragged(8192, 64, 4096) > 0 == fwd(64, 4096)
    assert size(1, 40000, FAKE, 64, 128) == 0   # one segment per sequence: no workspace


@needs_lib
def test_causal_dv32_workspace():
    """Causal d_v = 32 runs the 64-column kernels on padded copies in the
    workspace: the 64-column problem's segment states, then bf16 V and out
    copies [B H n 64] and fp32 S0 and S_final copies [B H r 64], each region
    256-byte aligned (the outer-product gate adds a bf16 copy of gv)."""
    lib = N.lib()
    up = lambda x: -(-x // 256) * 256

    def size(dv, gk=N.LA_GATE_NONE, B=2, H=3, n=1000, d=64):
        p = N.LaProblem(B, H, n, d, dv, N.LA_BF16, N.LA_BF16, 1e-6)
        f = N.LaFeatureMap(N.LA_FMAP_ELU1, d, None)
        g = N.LaGate(gk, 16.0, None, None)
        out = ctypes.c_size_t(0)
        assert lib.la_forward_workspace_size(ctypes.byref(p), ctypes.byref(f), 1, ctypes.byref(g),
                                             ctypes.byref(out)) == N.LA_OK
        return out.value
    for gk, copies in ((N.LA_GATE_NONE, 2), (N.LA_GATE_GLA, 2), (N.LA_GATE_OUTER, 3)):
        B, H, n, d = 2, 3, 1000, 64
        pads = copies * up(B * H * n * 64 * 2) + 2 * up(B * H * d * 64 * 4)
        assert size(32, gk) == up(size(64, gk)) + pads
    # one segment: only the copies
    assert size(32, B=1, H=1, n=64) == 2 * up(64 * 64 * 2) + 2 * up(64 * 64 * 4)

    # FAVOR+ r = 32: the 64-feature problem's segment states, omega padded to 64 rows (bf16),
    # S0 / S_final copies [B H 64 d_v] and z0 / z_final copies [B H 64] (fp32)
    def fsize(r, dv, B=2, H=3, n=3000, d=64):
        p = N.LaProblem(B, H, n, d, dv, N.LA_BF16, N.LA_BF16, 1e-6)
        f = N.LaFeatureMap(N.LA_FMAP_FAVOR, r, ctypes.c_void_p(FAKE))
        g = N.LaGate(N.LA_GATE_NONE, 16.0, None, None)
        out = ctypes.c_size_t(0)
        assert lib.la_forward_workspace_size(ctypes.byref(p), ctypes.byref(f), 1, ctypes.byref(g),
                                             ctypes.byref(out)) == N.LA_OK
        return out.value
    BH = 6
    assert fsize(32, 64) == up(fsize(64, 64)) + up(64 * 64 * 2) + 2 * up(BH * 64 * 64 * 4) + 2 * up(BH * 64 * 4)
    # both at once: r = 32 and d_v = 32
    assert fsize(32, 32) == (up(fsize(64, 64)) + 2 * up(BH * 3000 * 64 * 2) + up(64 * 64 * 2) +
                             2 * up(BH * 64 * 64 * 4) + 2 * up(BH * 64 * 4))


@needs_lib
@no_gpu
def test_valid_calls_without_a_device_return_hip_error():
    """A well-formed call on a host with no GPU gets LA_ERR_HIP from the HIP
    runtime's refusal, not a crash: every argument passes validation (fake,
    aligned, non-overlapping device addresses that are never dereferenced),
    so the first HIP call is the one that fails."""
    lib = N.lib()
    at = lambda i: ctypes.c_void_p(0x10000000 * (i + 1))  # 256 MB apart: no two ranges overlap
    elu = N.LaFeatureMap(N.LA_FMAP_ELU1, 64, None)
    none = N.LaGate(N.LA_GATE_NONE, 1.0, None, None)
    for causal, n in ((1, 1000), (0, 1000)):
        p = N.LaProblem(2, 4, n, 64, 64, N.LA_BF16, N.LA_BF16, 1e-6)
        ws = ctypes.c_size_t(0)
        assert lib.la_forward_workspace_size(ctypes.byref(p), ctypes.byref(elu), causal, ctypes.byref(none),
                                             ctypes.byref(ws)) == N.LA_OK
        st = lib.la_forward(ctypes.byref(p), at(0), at(1), at(2), ctypes.byref(elu), causal, ctypes.byref(none),
                            None, None, None, None, at(3), at(4) if ws.value else None, ws.value, None)
        assert st == N.LA_ERR_HIP, (causal, st)
    p1 = N.LaProblem(2, 4, 1, 64, 64, N.LA_BF16, N.LA_F32, 1e-6)
    assert lib.la_decode_step(ctypes.byref(p1), at(0), at(1), at(2), at(3), at(4), ctypes.byref(elu),
                              ctypes.byref(none), at(5), None) == N.LA_ERR_HIP
    p = N.LaProblem(2, 4, 1000, 64, 64, N.LA_BF16, N.LA_BF16, 1e-6)
    ws = ctypes.c_size_t(0)
    assert lib.la_backward_workspace_size(ctypes.byref(p), ctypes.byref(elu), 1, ctypes.byref(none),
                                          ctypes.byref(ws)) == N.LA_OK
    assert lib.la_backward(ctypes.byref(p), at(0), at(1), at(2), at(3), ctypes.byref(elu), 1, ctypes.byref(none),
                           None, None, at(4), at(5), at(6), None, None, at(7), ws.value, None) == N.LA_ERR_HIP
    assert lib.la_feature_map_apply(ctypes.byref(elu), 1000, 64, N.LA_BF16, at(0), at(1), None) == N.LA_ERR_HIP


@needs_lib
def test_timing_bracket_rules():
    """la_timing_begin / la_timing_end: argument checks and nesting, without a
    launch (an empty bracket records nothing when no events are given)."""
    lib = N.lib()
    n = ctypes.c_int32(-1)
    assert lib.la_timing_end(None, ctypes.byref(n)) == N.LA_ERR_INVALID_ARG  # none open
    assert lib.la_timing_begin(None, 2) == N.LA_ERR_INVALID_ARG
    assert lib.la_timing_begin(None, -1) == N.LA_ERR_INVALID_ARG
    nulls = (ctypes.c_void_p * 2)(None, None)
    assert lib.la_timing_begin(nulls, 2) == N.LA_ERR_INVALID_ARG
    assert lib.la_timing_begin(None, 0) == N.LA_OK
    assert lib.la_timing_begin(None, 0) == N.LA_ERR_INVALID_ARG  # brackets do not nest
    assert lib.la_timing_end(None, ctypes.byref(n)) == N.LA_OK
    assert n.value == 0
    assert lib.la_timing_end(None, None) == N.LA_ERR_INVALID_ARG
