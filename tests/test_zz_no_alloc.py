"""la_forward_noalloc (the library's fixed scratch array in place of a
workspace) against la_forward (a caller workspace) through the C ABI: the two
run the same kernels on the same plan, so their outputs and final states must
agree bit for bit. Two calls in a row, the second smaller than the first (the
array keeps the first call's contents), plus the host-side size limit."""
import ctypes

import numpy as np
import pytest
import torch

from workloads import WORKLOADS, make_inputs
from _helpers import dev, gpu_gate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _pair(inp):
    """(out, S, z) of la_forward and of la_forward_noalloc on the same inputs."""
    import kernelized_sequence_mixing_amd as ksm
    Q, K, V = dev(inp["Q"]), dev(inp["K"]), dev(inp["V"])
    om = dev(inp.get("omega"))
    gate = gpu_gate(inp)
    ref, Sr, zr = ksm.forward(Q, K, V, fmap=inp["fmap"], omega=om, causal=True, gate=gate, eps=inp["eps"],
                              return_state=True)
    out = torch.full_like(ref, float("nan"))
    S = torch.full_like(Sr, float("nan"))
    z = torch.full_like(zr, float("nan"))
    ksm.forward_noalloc(Q, K, V, fmap=inp["fmap"], omega=om, causal=True, gate=gate, eps=inp["eps"], out=out,
                        S_final=S, z_final=z)
    torch.cuda.synchronize()
    return (ref.cpu(), Sr.cpu(), zr.cpu()), (out.cpu(), S.cpu(), z.cpu())


def _same(a, b, what):
    for x, y, nm in zip(a, b, ("out", "S", "z")):
        assert torch.equal(x, y), f"{what}: {nm} differs"
    print(f"  {what}: bit-equal", flush=True)


def test_noalloc_matches_forward_twice_in_a_row():
    """The GLA workload at full size (17 MB of segment states), then a smaller
    ungated problem with a ragged tail, then the first again."""
    import kernelized_sequence_mixing_amd as ksm
    wl = WORKLOADS["gla_gate"]
    need = ksm.workspace_size(wl.B, wl.H, wl.n, wl.d_k, wl.d_v, gate_kind="gla")
    from kernelized_sequence_mixing_amd import _native as N
    assert 0 < need <= N.LA_NOALLOC_SCRATCH_BYTES
    big = make_inputs(wl, seed=0)
    a, b = _pair(big)
    _same(a, b, "GLA B2 H16 n16384 d128")
    small = make_inputs(WORKLOADS["causal_elu1"], seed=1, B=2, H=4, n=1285)
    a, b = _pair(small)
    _same(a, b, "elu+1 B2 H4 n1285 d64")
    a, b = _pair(big)
    _same(a, b, "GLA again")


def test_noalloc_rejects_problems_beyond_the_array():
    """A problem whose workspace exceeds the array is refused on the host
    (LA_ERR_WORKSPACE) before anything is launched."""
    from kernelized_sequence_mixing_amd import _native as N
    lib = N.lib()
    # FAVOR+ r 256 on one long head: 512 segments of fp32 states, 32.5 MiB
    x = torch.empty(16, device="cuda")
    p = N.LaProblem(1, 1, 65536, 64, 64, N.LA_BF16, N.LA_BF16, 1e-6)
    f = N.LaFeatureMap(N.LA_FMAP_FAVOR, 256, x.data_ptr())
    g = N.LaGate(N.LA_GATE_NONE, 1.0, None, None)
    need = ctypes.c_size_t(0)
    assert lib.la_forward_workspace_size(ctypes.byref(p), ctypes.byref(f), 1, ctypes.byref(g),
                                         ctypes.byref(need)) == N.LA_OK
    assert need.value > N.LA_NOALLOC_SCRATCH_BYTES
    ptr = ctypes.c_void_p(x.data_ptr())
    st = lib.la_forward_noalloc(ctypes.byref(p), ptr, ptr, ptr, ctypes.byref(f), 1, ctypes.byref(g), None, None,
                                None, None, ptr, None)
    assert st == N.LA_ERR_WORKSPACE
