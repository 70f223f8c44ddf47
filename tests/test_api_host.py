"""Host-side argument checks of the Python binding (CPU only, no library call).

The C ABI indexes the gate inputs g, gv and the FAVOR+ frequencies omega with
the element size of the input dtype, so a tensor of another dtype would be read
wrongly or past its end on the device. The binding must refuse such a call with
a TypeError before it reaches the library. The device check is relaxed to any
tensor here and the library is replaced by a stub that fails if it is touched.
"""
import pytest
import torch

from kernelized_sequence_mixing_amd import api
from kernelized_sequence_mixing_amd import _native


@pytest.fixture
def host_only(monkeypatch):
    def _dev(t, name):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        return t

    def _no_lib():
        raise AssertionError("the library was called before the dtype check")

    monkeypatch.setattr(api, "_dev", _dev)
    monkeypatch.setattr(_native, "lib", _no_lib)
    return api


B, H, n, d = 2, 3, 5, 64
F32, BF16 = torch.float32, torch.bfloat16


def qkv(dtype):
    return (torch.zeros(B, H, n, d, dtype=dtype), torch.zeros(B, H, n, d, dtype=dtype),
            torch.zeros(B, H, n, d, dtype=dtype))


@pytest.mark.parametrize("kind", ["gla", "sel", "outer_g", "outer_gv"])
@pytest.mark.parametrize("in_dt,g_dt", [(F32, BF16), (BF16, F32)])
def test_forward_gate_dtype(host_only, kind, in_dt, g_dt):
    Q, K, V = qkv(in_dt)
    if kind == "gla":
        gate = ("gla", torch.zeros(B, H, n, d, dtype=g_dt), 16.0)
    elif kind == "sel":
        gate = ("sel", torch.zeros(B, H, n, dtype=g_dt), 16.0)
    elif kind == "outer_g":
        gate = ("outer", torch.zeros(B, H, n, d, dtype=g_dt), torch.zeros(B, H, n, d, dtype=in_dt), 16.0)
    else:
        gate = ("outer", torch.zeros(B, H, n, d, dtype=in_dt), torch.zeros(B, H, n, d, dtype=g_dt), 16.0)
    with pytest.raises(TypeError, match="input dtype"):
        host_only.forward(Q, K, V, gate=gate)
    with pytest.raises(TypeError, match="input dtype"):
        host_only.forward_batch(Q, K, V, gate=gate)


@pytest.mark.parametrize("kind", ["gla", "sel"])
def test_backward_gate_dtype(host_only, kind):
    Q, K, V = qkv(BF16)
    shape = (B, H, n, d) if kind == "gla" else (B, H, n)
    with pytest.raises(TypeError, match="input dtype"):
        host_only.backward(Q, K, V, torch.zeros_like(V), gate=(kind, torch.zeros(shape, dtype=F32), 16.0))


@pytest.mark.parametrize("kind", ["gla", "sel", "outer_g", "outer_gv", "omega"])
def test_decode_dtype(host_only, kind):
    # fp32 tokens with bf16 gate inputs: the kernel would read twice the bf16 buffer's size
    r = 64
    S = torch.zeros(B, H, r, d, dtype=F32)
    z = torch.zeros(B, H, r, dtype=F32)
    q = k = v = torch.zeros(B, H, d, dtype=F32)
    fmap, omega, gate = "elu1", None, None
    if kind == "gla":
        gate = ("gla", torch.zeros(B, H, r, dtype=BF16), 16.0)
    elif kind == "sel":
        gate = ("sel", torch.zeros(B, H, dtype=BF16), 16.0)
    elif kind == "outer_g":
        gate = ("outer", torch.zeros(B, H, r, dtype=BF16), torch.zeros(B, H, d, dtype=F32), 16.0)
    elif kind == "outer_gv":
        gate = ("outer", torch.zeros(B, H, r, dtype=F32), torch.zeros(B, H, d, dtype=BF16), 16.0)
    else:
        fmap, omega = "favor", torch.zeros(r, d, dtype=BF16)
    with pytest.raises(TypeError, match="input dtype"):
        host_only.decode_step(S, z, q, k, v, fmap=fmap, omega=omega, gate=gate)


def test_batch_and_feature_map_omega_dtype(host_only):
    Q, K, V = qkv(BF16)
    omega = torch.zeros(256, d, dtype=F32)
    with pytest.raises(TypeError, match="input dtype"):
        host_only.forward_batch(Q, K, V, fmap="favor", omega=omega)
    with pytest.raises(TypeError, match="input dtype"):
        host_only.forward(Q, K, V, fmap="favor", omega=omega)
    with pytest.raises(TypeError, match="input dtype"):
        host_only.feature_map(Q, fmap="favor", omega=omega)
