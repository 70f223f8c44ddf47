"""The seeded generators: determinism, dtypes, rounding, and the omega draw."""
import hashlib

import numpy as np
import torch

from workloads import WORKLOADS, make_inputs, orthogonal_gaussian_omega, retnet_gammas


def _digest(d):
    h = hashlib.sha256()
    for k in sorted(d):
        v = d[k]
        if isinstance(v, torch.Tensor):
            h.update(k.encode())
            h.update(v.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def test_generators_deterministic():
    for name in WORKLOADS:
        a = make_inputs(name, seed=0, B=1, H=2, n=70) if not WORKLOADS[name].decode else make_inputs(name, B=2, H=2)
        b = make_inputs(name, seed=0, B=1, H=2, n=70) if not WORKLOADS[name].decode else make_inputs(name, B=2, H=2)
        assert _digest(a) == _digest(b), name
    c = make_inputs("causal_elu1", seed=1, B=1, H=2, n=70)
    assert _digest(c) != _digest(make_inputs("causal_elu1", seed=0, B=1, H=2, n=70))


def test_shapes_and_dtypes():
    d = make_inputs("gla_gate", B=1, H=2, n=33)
    assert d["Q"].shape == (1, 2, 33, 128) and d["Q"].dtype == torch.bfloat16
    assert d["g"].shape == (1, 2, 33, 128)
    d = make_inputs("favor_causal", B=1, H=2, n=10)
    assert d["omega"].shape == (256, 64) and d["omega"].dtype == torch.bfloat16
    d = make_inputs("noncausal_elu1_f32")
    assert d["Q"].shape == (1, 1, 256, 32) and d["Q"].dtype == torch.float32
    d = make_inputs("gla_decode", B=3, H=2)
    assert d["S0"].shape == (3, 2, 128, 128) and d["S0"].dtype == torch.float32
    assert d["q"].shape == (3, 2, 128) and torch.all(d["z0"] > 0)
    d = make_inputs("retnet_decay", B=1, H=8, n=5)
    np.testing.assert_array_equal(d["gamma"].numpy(), np.float32(1) - np.float32(2.0) ** -(5 + np.arange(8.0, dtype=np.float32)))


def test_bf16_cast_is_round_to_nearest_even():
    # 1 + 2^-8 sits exactly halfway between bf16 neighbours 1 and 1 + 2^-7;
    # ties go to the even mantissa (1.0); 1 + 3*2^-8 ties up to 1 + 2^-6.
    x = torch.tensor([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20], dtype=torch.float32)
    y = x.to(torch.bfloat16).to(torch.float32)
    assert y.tolist() == [1.0, 1 + 2 ** -6, 1 + 2 ** -7]


def test_omega_blocks_orthogonal():
    rng = np.random.default_rng(0)
    om = orthogonal_gaussian_omega(rng, 256, 64).astype(np.float64)
    for b in range(4):
        blk = om[64 * b:64 * (b + 1)]
        unit = blk / np.linalg.norm(blk, axis=1, keepdims=True)
        np.testing.assert_allclose(unit @ unit.T, np.eye(64), atol=1e-5)
    norms = np.linalg.norm(om, axis=1)
    assert 7.0 < norms.mean() < 9.0  # chi distribution with 64 d.o.f.: mean ~ 7.98


def test_retnet_gammas():
    g = retnet_gammas(8)
    assert g[0] == np.float32(1 - 1 / 32) and g[7] == np.float32(1 - 2.0 ** -12)
