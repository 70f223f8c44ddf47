"""Seeded synthetic workloads (shapes, distributions, generators).

Shared by tests, the smoke check and the benchmark; contains none of the
attention method's arithmetic.
"""
from .configs import WORKLOADS, HEADLINE, Workload, describe  # noqa: F401
from .generate import make_inputs, to_f64, retnet_gammas, orthogonal_gaussian_omega, incoming_gradient  # noqa: F401
from .generate import serving_lengths, strong_gate_input  # noqa: F401
