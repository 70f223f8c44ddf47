"""fp64 CPU oracle for kernelized linear attention.

Test infrastructure: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package. It shares no code with the HIP
library.
"""
from .la_oracle import (  # noqa: F401
    FMAPS, GATES, phi_elu1, phi_favor, feature_map, gla_alpha, noncausal,
    kernel_weights, attention_from_weights, brute, causal_recurrent, causal_blocked,
    decode_step, softmax_score_matrix_bytes, outer_beta, brute_outer,
)
from .metrics import rowwise_rel_err  # noqa: F401
from . import la_backward  # noqa: F401
