"""GPU parity of the softmax-attention baseline kernel (la_softmax_attention)
against the fp64 oracle (oracle/softmax.py) on the same seeded bf16 inputs.

Tolerance: the row-relative 1e-2 of the bf16 paths. Each output is a convex
combination of the values; the kernel rounds the softmax weights to bf16 for
the matrix cores (2^-9 relative each) and the output to bf16 (2^-9), with the
scores, the running maximum and the row sums in fp32.
"""
import numpy as np
import pytest
import torch

from oracle import softmax as osm
from workloads import WORKLOADS, make_inputs, to_f64
from _helpers import TOL_BF16, check_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from kernelized_sequence_mixing_amd import _native
    _native.lib()


def _inputs(B, H, n, d, seed=0):
    wl = WORKLOADS["causal_elu1"].resized(d_k=d, d_v=d, r=d, qk_scale=1.0, v_scale=1.0)
    return make_inputs(wl, seed=seed, B=B, H=H, n=n)


def _run(inp, causal):
    import kernelized_sequence_mixing_amd as ksm
    out = ksm.softmax_attention(dev(inp["Q"]), dev(inp["K"]), dev(inp["V"]), causal=causal)
    torch.cuda.synchronize()
    return out.cpu()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,n", [(2, 4, 300), (1, 2, 1000), (2, 3, 129), (1, 1, 1), (2, 1, 63), (2, 1, 64),
                                   (2, 1, 65), (3, 2, 128)])
def test_softmax_parity_small(causal, d, B, H, n):
    """Every head, element by element: ragged key and query blocks, tiny n,
    blocks of exactly 64 and 128."""
    inp = _inputs(B, H, n, d, seed=n + d)
    out = _run(inp, causal)
    Q, K, V = (to_f64(inp[k]) for k in ("Q", "K", "V"))
    check_close(out, osm.softmax_attention(Q, K, V, causal=causal), TOL_BF16,
                f"softmax {'causal' if causal else 'full'} d{d} B{B} H{H} n{n}")


@pytest.mark.parametrize("n", [4096, 32768])
def test_softmax_matched_shape_sampled_rows(n):
    """The benchmark's shapes (H16 d64) on sampled rows of two heads, against
    the per-row oracle; every output finite and inside the values' range."""
    B = 4 if n == 4096 else 1
    inp = _inputs(B, 16, n, 64, seed=7)
    out = _run(inp, True)
    o = to_f64(out)
    assert np.isfinite(o).all()
    V = to_f64(inp["V"])
    assert np.all(np.abs(o) <= np.max(np.abs(V), axis=(2, 3), keepdims=True) * (1 + 1e-2))
    rows = [0, 1, 63, 64, 127, 128, n // 2, n - 1]
    for b, h in [(0, 0), (B - 1, 15)]:
        sl = lambda x: to_f64(x)[b:b + 1, h:h + 1]
        ref = osm.softmax_attention_rows(sl(inp["Q"]), sl(inp["K"]), sl(inp["V"]), rows, causal=True)
        check_close(out[b:b + 1, h:h + 1, rows], ref, TOL_BF16, f"softmax n{n} head ({b},{h}) rows")


def test_softmax_causal_mask_exact_zero():
    """V = 0 except v_p = 1 in one column: outputs before p are exactly 0."""
    inp = _inputs(1, 1, 400, 64, seed=9)
    for p in (0, 63, 64, 127, 128, 399):
        V = torch.zeros_like(inp["V"])
        V[0, 0, p, 5] = 1.0
        out = to_f64(_run({**inp, "V": V}, True))
        assert np.all(out[0, 0, :p] == 0.0), p
        assert out[0, 0, p, 5] > 0.0
        other = np.delete(out[0, 0], 5, axis=1)
        assert np.all(other == 0.0)


def test_softmax_deterministic():
    inp = _inputs(2, 4, 777, 64, seed=11)
    a, b = _run(inp, True), _run(inp, True)
    assert torch.equal(a, b)
