"""A seeded sweep of layer shapes the hand-picked cases do not pin: each one
against the oracle (staged and end to end, decode kernels) and the prefill
kernels' rows bitwise equal to the decode kernels' rows.  The shapes are
drawn once from a fixed seed, so the list is the same on every run."""
import numpy as np
import pytest

from block_scaled_fp8xfp4_amd import mxmoe
from gpu_common import host, say, small_workload
from test_gpu_parity import ffn_parity

pytestmark = pytest.mark.gpu


def sweep_shapes(n=12, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.integers(2, 97))
        out.append(dict(seed=600 + i, T=int(rng.integers(1, 201)), H=256 * int(rng.integers(1, 9)), E=E,
                        k=int(rng.integers(1, min(8, E) + 1)), I=32 * int(rng.integers(1, 20)),
                        skip=float(rng.choice([0.0, 0.3]))))
    return out


@pytest.mark.parametrize("shape", sweep_shapes(), ids=lambda s: "T{T}_H{H}_E{E}_k{k}_I{I}".format(**s))
def test_sweep_shape(shape):
    inp, r, layer = small_workload(**shape)
    say(f"sweep {shape}")
    # I down to 32: one requant code flip moves y by up to ~1e-2 of max|y| (as for the small shapes)
    y_dec = ffn_parity(inp, r, layer, what=str(shape), e2e_tol=3e-2)
    old = mxmoe.set_ffn_path(2)
    try:
        y_pre, _, _ = layer.gpu_y()
    finally:
        mxmoe.set_ffn_path(old)
    assert mxmoe.last_variant().startswith("ffn:gu_prefill")
    assert np.array_equal(host(y_pre).view(np.uint32), y_dec.view(np.uint32)), "prefill rows differ from decode rows"
