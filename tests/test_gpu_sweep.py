"""A seeded sweep of layer shapes the hand-picked cases do not pin: each one
against the oracle on both kernel paths (staged and end to end), and the
prefill kernels' rows bitwise equal to the decode kernels' rows.  The shapes are
drawn once from a fixed seed, so the list is the same on every run."""
import numpy as np
import pytest

from gpu_common import ffn_parity, say, small_workload

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
    y_dec = ffn_parity(inp, r, layer, what=str(shape), path=1)
    y_pre = ffn_parity(inp, r, layer, what=str(shape), path=2)
    assert np.array_equal(y_pre.view(np.uint32), y_dec.view(np.uint32)), "prefill rows differ from decode rows"
