"""CPU pins of the comparison rules the GPU parity tests apply (no GPU): the
rule that accepts an intermediate code of the GPU only where the gate/up
difference carries a across an E4M3 rounding boundary must accept exactly
such flips and reject anything else.  Mistakes are planted in oracle-made
arrays on the CPU."""
import numpy as np
import pytest

import oracle
from gpu_common import explain_code_differences, rel_err_cos


def intermediate(seed=3, n=64, I=96):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((n, 2 * I)) * 3).astype(np.float32)
    q, sc, a = oracle.swiglu_requant(h)
    return h, q, sc, a


def test_identical_intermediates_have_nothing_to_explain():
    h, q, sc, a = intermediate()
    assert explain_code_differences(q, sc, a, q, sc, a) == (0, 0)


def test_small_h_perturbations_flip_only_explainable_codes():
    """h perturbed by a few 1e-6 relative (the size of the matrix cores'
    accumulation error): the codes that change are all accepted, and there
    are some."""
    h, q, sc, a = intermediate(n=512)
    rng = np.random.default_rng(4)
    total = 0
    for eps in (3e-6, 1e-5, 1e-4):
        h2 = (h.astype(np.float64) * (1 + eps * rng.standard_normal(h.shape))).astype(np.float32)
        q2, sc2, a2 = oracle.swiglu_requant(h2)
        nel, nsc = explain_code_differences(q2, sc2, a2, q, sc, a)
        assert nel == int(((q2 != q) & np.repeat(sc2 == sc, 32, axis=1)).sum())
        total += nel + nsc
    assert total > 0


def test_planted_code_error_is_rejected():
    h, q, sc, a = intermediate()
    bad = q.copy()
    r, i = 5, 17
    bad[r, i] = (int(bad[r, i]) & 0x80) | min(0x7E, (int(bad[r, i]) & 0x7F) + 1)   # a code one step off
    with pytest.raises(AssertionError):
        explain_code_differences(bad, sc, a, q, sc, a)                  # same a: no boundary between them
    bad[r, i] = (int(q[r, i]) & 0x80) | max(0, (int(q[r, i]) & 0x7F) - 2)            # two steps off
    a2 = a.copy()
    with pytest.raises(AssertionError):
        explain_code_differences(bad, sc, a2, q, sc, a)


def test_multi_step_difference_in_the_subnormal_range():
    """A block whose maximum is 448 X and one element a few subnormal steps
    (X 2^-9 each) from zero: moving that element by 3.2 steps changes its code
    by three steps, which is explained; the same code change with a moved by
    only half a step is not."""
    I = 32
    a = np.zeros((1, I), np.float32)
    a[0, 0] = 448.0
    a[0, 5] = 2.0 ** -9 * 1.2                      # code 0x01 after rounding
    q, sc = oracle.quantize_e4m3(a)
    assert sc[0, 0] == 127 and q[0, 5] == 0x01
    a2 = a.copy()
    a2[0, 5] = 2.0 ** -9 * 4.4                     # code 0x04
    q2, sc2 = oracle.quantize_e4m3(a2)
    assert q2[0, 5] == 0x04
    assert explain_code_differences(q2, sc2, a2, q, sc, a) == (1, 0)
    a3 = a.copy()
    a3[0, 5] = 2.0 ** -9 * 1.7                     # would round to 0x02, not 0x04
    with pytest.raises(AssertionError):
        explain_code_differences(q2, sc2, a3, q, sc, a)


def test_planted_scale_error_is_rejected():
    h, q, sc, a = intermediate()
    bad = sc.copy()
    bad[3, 1] += 1
    with pytest.raises(AssertionError):
        explain_code_differences(q, bad, a, q, sc, a)


def test_rel_err_cos():
    ref = np.array([1.0, -2.0, 4.0])
    assert rel_err_cos(ref, ref) == (0.0, 1.0)
    err, cos = rel_err_cos(ref + np.array([0.0, 0.0, 0.004]), ref)
    assert abs(err - 1e-3) < 1e-12 and cos < 1.0
    assert rel_err_cos(np.zeros(3), np.zeros(3)) == (0.0, 1.0)
