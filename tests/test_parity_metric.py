"""Pins of the parity metric itself (oracle.kda_ref.rel_l2), on which every GPU
assertion rests: relL2 = ||x - ref||_2 / ||ref||_2 over the WHOLE tensor,
computed in float64, with the absolute L2 distance when ||ref||_2 < 1e-30 (a
zero reference, e.g. beta = 0 with a zero state). Each case below is worked by
hand and fails a plausible slip: the norm of x in the denominator, a mean of
per-row errors, float32 accumulation, a missing near-zero branch or a
threshold on the wrong side.
"""
import math

import numpy as np

from oracle.kda_ref import rel_l2


def test_identical_tensors_give_zero():
    x = np.arange(12.0).reshape(3, 4)
    assert rel_l2(x, x) == 0.0


def test_denominator_is_the_reference_norm():
    # |2 - 1| / |1| = 1, but |1 - 2| / |2| = 0.5: the metric is not symmetric
    assert rel_l2(np.array([2.0]), np.array([1.0])) == 1.0
    assert rel_l2(np.array([1.0]), np.array([2.0])) == 0.5


def test_pythagorean_worked_example():
    # x - ref = (0.3, -0.4) -> 0.5; |ref| = |(3, 4)| = 5 -> 0.1
    assert math.isclose(rel_l2(np.array([3.3, 3.6]), np.array([3.0, 4.0])), 0.1, rel_tol=1e-12)


def test_whole_tensor_not_mean_of_rows():
    # diff norm 1, ref norm sqrt(2): 1/sqrt(2). A mean of per-row relative errors would give 0.5.
    x = np.array([[1.0, 0.0], [0.0, 0.0]])
    ref = np.array([[1.0, 0.0], [0.0, 1.0]])
    assert math.isclose(rel_l2(x, ref), 1.0 / math.sqrt(2.0), rel_tol=1e-12)


def test_float32_inputs_are_widened_before_squaring():
    # 1e20 squared overflows float32 but not float64: diff 1 over norm ~1e20 = 1e-20
    ref = np.array([1e20, 1.0], dtype=np.float32)
    x = np.array([1e20, 2.0], dtype=np.float32)
    e = rel_l2(x, ref)
    assert np.isfinite(e) and math.isclose(e, 1e-20, rel_tol=1e-6)


def test_zero_reference_uses_absolute_distance():
    # ||ref|| = 0 -> ||x - ref|| = |(3, 4)| = 5
    assert rel_l2(np.array([3.0, 4.0]), np.zeros(2)) == 5.0
    assert rel_l2(np.zeros(3), np.zeros(3)) == 0.0


def test_near_zero_threshold_sides():
    # below 1e-30 the distance is absolute; at and above it, relative
    tiny = np.array([1e-31])
    assert rel_l2(2 * tiny, tiny) == 1e-31
    small = np.array([1e-29])
    assert math.isclose(rel_l2(2 * small, small), 1.0, rel_tol=1e-12)


def test_scale_invariance_above_threshold():
    rng = np.random.default_rng(5)
    ref = rng.standard_normal((4, 5, 6))
    x = ref + 1e-3 * rng.standard_normal(ref.shape)
    e = rel_l2(x, ref)
    for c in (1e-10, 1.0, 1e10):
        assert math.isclose(rel_l2(c * x, c * ref), e, rel_tol=1e-12)
