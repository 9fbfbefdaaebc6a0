"""Pins of the two error measures every GPU parity test and the smoke run rely on (CPU only).

Each case is worked out by hand, so a slip in either measure (a wrong norm, the wrong operand in the denominator,
an RMS over the wrong axis, the own-size allowance applied too widely or not at all) fails here rather than
silently loosening every GPU check.
"""
import math

import numpy as np
import pytest

import oracle as O
from parity_utils import BF16_MAX_ABS_UNIT, KAPPA, check_close, max_err_unit_scale


def test_rel_frobenius_hand_cases():
    # ||(0, 0, 0, 0.5)|| / ||(1, 0, 0, 0)|| = 0.5
    assert O.rel_frobenius(np.array([1.0, 0, 0, 0.5]), np.array([1.0, 0, 0, 0])) == 0.5
    # the reference's norm is the denominator (3-4-5): ||(3, 4)|| = 5, got = 0 -> 1
    assert O.rel_frobenius(np.zeros(2), np.array([3.0, 4.0])) == 1.0
    # not the got's norm: got = (6, 8) against (3, 4) -> ||(3, 4)|| / 5 = 1, where /||got|| would give 0.5
    assert O.rel_frobenius(np.array([6.0, 8.0]), np.array([3.0, 4.0])) == 1.0
    # a matrix is taken as one vector (Frobenius, not the spectral norm): ref [[1, 2], [2, 4]] has norm 5, the
    # difference [[0, 0], [0, 3]] norm 3 -> 0.6 (the spectral norm of ref is also 5, of the difference 3; a
    # row-wise max would give 3/4.47)
    assert abs(O.rel_frobenius(np.array([[1.0, 2], [2, 1]]), np.array([[1.0, 2], [2, 4]])) - 0.6) < 1e-15
    # the sum of squares is not replaced by the sum of magnitudes: ref (1, 1, 1, 1) norm 2, error (1, 1, 0, 0)
    # norm sqrt 2 -> 0.7071 (an L1 ratio would give 0.5)
    assert abs(O.rel_frobenius(np.array([2.0, 2, 1, 1]), np.ones(4)) - math.sqrt(2) / 2) < 1e-15
    # a zero reference leaves the absolute norm
    assert O.rel_frobenius(np.array([0.0, 0.25]), np.zeros(2)) == 0.25


def test_kappa_is_two_ulps_over_the_bound():
    assert KAPPA * BF16_MAX_ABS_UNIT == 2.0 ** -7


def test_max_err_unit_scale_tensor_rms():
    ref = np.array([[1.0, -1.0], [1.0, -1.0]])  # RMS 1
    got = ref.copy()
    got[1, 0] += 0.03
    assert abs(max_err_unit_scale(got, ref) - 0.03) < 1e-15
    # the unit is the RMS, not the mean magnitude of the error or of got: scaling ref by 10 scales the unit by 10
    assert abs(max_err_unit_scale(10 * got, 10 * ref) - 0.03) < 1e-15
    # ref (10, 0, 0, 0): RMS 5; element 0 has KAPPA * 10 = 2.60 < 5, so its unit is the RMS: error 0.15 -> 0.03
    ref = np.array([10.0, 0, 0, 0])
    got = ref + np.array([0.15, 0, 0, 0])
    assert abs(max_err_unit_scale(got, ref) - 0.03) < 1e-15
    # an error on a zero element is measured against the RMS too
    got = ref + np.array([0, 0, 0.15, 0])
    assert abs(max_err_unit_scale(got, ref) - 0.03) < 1e-15


def test_max_err_unit_scale_own_size_allowance():
    # one element of 100 among 9999 zeros: RMS = 100 / 100 = 1; the element's allowance is max(3e-2 * 1, 2^-7 * 100)
    ref = np.zeros(10000)
    ref[0] = 100.0
    got = ref.copy()
    got[0] += 2.0 ** -7 * 100  # exactly at the allowance
    assert abs(max_err_unit_scale(got, ref) - BF16_MAX_ABS_UNIT) < 1e-12
    got[0] = 100.0 + 2.0 ** -6 * 100  # twice the allowance: fails the 3e-2 bound
    assert max_err_unit_scale(got, ref) > 1.99 * BF16_MAX_ABS_UNIT
    # under the old unit max(RMS, |ref|) that error would have scored 0.015 and passed: the allowance is tighter
    assert 2.0 ** -6 < BF16_MAX_ABS_UNIT
    # an element between the RMS and 3.84 RMS gets no own-size allowance: ref 3 (RMS 1 with the rest), error 0.06
    ref = np.zeros(9)
    ref[0] = 3.0  # RMS = 3 / 3 = 1
    got = ref.copy()
    got[0] += 0.06
    assert abs(max_err_unit_scale(got, ref) - 0.06) < 1e-12
    with pytest.raises(AssertionError):
        check_close(got, ref, "bf16")


def test_max_err_unit_scale_row_unit():
    # rows with RMS 1 and 10: per-row units make errors of 0.03 and 0.3 both 0.03
    ref = np.array([[1.0, 1.0], [10.0, 10.0]])
    got = ref + np.array([[0.03, 0.0], [0.0, 0.3]])
    assert abs(max_err_unit_scale(got, ref, row_unit=True) - 0.03) < 1e-15
    # with one unit for the tensor (RMS sqrt(50.5) = 7.11) the 0.3 error scores 0.042 and the 0.03 one 0.0042
    assert abs(max_err_unit_scale(got, ref) - 0.3 / math.sqrt(50.5)) < 1e-15


def test_check_close_bounds():
    ref = np.linspace(-1.0, 1.0, 101)
    check_close(ref * (1 + 5e-6), ref, "f32")
    with pytest.raises(AssertionError):
        check_close(ref * (1 + 2e-5), ref, "f32")
    with pytest.raises(AssertionError):
        check_close(np.where(ref > 0.99, np.nan, ref), ref, "bf16")
    rms = math.sqrt(np.mean(ref * ref))
    got = ref.copy()
    got[50] += 0.029 * rms
    check_close(got, ref, "bf16")
    got[50] += 0.002 * rms
    with pytest.raises(AssertionError):
        check_close(got, ref, "bf16")
