"""The comparator every GPU parity verdict goes through (oracle.scaled_error),
checked with negative controls on the CPU: a result off by twice the
tolerance of its scale must fail, a NaN where the reference has a number (or
the reverse) must give an infinite error, a zero scale with a nonzero
difference must fail, and arrays of different shapes must be refused rather
than broadcast."""
import numpy as np
import pytest

import oracle

TOLS = (1e-4, 2e-2)


def _case(seed=0, n=(3, 5, 7)):
    rng = np.random.default_rng(seed)
    ref = rng.standard_normal(n)
    scale = np.abs(ref) + rng.uniform(0.5, 2.0, n)  # scale >= |ref|, as the oracle's sums are
    return ref, scale


def test_exact_result_has_zero_error():
    ref, scale = _case()
    assert oracle.scaled_error(ref.copy(), ref, scale) == 0.0


@pytest.mark.parametrize("tol", TOLS)
def test_perturbation_at_twice_the_tolerance_fails(tol):
    ref, scale = _case(1)
    got = ref.copy()
    idx = (1, 2, 3)
    got[idx] += 2.0 * tol * scale[idx]  # one element, twice the allowed error
    err = oracle.scaled_error(got, ref, scale)
    assert err == pytest.approx(2.0 * tol, rel=1e-9)
    assert err > tol


@pytest.mark.parametrize("tol", TOLS)
def test_perturbation_at_half_the_tolerance_passes(tol):
    ref, scale = _case(2)
    got = ref + 0.5 * tol * scale * np.sign(np.random.default_rng(3).standard_normal(ref.shape))
    err = oracle.scaled_error(got, ref, scale)
    assert err == pytest.approx(0.5 * tol, rel=1e-9)
    assert err <= tol


def test_error_is_the_maximum_not_a_mean():
    ref, scale = _case(4, n=(1000,))
    got = ref.copy()
    got[637] += 3e-3 * scale[637]
    assert oracle.scaled_error(got, ref, scale) == pytest.approx(3e-3, rel=1e-9)


def test_nan_mismatch_is_infinite():
    ref, scale = _case(5)
    got = ref.copy()
    got[0, 0, 0] = np.nan
    assert oracle.scaled_error(got, ref, scale) == float("inf")
    ref2 = ref.copy()
    ref2[2, 4, 6] = np.nan
    assert oracle.scaled_error(ref.copy(), ref2, scale) == float("inf")
    # NaN in both places: excluded, the rest compared
    got2 = ref2.copy()
    assert oracle.scaled_error(got2, ref2, scale) == 0.0


def test_infinity_must_match_exactly():
    ref, scale = _case(6)
    ref[1, 1, 1] = np.inf
    got = ref.copy()
    assert oracle.scaled_error(got, ref, scale) == 0.0
    got[1, 1, 1] = -np.inf
    assert oracle.scaled_error(got, ref, scale) == float("inf")
    got[1, 1, 1] = 1e30
    assert oracle.scaled_error(got, ref, scale) == float("inf")


def test_zero_scale_with_a_difference_fails():
    ref, scale = _case(7)
    scale[0, 1, 2] = 0.0
    ref[0, 1, 2] = 0.0
    got = ref.copy()
    assert oracle.scaled_error(got, ref, scale) == 0.0  # zero difference: fine
    got[0, 1, 2] = 1e-20
    assert oracle.scaled_error(got, ref, scale) > 1.0


def test_shape_mismatch_is_refused():
    ref, scale = _case(8)
    with pytest.raises(ValueError):
        oracle.scaled_error(ref[:1], ref, scale)  # would broadcast
    with pytest.raises(ValueError):
        oracle.scaled_error(ref, ref, scale[0])
    with pytest.raises(ValueError):
        oracle.scaled_error(ref.reshape(-1), ref, scale)


def test_bfloat16_rounding_of_the_reference_stays_within_the_bf16_limit():
    """A result that is the reference rounded to bfloat16 (what a correct
    kernel's RNE store does) passes the bf16 limit and fails the fp32 one, so
    the two limits really separate the precisions."""
    import torch
    ref, _ = _case(9, n=(4096,))
    scale = np.abs(ref)  # the tightest possible scale: each output a single term
    got = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    err = oracle.scaled_error(got, ref, scale)
    assert 1e-4 < err <= 2 ** -8 < 2e-2  # unit roundoff of an 8-bit significand
