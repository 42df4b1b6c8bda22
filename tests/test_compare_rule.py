"""The comparison rule of the parity tests (tests/helpers.py) on the CPU:
what it accepts and what it rejects, including the term-magnitude scale
that the pile-up tests use for sums of thousands of cancelling terms."""
import numpy as np
import pytest

from helpers import compare


def test_rule_accepts_within_and_rejects_beyond_rtol():
    want = np.array([1.0, -2.0, 0.0, 4.0])
    rms = np.sqrt(np.mean(want * want))
    ok = want + 0.9e-5 * (np.abs(want) + rms)
    compare("within", ok, want, 1e-5)
    bad = ok.copy()
    bad[2] = want[2] + 1.1e-5 * rms
    with pytest.raises(AssertionError):
        compare("beyond", bad, want, 1e-5)


def _pile_up(n, seed):
    """n float32 terms with random signs, as many samples' A * w * G land on
    one pixel; returns the terms, their float32 running sum and the exact sum."""
    rng = np.random.default_rng(seed)
    terms = (rng.uniform(0.0, 0.2, n) * rng.standard_normal(n)).astype(np.float32)
    acc = np.float32(0.0)
    for t in terms:
        acc = np.float32(acc + t)
    return terms, acc, float(np.sum(terms.astype(np.float64)))


def test_magnitude_scale_admits_float32_summation_of_a_pile_up():
    # one piled-up element among many small ones: rms stays small, the element
    # cancels, so its float32 rounding error can pass rtol * (|o| + rms)
    terms, acc, exact = _pile_up(6000, 3)
    want = np.full(1000, 1e-3)
    want[0] = exact
    got = want.copy()
    got[0] = acc
    mag = np.zeros_like(want)
    mag[0] = float(np.sum(np.abs(terms.astype(np.float64))))
    compare("pile-up", got, want, 1e-5, magnitude=mag)


def test_magnitude_scale_still_catches_one_missing_term():
    terms, acc, exact = _pile_up(6000, 5)
    want = np.full(1000, 1e-3)
    want[0] = exact
    mag = np.zeros_like(want)
    mag[0] = float(np.sum(np.abs(terms.astype(np.float64))))
    # the gpu side dropped its largest term: fewer than 1 / rtol terms, so
    # that term exceeds rtol times their total magnitude
    k = int(np.argmax(np.abs(terms)))
    got = want.copy()
    got[0] = exact - float(terms[k])
    with pytest.raises(AssertionError):
        compare("pile-up, one term missing", got, want, 1e-5, magnitude=mag)
    # and any term of at least the mean magnitude
    k = int(np.argmin(np.abs(np.abs(terms) - np.mean(np.abs(terms)))))
    got[0] = exact - float(terms[k])
    with pytest.raises(AssertionError):
        compare("pile-up, a mean term missing", got, want, 1e-5, magnitude=mag)
