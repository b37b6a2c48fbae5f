"""Pins for the oracle's codebook (Lloyd-Max on N(0,1) samples, ternary table).

Independent references: hand-worked tiny examples, Max's 1960 table of
Gaussian Lloyd-Max quantizers, and an exact-integral Lloyd-Max solved here on
the continuous Gaussian (no sampling), whose fixed point and mean-square error
the sampled codebook must approach.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import ndtr

from oracle import cq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _phi(x):
    return np.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def gaussian_mse(levels):
    """Exact E[(X - Q(X))^2] for X ~ N(0,1) and nearest-level quantizer Q."""
    c = np.sort(np.asarray(levels, dtype=np.float64))
    t = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    a, b = t[:-1], t[1:]
    pa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
    pb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
    apa = np.where(np.isinf(a), 0.0, np.where(np.isinf(a), 0.0, a) * pa)
    bpb = np.where(np.isinf(b), 0.0, np.where(np.isinf(b), 0.0, b) * pb)
    m0 = ndtr(b) - ndtr(a)            # integral of phi
    m1 = pa - pb                      # integral of x phi
    m2 = m0 - (bpb - apa)             # integral of x^2 phi
    return float(np.sum(m2 - 2 * c * m1 + c * c * m0))


def exact_lloyd(levels, iters=5000):
    """Lloyd-Max on the continuous N(0,1): centroids by exact integrals."""
    c = np.linspace(-2, 2, levels)
    for _ in range(iters):
        t = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        a, b = t[:-1], t[1:]
        pa = np.where(np.isinf(a), 0.0, _phi(np.where(np.isinf(a), 0.0, a)))
        pb = np.where(np.isinf(b), 0.0, _phi(np.where(np.isinf(b), 0.0, b)))
        c = (pa - pb) / (ndtr(b) - ndtr(a))
    return c


# -- hand-worked examples ----------------------------------------------------

def test_lloyd_tiny_hand_example():
    ex = _load("hand_examples.json")["lloyd_tiny"]
    init = O.lloyd_max(ex["samples"], ex["levels"], iters=0)
    np.testing.assert_array_equal(init, ex["init"])
    got = O.lloyd_max(ex["samples"], ex["levels"], iters=10)
    np.testing.assert_allclose(got, ex["result"], rtol=0, atol=1e-15)


def test_lloyd_boundary_tie_goes_to_lower_cell():
    ex = _load("hand_examples.json")["lloyd_tie"]
    got = O.lloyd_max(ex["samples"], ex["levels"], iters=5)
    np.testing.assert_allclose(got, ex["result"], rtol=0, atol=1e-15)


def test_lloyd_returns_sorted_and_runs_requested_iterations():
    x = np.random.RandomState(3).randn(5000)
    one = O.lloyd_max(x, 4, iters=1)
    two = O.lloyd_max(x, 4, iters=2)
    assert np.all(np.diff(one) > 0)
    assert not np.array_equal(one, two)
    # Every level is the mean of its cell after an update (centroid condition).
    c = O.lloyd_max(x, 4, iters=50)
    c_next = O.lloyd_max(x, 4, iters=51)
    np.testing.assert_allclose(c, c_next, atol=1e-6)


# -- ternary table ---------------------------------------------------------------

def test_ternary_levels_as_printed():
    want = _load("pages_constants.json")["ternary_levels"]["value"]
    np.testing.assert_array_equal(O.codebook(O.TERNARY), want)
    assert O.n_levels(O.TERNARY) == 3 and O.storage_bits(O.TERNARY) == 2


def test_ternary_is_the_gaussian_optimum():
    c = exact_lloyd(3)
    np.testing.assert_allclose(O.codebook(O.TERNARY), c, atol=1e-6)


# -- Lloyd-Max on the seeded Gaussian samples -----------------------------------

def test_exact_solver_matches_max_table():
    table = _load("max1960_gaussian.json")["quantizers"]
    for n in (2, 3, 4, 8, 16):
        c = exact_lloyd(n)
        pos = np.sort(c[c >= -1e-12])
        np.testing.assert_allclose(pos, table[str(n)]["levels"], atol=6e-4)
        assert gaussian_mse(c) == pytest.approx(table[str(n)]["mse"], rel=2e-3)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_sampled_codebook_near_gaussian_optimum(bits, oracle_levels):
    levels = oracle_levels[bits]
    n = 1 << bits
    assert levels.shape == (n,) and np.all(np.diff(levels) > 0)
    d_star = gaussian_mse(exact_lloyd(n))
    d = gaussian_mse(levels)
    # Lloyd-Max optimum for a log-concave density is unique: D >= D*.
    assert d_star <= d <= 1.002 * d_star


def test_two_bit_levels_match_textbook(oracle_levels):
    table = _load("max1960_gaussian.json")["quantizers"]["4"]["levels"]
    want = np.array([-table[1], -table[0], table[0], table[1]])
    np.testing.assert_allclose(oracle_levels[2], want, atol=5e-3)


def test_seed0_levels_regression(oracle_levels):
    # Seed-0 Lloyd-Max levels computed separately, before this oracle was
    # written (an independent script); six printed decimals.
    want = {
        1: [-0.792722, 0.800951],
        2: [-1.506671, -0.451441, 0.452947, 1.509933],
        3: [-2.141248, -1.333716, -0.748398, -0.237740, 0.250045, 0.755587, 1.337983, 2.147636],
    }
    for bits, w in want.items():
        np.testing.assert_allclose(oracle_levels[bits], w, atol=1.5e-6)


def test_runtime_levels_and_thresholds(oracle_levels):
    c32 = O.runtime_levels(oracle_levels[2])
    assert np.all(c32 == c32.astype(np.float32).astype(np.float64))
    t = O.thresholds(c32)
    assert np.all((c32[:-1] < t) & (t < c32[1:]))
    # Midpoints of float32 values are exact in float64.
    assert np.all(2 * t == c32[:-1] + c32[1:])


def test_bad_widths_rejected():
    for bits in (0, 5, 8):
        with pytest.raises(ValueError):
            O.n_levels(bits)
