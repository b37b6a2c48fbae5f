"""Pins for the oracle's tolerance helpers and for the index rule built on them.

The codebook here is (-1.5, -0.5, 0.5, 1.5): exact in float32, with decision
thresholds at exactly -1, 0 and 1 (midpoints of neighbouring levels, "How
Quantization Codebooks Are Trained in Cactus Quants", section Iterative
Refinement of Quantization Levels).  Every expected value below is worked by
hand from those three numbers.
"""

import numpy as np
import pytest

from oracle import cq_oracle as O
from parity import BAND, check_indices

LEVELS = np.array([-1.5, -0.5, 0.5, 1.5])

# (z, distance to the nearest threshold).  A distance taken to the levels
# instead of the thresholds would give 0.2, 0.5, 0.0, 1.0, 1.5, 0.25 here.
DISTANCES = [
    (0.3, 0.3),     # nearest threshold 0
    (-1.0, 0.0),    # exactly on a threshold
    (0.5, 0.5),     # midway between thresholds 0 and 1
    (-2.5, 1.5),    # below every threshold
    (3.0, 2.0),     # above every threshold
    (-0.75, 0.25),  # between -1 and 0, nearer -1
]


def test_threshold_distance_hand_worked():
    z = np.array([a for a, _ in DISTANCES])
    want = np.array([d for _, d in DISTANCES])
    np.testing.assert_array_equal(O.threshold_distance(z, LEVELS), want)


def test_threshold_distance_keeps_the_shape():
    """The minimum runs over the thresholds, element by element: a (2, 3)
    array of z gives a (2, 3) array of distances in the same places."""
    z = np.array([[a for a, _ in DISTANCES[:3]], [a for a, _ in DISTANCES[3:]]])
    want = np.array([[d for _, d in DISTANCES[:3]], [d for _, d in DISTANCES[3:]]])
    got = O.threshold_distance(z, LEVELS)
    assert got.shape == (2, 3)
    np.testing.assert_array_equal(got, want)


# (z, (lo, hi)) for band 0.25: the index of z - 0.25 and of z + 0.25, where
# the index is the count of thresholds strictly below the value.
ADMISSIBLE = [
    (0.3, (2, 2)),    # 0.05 .. 0.55 lies inside one cell
    (0.1, (1, 2)),    # -0.15 .. 0.35 straddles 0
    (-0.1, (1, 2)),   # -0.35 .. 0.15 straddles 0
    (1.0, (2, 3)),    # exactly on the threshold 1 (its own index is 2)
    (0.25, (1, 2)),   # z - band lands exactly on 0, which belongs to the lower cell
    (-3.0, (0, 0)),
    (3.0, (3, 3)),
    (-0.5, (1, 1)),   # a level: the middle of its cell
]


def test_admissible_indices_hand_worked():
    z = np.array([a for a, _ in ADMISSIBLE])
    lo, hi = O.admissible_indices(z, LEVELS, 0.25)
    np.testing.assert_array_equal(lo, [r[0] for _, r in ADMISSIBLE])
    np.testing.assert_array_equal(hi, [r[1] for _, r in ADMISSIBLE])
    # The oracle's own index always lies in the range.
    own = np.searchsorted(O.thresholds(LEVELS), z, side="left")
    assert np.all((lo <= own) & (own <= hi))


def test_admissible_indices_zero_band_is_the_index():
    z = np.linspace(-2.0, 2.0, 41)
    lo, hi = O.admissible_indices(z, LEVELS, 0.0)
    own = np.searchsorted(O.thresholds(LEVELS), z, side="left")
    np.testing.assert_array_equal(lo, own)
    np.testing.assert_array_equal(hi, own)


def _fake_q(z, idx_ref):
    """A Quantized record with chosen z and reference indices (one group)."""
    z = np.asarray(z, dtype=np.float64).reshape(1, 1, -1)
    idx = np.asarray(idx_ref, dtype=np.int64).reshape(1, 1, -1)
    n = np.ones((1, 1))
    return O.Quantized(idx, z, n, O.fp16_bits(n), 1, z.size, 2, z.size, O.runtime_levels(LEVELS))


@pytest.mark.parametrize("side", [-1, 1])
def test_index_rule_admits_only_the_far_side_of_the_near_threshold(side):
    """z just below the threshold 0 (oracle index 1): the GPU may return 2
    (the value crossed the threshold), never 0; just above (oracle index 2):
    1 is admissible, 3 is not."""
    eps = 0.5 * BAND
    if side < 0:
        z, ref, ok, bad = -eps, 1, 2, 0
    else:
        z, ref, ok, bad = eps, 2, 1, 3
    q = _fake_q([z, 1.2], [ref, 3])
    rep = check_indices(np.array([ok, 3]), q, enforce_count=False)
    assert rep["index_mismatches"] == 1
    with pytest.raises(AssertionError):
        check_indices(np.array([bad, 3]), q, enforce_count=False)


def test_index_rule_rejects_mismatch_outside_the_band():
    q = _fake_q([-3 * BAND, 0.7], [1, 2])
    with pytest.raises(AssertionError):
        check_indices(np.array([2, 2]), q, enforce_count=False)
    assert check_indices(np.array([1, 2]), q, enforce_count=False)["index_mismatches"] == 0
