"""Pins for the oracle's Hadamard rotation, packing and fp16 rounding."""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import cq_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def fwht(x):
    """In-place iterative fast Walsh-Hadamard transform (unnormalised)."""
    x = np.array(x, dtype=np.float64)
    n = x.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x


@pytest.mark.parametrize("g", [1, 2, 4, 8, 128])
def test_hadamard_orthonormal_symmetric(g):
    h = O.hadamard(g)
    np.testing.assert_allclose(h @ h.T, np.eye(g), atol=1e-15)
    np.testing.assert_array_equal(h, h.T)
    np.testing.assert_allclose(np.abs(h), 1 / math.sqrt(g), rtol=0, atol=0)


def test_sylvester_closed_form():
    g = 128
    i = np.arange(g)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    np.testing.assert_array_equal(O.sylvester(g), np.where(pc % 2 == 0, 1.0, -1.0))


def test_fwht_matches_dense_rotation():
    x = np.random.RandomState(1).randn(7, 128)
    np.testing.assert_allclose(fwht(x) / math.sqrt(128), x @ O.hadamard(128), atol=1e-14)


def test_rotation_preserves_norm():
    x = np.random.RandomState(2).randn(50, 128) * 3
    y = x @ O.hadamard(128)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)


@pytest.mark.parametrize("g", [32, 128, 256])
def test_normalised_groups(g):
    """n is the group's L2 norm (the rotation preserves it), z the rotated
    group (by the independent in-lane transform above) scaled to norm
    sqrt(g); a zero group gives n = 0 and z = 0; bf16-representable inputs
    give exactly the integer-scaled sums the butterfly gives."""
    x = np.random.RandomState(g).randn(40, g) * 0.02
    x[3] = 0.0
    n, z = O.normalised_groups(x, g)
    np.testing.assert_allclose(n, np.linalg.norm(x, axis=1), rtol=1e-14)
    live = n > 0
    np.testing.assert_allclose(z[live], (fwht(x)[live] / math.sqrt(g)) * math.sqrt(g) / n[live, None],
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(np.linalg.norm(z[live], axis=1), math.sqrt(g), rtol=1e-14)
    assert n[3] == 0 and not z[3].any()
    # Small integers: the +-1 sums are exact, so z * n equals fwht exactly.
    xi = np.random.RandomState(7).randint(-20, 21, size=(5, g)).astype(np.float64)
    ni, zi = O.normalised_groups(xi, g)
    exact = fwht(xi)
    np.testing.assert_array_equal(zi == 0, exact == 0)
    np.testing.assert_allclose(zi * ni[:, None], exact, rtol=1e-15)


def test_non_power_of_two_rejected():
    with pytest.raises(ValueError):
        O.sylvester(96)


# -- packing ---------------------------------------------------------------------

def test_pack_hand_examples():
    for case in json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["pack"]:
        sb = case["sbits"]
        idx = np.zeros(128, dtype=np.int64)
        idx[:len(case["idx_prefix"])] = case["idx_prefix"]
        p = O.pack(idx, sb)
        assert p.shape == (128 * sb // 8,)
        assert list(p[:len(case["bytes_prefix"])]) == case["bytes_prefix"]
        assert not p[len(case["bytes_prefix"]):].any()


@pytest.mark.parametrize("sb", [2, 3, 4])
def test_pack_unpack_roundtrip(sb):
    idx = np.random.RandomState(sb).randint(0, 1 << sb, size=(3, 5, 128))
    p = O.pack(idx, sb)
    assert p.shape == (3, 5, 16 * sb)
    np.testing.assert_array_equal(O.unpack(p, sb), idx)


def test_pack_bit_positions_one_hot():
    # Element j with value 1 sets exactly stream bit sbits*j.
    for sb in (2, 3, 4):
        for j in (0, 1, 7, 63, 127):
            idx = np.zeros(128, dtype=np.int64)
            idx[j] = 1
            bits = np.unpackbits(O.pack(idx, sb), bitorder="little")
            assert list(np.flatnonzero(bits)) == [sb * j]


# -- fp16 rounding -----------------------------------------------------------------

def test_fp16_hand_cases():
    cases = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))["fp16_rounding"]["cases"]
    values = [1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 1 + 2.0 ** -11 + 2.0 ** -40, 65504.0, 65520.0]
    for v, case in zip(values, cases):
        assert int(O.fp16_bits(np.array([v]))[0]) == case["bits"], case["x"]
