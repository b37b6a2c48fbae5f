"""Pins for the oracle's quantize / dequantize / matvec / byte accounting."""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import cq_oracle as O
from rotated_codebook_bit_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BITS = [O.TERNARY, 1, 2, 3, 4]


def _hand():
    return json.load(open(os.path.join(GOLDEN, "hand_examples.json")))


# -- nearest level ---------------------------------------------------------------

@pytest.mark.parametrize("bits", BITS)
def test_index_is_brute_force_nearest(bits, oracle_levels):
    w = np.random.RandomState(5).randn(64, 256)
    q = O.quantize(w, bits, oracle_levels[bits])
    c = O.runtime_levels(oracle_levels[bits])
    d = np.abs(q.z[..., None] - c)                 # distance to every level
    best = np.argmin(d, axis=-1)                   # first minimum = lower index on ties
    np.testing.assert_array_equal(q.idx, best)


@pytest.mark.parametrize("g", [2, 4, 8])
def test_tiny_groups_exhaustive_optimum(g, oracle_levels):
    """For a fixed norm, the chosen code minimises the reconstruction error
    over all L^g codes (the rotation is orthonormal, so the error separates)."""
    levels = oracle_levels[2]
    c = O.runtime_levels(levels)
    h = O.hadamard(g)
    codes = np.array(list(itertools.product(range(4), repeat=g)))
    rs = np.random.RandomState(g)
    for _ in range(5):
        x = rs.randn(1, g)
        q = O.quantize(x, 2, levels, g=g)
        n = q.norm[0, 0]
        recon = (c[codes] * (n / math.sqrt(g))) @ h  # every candidate, unrounded norm
        err = np.sum((recon - x) ** 2, axis=1)
        best = codes[np.argmin(err)]
        np.testing.assert_array_equal(q.idx[0, 0], best)


# -- invariants ------------------------------------------------------------------

@pytest.mark.parametrize("bits", [O.TERNARY, 2, 4])
def test_power_of_two_scale_invariance(bits, oracle_levels):
    w = np.random.RandomState(7).randn(16, 384)
    a = O.quantize(w, bits, oracle_levels[bits])
    b = O.quantize(w * 8.0, bits, oracle_levels[bits])
    np.testing.assert_array_equal(a.idx, b.idx)
    np.testing.assert_array_equal(b.norm, a.norm * 8.0)


def test_group_permutation_equivariance(oracle_levels):
    w = np.random.RandomState(8).randn(1, 128 * 6)
    perm = [3, 0, 5, 1, 4, 2]
    wp = w.reshape(6, 128)[perm].reshape(1, -1)
    a = O.quantize(w, 2, oracle_levels[2])
    b = O.quantize(wp, 2, oracle_levels[2])
    np.testing.assert_array_equal(b.idx[0], a.idx[0][perm])
    np.testing.assert_array_equal(b.norm16[0], a.norm16[0][perm])


def test_fixed_point(oracle_levels):
    """x = H c[idx] with every z interior to its cell quantizes to idx and
    reconstructs to x up to the binary16 rounding of the norm."""
    levels = oracle_levels[2]
    c = O.runtime_levels(levels)
    rs = np.random.RandomState(9)
    idx = rs.randint(0, 4, size=128)
    v = c[idx]
    v = v * (math.sqrt(128) / np.linalg.norm(v))      # make ||v||^2 = G so z = v
    # Rescaling moves v off the exact levels; rebuild from the scaled vector.
    x = v @ O.hadamard(128)
    q = O.quantize(x[None, :], 2, levels)
    t = O.thresholds(c)
    assert np.min(np.abs(v[:, None] - t)) > 1e-3
    want = np.searchsorted(t, v, side="left")
    np.testing.assert_array_equal(q.idx[0, 0], want)
    np.testing.assert_allclose(q.z[0, 0], v, atol=1e-13)


def test_padding_equals_explicit_zero_pad(oracle_levels):
    w = np.random.RandomState(10).randn(30, 1000) * 0.02
    wp = np.zeros((30, 1024))
    wp[:, :1000] = w
    a = O.quantize(w, 2, oracle_levels[2])
    b = O.quantize(wp, 2, oracle_levels[2])
    np.testing.assert_array_equal(a.packed, b.packed)
    np.testing.assert_array_equal(a.norm16, b.norm16)
    da = O.dequantize(a.packed, a.norm16, 30, 1000, 2, oracle_levels[2])
    db = O.dequantize(b.packed, b.norm16, 30, 1024, 2, oracle_levels[2])
    assert da.shape == (30, 1000)
    np.testing.assert_array_equal(da, db[:, :1000])


@pytest.mark.parametrize("bits", [O.TERNARY, 2, 3, 4])
def test_constant_group_closed_form(bits, oracle_levels):
    """A constant group a*1 rotates to a*sqrt(G)*e_0: index L-1 at j=0, the
    level containing 0 elsewhere; the reconstruction is (n16/G) *
    (c_top + c_m * (G*delta_i0 - 1)) by the column sums of the +-1 matrix."""
    levels = oracle_levels[bits]
    c = O.runtime_levels(levels)
    a = 0.25
    q = O.quantize(np.full((1, 128), a), bits, levels)
    m = int(np.sum(O.thresholds(c) < 0))
    want = np.full(128, m)
    want[0] = c.size - 1
    np.testing.assert_array_equal(q.idx[0, 0], want)
    n16 = float(np.float16(a * math.sqrt(128)))
    xh = O.dequantize(q.packed, q.norm16, 1, 128, bits, levels)[0]
    expect = np.full(128, (n16 / 128) * (c[-1] - c[m]))
    expect[0] = (n16 / 128) * (c[-1] + 127 * c[m])
    np.testing.assert_allclose(xh, expect, rtol=1e-14, atol=1e-16)


def test_zero_group(oracle_levels):
    levels = oracle_levels[2]
    q = O.quantize(np.zeros((2, 256)), 2, levels)
    m = int(np.sum(O.thresholds(O.runtime_levels(levels)) < 0))
    assert np.all(q.idx == m) and np.all(q.norm16 == 0)
    assert not O.dequantize(q.packed, q.norm16, 2, 256, 2, levels).any()


def test_exact_cancellation_takes_the_tie_rule():
    """A group whose +-1 transform cancels exactly at some positions: with a
    codebook symmetric about 0 (Max's 4-level table), those components sit
    exactly on the middle threshold 0, so z must be exactly 0 there and the
    index the lower level's (the tie rule), whatever the rounding of
    1/sqrt(G).  The integer group [5, 5, 1, 9, 0, ...] cancels at 32 of its
    128 positions (5 + 5 - 1 - 9 = 0 and sign patterns with the same sum)."""
    table = json.load(open(os.path.join(GOLDEN, "max1960_gaussian.json")))
    pos = table["quantizers"]["4"]["levels"]
    levels = np.array([-pos[1], -pos[0], pos[0], pos[1]])
    x = np.zeros((1, 128))
    x[0, :4] = [5, 5, 1, 9]
    hx = x[0] @ O.sylvester(128)  # small integers: exact
    zero = hx == 0
    assert zero.sum() == 32
    q = O.quantize(x, 2, levels)
    assert np.all(q.z[0, 0][zero] == 0.0)
    np.testing.assert_array_equal(q.idx[0, 0][zero], 1)
    # Away from the zeros every component is an integer multiple of
    # 1/sqrt(128) of size >= 2, far from all thresholds: the plain rule.
    t = O.thresholds(O.runtime_levels(levels))
    np.testing.assert_array_equal(q.idx[0, 0][~zero], np.searchsorted(t, q.z[0, 0][~zero], side="left"))


def test_leading_dims_flatten(oracle_levels):
    w = np.random.RandomState(11).randn(3, 4, 256)
    a = O.quantize(w, 2, oracle_levels[2])
    b = O.quantize(w.reshape(12, 256), 2, oracle_levels[2])
    np.testing.assert_array_equal(a.packed, b.packed)
    assert (a.rows, a.cols) == (12, 256)


# -- dequantize ------------------------------------------------------------------

def test_dequantize_matches_explicit_formula(oracle_levels):
    levels = oracle_levels[3]
    c = O.runtime_levels(levels)
    rs = np.random.RandomState(12)
    idx = rs.randint(0, 8, size=(4, 2, 128))
    n16 = O.fp16_bits(rs.rand(4, 2) * 3)
    packed = O.pack(idx, 3)
    xh = O.dequantize(packed, n16, 4, 256, 3, levels)
    h = O.sylvester(128)
    n = n16.view(np.float16).astype(np.float64)
    for r in range(4):
        for g in range(2):
            manual = (n[r, g] / 128.0) * (h @ c[idx[r, g]])
            np.testing.assert_allclose(xh[r, g * 128:(g + 1) * 128], manual, rtol=1e-13, atol=1e-16)


@pytest.mark.parametrize("bits,expect", [(2, 0.1175), (4, 0.009497)])
def test_distortion_tracks_codebook_mse(bits, expect, oracle_levels):
    """Gaussian input: the relative MSE is close to the codebook's Gaussian
    MSE (D* from Max's table); the pages' ~0.30 / ~0.09 sit near the RMS
    form sqrt(MSE), reported, not gated."""
    w = np.random.RandomState(0).randn(2048, 128)
    e2 = O.relative_mse(w, O.fake_quant(w, bits, oracle_levels[bits]))
    assert e2 == pytest.approx(expect, rel=0.03)


def test_rotation_helps_outliers(oracle_levels):
    bits = W.sweep_bits(n=512)
    w = W.bf16_bits_to_f32(bits).astype(np.float64)
    rot = O.relative_mse(w, O.fake_quant(w, 2, oracle_levels[2]))
    plain = O.relative_mse(w, O.fake_quant(w, 2, oracle_levels[2], rotate=False))
    assert rot < 0.5 * plain


# -- matvec ----------------------------------------------------------------------

def test_matvec_two_routes_agree(oracle_levels):
    levels = oracle_levels[2]
    w = np.random.RandomState(13).randn(40, 512) * 0.02
    q = O.quantize(w, 2, levels)
    x = np.random.RandomState(14).randn(3, 512)
    a = O.matvec(q.packed, q.norm16, 40, 512, 2, levels, x)
    b = O.matvec_rotated(q.packed, q.norm16, 40, 512, 2, levels, x)
    assert a.shape == (3, 40)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12 * np.abs(a).max())


def test_matvec_brute_force_small(oracle_levels):
    levels = oracle_levels[2]
    c = O.runtime_levels(levels)
    w = np.random.RandomState(15).randn(3, 128)
    q = O.quantize(w, 2, levels)
    x = np.random.RandomState(16).randn(1, 128)
    h = O.sylvester(128)
    y = O.matvec(q.packed, q.norm16, 3, 128, 2, levels, x)
    for r in range(3):
        n = float(q.norm16[r, 0].view(np.float16))
        row = (n / 128.0) * (h @ c[q.idx[r, 0]])
        assert y[0, r] == pytest.approx(float(np.dot(x[0], row)), rel=1e-12)


# -- bytes -----------------------------------------------------------------------

def test_model_bytes_hand_cases():
    for case in _hand()["model_bytes"]["cases"]:
        assert O.model_bytes(case["shapes"], case["bits"]) == case["bytes"]


def test_model_bytes_needle2_set():
    want = _hand()["needle2_model_bytes"]
    shapes = [s for _, s in W.needle2_shapes()]
    assert O.model_bytes(shapes, 2) == want["bits_2"]
    assert O.model_bytes(shapes, 3) == want["bits_3"]
    assert O.model_bytes(shapes, 4) == want["bits_4"]
    assert 2 * sum(r * c for r, c in shapes[:-1]) == want["fp16_without_pad_tensor"]
    assert O.model_bytes(shapes, O.TERNARY) == want["bits_2"]


def test_model_bytes_matches_packed_sizes(oracle_levels):
    w = np.random.RandomState(17).randn(5, 300)
    for bits in BITS:
        q = O.quantize(w, bits, oracle_levels[bits])
        assert q.packed.nbytes + q.norm16.nbytes == O.model_bytes([w.shape], bits)


# -- fake quant (quantize then reconstruct with the unrounded norm) ----------------

@pytest.mark.parametrize("bits", [O.TERNARY, 2, 3, 4])
def test_fake_quant_equals_stored_round_trip_when_norm_is_fp16_exact(bits, oracle_levels):
    """Groups whose norm is exactly representable in binary16 reconstruct the
    same with the stored and the unrounded norm: 64 entries of +-2 and 64
    zeros have norm exactly 16."""
    levels = oracle_levels[bits]
    rs = np.random.RandomState(21)
    w = np.zeros((6, 128))
    for r in range(6):
        pos = rs.permutation(128)[:64]
        w[r, pos] = rs.choice([-2.0, 2.0], size=64)
    q = O.quantize(w, bits, levels)
    assert np.all(q.norm == 16.0)
    rt = O.dequantize(q.packed, q.norm16, 6, 128, bits, levels)
    # Same formula; only the float64 summation order of the two products differs.
    np.testing.assert_allclose(O.fake_quant(w, bits, levels), rt, rtol=1e-13, atol=1e-15)


def test_fake_quant_constant_group_closed_form(oracle_levels):
    levels = oracle_levels[2]
    c = O.runtime_levels(levels)
    a = 0.3
    n = a * math.sqrt(128)
    m = int(np.sum(O.thresholds(c) < 0))
    xh = O.fake_quant(np.full((1, 128), a), 2, levels)[0]
    expect = np.full(128, (n / 128) * (c[-1] - c[m]))
    expect[0] = (n / 128) * (c[-1] + 127 * c[m])
    np.testing.assert_allclose(xh, expect, rtol=1e-13)


def test_fake_quant_shape_and_padding(oracle_levels):
    w = np.random.RandomState(22).randn(2, 3, 200)
    out = O.fake_quant(w, 2, oracle_levels[2])
    assert out.shape == w.shape
    wp = np.zeros((2, 3, 256))
    wp[..., :200] = w
    np.testing.assert_array_equal(out, O.fake_quant(wp, 2, oracle_levels[2])[..., :200])
