import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libcq")


@pytest.fixture(scope="session")
def lloyd_samples():
    from rotated_codebook_bit_amd.workloads import lloyd_samples as draw
    return draw()


@pytest.fixture(scope="session")
def oracle_levels(lloyd_samples):
    """Oracle codebooks (N(0,1) units, float64) for every supported width."""
    from oracle import cq_oracle as O
    return {b: O.codebook(b, lloyd_samples) for b in (1, 2, 3, 4, O.TERNARY)}


@pytest.fixture(scope="session")
def levels32(oracle_levels):
    """The oracle's codebooks as the float32 tables every parity run hands to
    both sides (GPU and oracle get bit-identical levels)."""
    from oracle import cq_oracle as O
    return {b: O.runtime_levels(v).astype(np.float32) for b, v in oracle_levels.items()}


@pytest.fixture(scope="session")
def sym_levels32(levels32):
    """The oracle's 2-bit float32 codebook made exactly antisymmetric
    (l[3-k] = -l[k], each pair's magnitude the mean of the oracle's two):
    its middle threshold is the centre of the outer pair, the case in which
    libcq's quantize kernels take their one-product decisions."""
    lv = levels32[2].astype(np.float64)
    h = np.array([(lv[3] - lv[0]) / 2, (lv[2] - lv[1]) / 2]).astype(np.float32)
    out = np.array([-h[0], -h[1], h[1], h[0]], dtype=np.float32)
    assert np.all(out == -out[::-1]) and np.all(np.diff(out) > 0)
    return out
