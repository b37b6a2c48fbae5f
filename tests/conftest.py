import os
import sys

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
