"""Property tests of libcq's pure host calls against the oracle over random
shapes, widths and group sizes (no GPU): layout, storage size and the
serialized layout agree exactly."""

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import rotated_codebook_bit_amd as cq
from oracle import cq_oracle as O

BITS = st.sampled_from([O.TERNARY, O.TERNARY_TRITS, 1, 2, 3, 4])
GROUPS = st.sampled_from([8, 16, 32, 64, 128, 256, 1024, 4096])
SHAPE = st.tuples(st.integers(0, 5000), st.integers(0, 20000))


@settings(max_examples=300, deadline=None)
@given(shapes=st.lists(SHAPE, min_size=0, max_size=12), bits=BITS, g=GROUPS)
def test_sizes_and_blob_layout_match_oracle(shapes, bits, g):
    assert cq.model_bytes(shapes, bits, g) == O.model_bytes(shapes, bits, g)
    po, no, total = cq.blob_layout(shapes, bits, g)
    want = O.blob_offsets(shapes, bits, g)
    assert (po, no, total) == (list(want[0]), list(want[1]), want[2])
    for (r, c) in shapes:
        ng, pb = cq.layout(r, c, bits, g)
        assert ng == r * (-(-c // g))
        assert pb == ng * O.group_bytes(bits, g)


@settings(max_examples=100, deadline=None)
@given(idx=st.lists(st.integers(0, 2), min_size=1, max_size=700))
def test_trit_pack_round_trip(idx):
    a = np.array(idx)
    assert np.array_equal(O.unpack_trits(O.pack_trits(a), a.size), a)
    assert O.pack_trits(a).size == -(-a.size // 5)
