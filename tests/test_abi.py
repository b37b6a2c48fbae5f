"""C-ABI checks that need no GPU: the library loads, exports every function
include/libcq.h declares, its host-only calls agree with the oracle, and
every argument-validation error is returned before any HIP call (so fake
device pointers are safe here)."""

import ctypes
import json
import os
import re

import numpy as np
import pytest

import rotated_codebook_bit_amd as cq
from oracle import cq_oracle as O
from rotated_codebook_bit_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libcq.h")

OK, E_NULL, E_ARG, E_ALIGN, E_UNSUP = 0, -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cq_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = cq.lib()
    names = declared_functions()
    assert {"cq_quantize", "cq_dequantize", "cq_dequant_matvec", "cq_model_bytes",
            "cq_fake_quant"} <= set(names)
    for name in names:
        assert hasattr(L, name), name
    assert L.cq_version().decode().startswith("libcq")


def test_status_strings():
    L = cq.lib()
    for s in (OK, E_NULL, E_ARG, E_ALIGN, E_UNSUP, -5):
        assert L.cq_status_str(s)
    assert L.cq_status_str(-99) == b"unknown status"


# -- host-only calls vs the oracle ------------------------------------------------

@pytest.mark.parametrize("bits", [O.TERNARY, 1, 2, 3, 4])
def test_codebook_train_equals_oracle_float32(bits, lloyd_samples, oracle_levels):
    got = cq.codebook_train(bits, lloyd_samples)
    want = O.runtime_levels(oracle_levels[bits]).astype(np.float32)
    np.testing.assert_array_equal(got, want)


def test_codebook_train_iterations_and_tiny_example(lloyd_samples):
    import json
    ex = json.load(open(os.path.join(ROOT, "tests", "golden", "hand_examples.json")))["lloyd_tiny"]
    # 1 level-bit = 2 levels, the tiny hand example
    got = cq.codebook_train(1, np.array(ex["samples"]), iters=10)
    np.testing.assert_allclose(got, np.float32(ex["result"]), rtol=0, atol=0)
    got0 = cq.codebook_train(1, np.array(ex["samples"]), iters=0)
    np.testing.assert_array_equal(got0, np.float32(ex["init"]))


# -- the built-in codebook (levels == NULL) ----------------------------------------

@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_builtin_codebook_near_gaussian_optimum(bits):
    """libcq's own Lloyd-Max run on its own N(0,1) generator: the exact
    Gaussian mean-square error of its levels lies within 0.2% above the
    continuous optimum (unique for a log-concave density, so never below)."""
    from test_oracle_codebook import exact_lloyd, gaussian_mse
    lv = cq.codebook(bits)
    n = 1 << bits
    assert lv.dtype == np.float32 and lv.shape == (n,) and np.all(np.diff(lv) > 0)
    d_star = gaussian_mse(exact_lloyd(n))
    d = gaussian_mse(lv.astype(np.float64))
    assert d_star <= d <= 1.002 * d_star


def test_builtin_codebook_two_bit_levels_and_ternary():
    table = json.load(open(os.path.join(ROOT, "tests", "golden", "max1960_gaussian.json")))
    pos = table["quantizers"]["4"]["levels"]
    np.testing.assert_allclose(cq.codebook(2), [-pos[1], -pos[0], pos[0], pos[1]], atol=5e-3)
    np.testing.assert_array_equal(cq.codebook(O.TERNARY_TRITS), np.float32(O.TERNARY_LEVELS))
    np.testing.assert_array_equal(cq.codebook(O.TERNARY), np.float32(O.TERNARY_LEVELS))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_builtin_codebook_is_antisymmetric(bits):
    """The built-in generator's samples come in +- pairs, so the Lloyd-Max
    fixed point it reaches is symmetric about 0: level L-1-k is exactly
    -level k in float32 (then the middle threshold of the four-level code is
    0, the centre of the outer pair)."""
    lv = cq.codebook(bits)
    np.testing.assert_array_equal(lv, -lv[::-1])


def test_codebook_train_keeps_the_plain_recipe(lloyd_samples):
    """Caller samples get the page's recipe as it stands (plain quantile
    start, no symmetrisation; equal to the oracle's levels, see
    test_codebook_train_equals_oracle_float32): the pages' draws are not
    symmetric, nor are their levels."""
    trained = cq.codebook_train(2, lloyd_samples)
    assert not np.array_equal(trained, -trained[::-1])


def test_builtin_codebook_is_cached_and_independent_of_the_pages_draws(lloyd_samples):
    a = [cq.codebook(b) for b in (1, 2, 3, 4)]
    b = [cq.codebook(b) for b in (1, 2, 3, 4)]
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    # Its own generator, not the pages' seeded draws: close, not equal.
    trained = cq.codebook_train(2, lloyd_samples)
    assert not np.array_equal(a[1], trained)
    np.testing.assert_allclose(a[1], trained, atol=1e-2)


def test_layout_and_model_bytes():
    assert cq.layout(300, 1000, 2) == (2400, 2400 * 32)
    assert cq.layout(7, 128, 3) == (7, 7 * 48)
    assert cq.layout(0, 5, 4) == (0, 0)
    shapes = [s for _, s in W.needle2_shapes()]
    for bits in (O.TERNARY, 1, 2, 3, 4):
        assert cq.model_bytes(shapes, bits) == O.model_bytes(shapes, bits)
    assert cq.model_bytes(shapes, 2) == 12_162_752
    for g in (32, 64, 256):
        assert cq.model_bytes([(3, 1000)], 2, g) == O.model_bytes([(3, 1000)], 2, g)
    assert cq.model_bytes([], 2) == 0
    assert cq.model_bytes([(2, 3, 129)], 4) == O.model_bytes([(2, 3, 129)], 4)


def test_llama7b_byte_counts():
    shapes = W.llama7b_shapes()
    params = sum(r * c for r, c in shapes)
    assert params == 6_607_077_376
    assert cq.model_bytes(shapes, 2) == 1_651_769_344 + 103_235_584


# -- validation (no HIP call is reached) ---------------------------------------

F = ctypes.POINTER(ctypes.c_float)
FAKE = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x900000)
FAKE3 = ctypes.c_void_p(0x1100000)


def _levels(n):
    arr = np.linspace(-1.5, 1.5, n).astype(np.float32)
    return arr, arr.ctypes.data_as(F)


def quant(w=FAKE, dt=0, rows=4, cols=256, bits=2, g=128, levels=None, nl=None, packed=FAKE2,
          norms=FAKE3):
    lv, lp = _levels(4 if nl is None else nl) if levels is None else levels
    if nl is None:
        nl = lv.size
    return cq.lib().cq_quantize(w, dt, rows, cols, bits, g, lp, nl, packed, norms, None)


def test_quantize_validation():
    L = cq.lib()
    assert quant(bits=5) == E_ARG
    assert quant(bits=1) == E_ARG               # host-only width
    assert quant(dt=7) == E_ARG
    assert quant(rows=-1) == E_ARG
    assert quant(g=512) == E_UNSUP
    assert quant(nl=3) == E_ARG                 # 2 bits needs 4 levels
    bad = np.array([0.0, 0.0, 1.0, 2.0], dtype=np.float32)
    assert quant(levels=(bad, bad.ctypes.data_as(F))) == E_ARG
    nan = np.array([0.0, np.nan, 1.0, 2.0], dtype=np.float32)
    assert quant(levels=(nan, nan.ctypes.data_as(F))) == E_ARG
    # NULL levels select the built-in table and pass validation whatever
    # n_levels says: the call gets as far as the next check (alignment).
    assert quant(levels=(np.zeros(4, np.float32), None), w=ctypes.c_void_p(0x100004)) == E_ALIGN
    assert quant(levels=(np.zeros(4, np.float32), None), nl=0, w=ctypes.c_void_p(0x100004)) == E_ALIGN
    assert quant(levels=(np.zeros(4, np.float32), None), nl=0, rows=0) == OK
    assert quant(w=None) == E_NULL
    assert quant(packed=None) == E_NULL
    assert quant(w=ctypes.c_void_p(0x100004)) == E_ALIGN
    assert quant(norms=ctypes.c_void_p(0x1100001)) == E_ALIGN
    assert quant(packed=ctypes.c_void_p(0x100010)) == E_ARG   # overlaps w
    assert L.cq_last_error()
    # empty tensors are a no-op even with NULL pointers
    assert quant(rows=0, w=None, packed=None, norms=None) == OK
    assert quant(cols=0, w=None, packed=None, norms=None) == OK


def test_dequantize_validation():
    L = cq.lib()
    lv, lp = _levels(8)

    def deq(packed=FAKE, norms=FAKE2, rows=4, cols=256, bits=3, g=128, out=FAKE3, dt=0, nl=8):
        return L.cq_dequantize(packed, norms, rows, cols, bits, g, lp, nl, out, dt, None)

    assert deq(dt=2) == E_ARG
    assert deq(bits=7) == E_ARG
    assert deq(g=512) == E_UNSUP
    assert deq(nl=4) == E_ARG
    assert deq(out=None) == E_NULL
    assert deq(out=ctypes.c_void_p(0x1100008)) == E_ALIGN
    assert deq(out=ctypes.c_void_p(0x100000 + 64)) == E_ARG      # overlaps packed
    assert deq(rows=0, packed=None, norms=None, out=None) == OK


def test_matvec_validation():
    L = cq.lib()
    lv, lp = _levels(4)

    def mv(packed=FAKE, norms=FAKE2, n_out=8, k=256, bits=2, x=ctypes.c_void_p(0x2100000), batch=1,
           y=ctypes.c_void_p(0x3100000), g=128, nl=4):
        return L.cq_dequant_matvec(packed, norms, n_out, k, bits, g, lp, nl, x, batch, y, None)

    assert mv(k=200) == E_UNSUP
    assert mv(g=512) == E_UNSUP
    assert mv(g=64, k=96) == E_UNSUP                                 # k % G != 0
    assert mv(g=32, batch=0) == E_ARG                                # G = 32 validates as 128 does
    assert mv(batch=0) == E_ARG
    assert mv(bits=158, nl=4) == E_ARG
    assert mv(x=None) == E_NULL
    assert mv(y=None) == E_NULL
    assert mv(x=ctypes.c_void_p(0x2100004)) == E_ALIGN
    assert mv(y=ctypes.c_void_p(0x2100000)) == E_ARG              # y overlaps x
    assert mv(n_out=0, packed=None, norms=None, x=None, y=None) == OK


def test_host_call_validation():
    L = cq.lib()
    out = (ctypes.c_float * 16)()
    n = ctypes.c_int()
    assert L.cq_codebook_train(2, None, 10, 200, out, ctypes.byref(n)) == E_NULL
    s = np.zeros(3)
    assert L.cq_codebook_train(2, s.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), 3, 200, out,
                               ctypes.byref(n)) == E_ARG        # fewer samples than levels
    assert L.cq_codebook_train(9, None, 0, 200, out, ctypes.byref(n)) == E_ARG
    assert L.cq_codebook_train(158, None, 0, 0, out, ctypes.byref(n)) == OK and n.value == 3
    assert L.cq_codebook(9, out, ctypes.byref(n)) == E_ARG
    assert L.cq_codebook(2, None, ctypes.byref(n)) == E_NULL
    assert L.cq_codebook(2, out, None) == E_NULL
    assert L.cq_codebook(4, out, ctypes.byref(n)) == OK and n.value == 16
    ng = ctypes.c_int64()
    assert L.cq_layout(1, 1, 2, 96, ctypes.byref(ng), None) == E_ARG
    assert L.cq_layout(-1, 1, 2, 128, ctypes.byref(ng), None) == E_ARG
    r = (ctypes.c_int64 * 1)(-5)
    c = (ctypes.c_int64 * 1)(5)
    b = ctypes.c_uint64()
    assert L.cq_model_bytes(1, r, c, 2, 128, ctypes.byref(b)) == E_ARG
    assert L.cq_model_bytes(1, None, None, 2, 128, ctypes.byref(b)) == E_NULL
    assert L.cq_model_bytes(1, r, c, 2, 128, None) == E_NULL


def test_python_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(cq, "_lib", None)
    monkeypatch.setattr(cq, "LIB_PATH", "/nonexistent/libcq.so")
    with pytest.raises(ImportError):
        cq.lib()


def test_matvec_many_validation():
    L = cq.lib()
    lv, lp = _levels(4)
    D = cq.MatvecDesc

    def many(descs, n=None, batch=1, bits=2, nl=4):
        arr = (D * max(len(descs), 1))(*descs)
        return L.cq_dequant_matvec_many(len(descs) if n is None else n, arr if descs else None, bits, 128,
                                        lp, nl, batch, None)

    good = D(0x100000, 0x900000, 8, 256, 0x2100000, 0x3100000)
    assert many([], n=0) == OK
    assert many([good], n=-1) == E_ARG
    assert L.cq_dequant_matvec_many(1, None, 2, 128, lp, 4, 1, None) == E_NULL
    assert many([good], batch=0) == E_ARG
    assert many([good, D(0x100000, 0x900000, 8, 200, 0x2100000, 0x3100000)]) == E_UNSUP
    assert many([good, D(0x100000, 0x900000, 8, 256, 0x2100000, 0)]) == E_NULL
    assert many([D(0x100000, 0x900000, 8, 256, 0x2100004, 0x3100000)]) == E_ALIGN
    assert many([D(0x100000, 0x900000, 8, 256, 0x2100000, 0x2100000)]) == E_ARG   # y overlaps x
    assert many([D(0, 0, 0, 256, 0, 0)]) == OK                                    # empty matrix


def test_fake_quant_validation():
    L = cq.lib()
    lv, lp = _levels(4)

    def fq(w=FAKE, dt=1, rows=4, cols=256, bits=2, g=128, nl=4, out=FAKE2, odt=0):
        return L.cq_fake_quant(w, dt, rows, cols, bits, g, lp if nl == 4 else _levels(nl)[1], nl,
                               out, odt, None)

    assert fq(dt=3) == E_ARG
    assert fq(odt=-1) == E_ARG
    assert fq(bits=1) == E_ARG
    assert fq(g=16) == E_UNSUP
    assert fq(nl=8) == E_ARG
    assert fq(rows=-2) == E_ARG
    assert fq(w=None) == E_NULL
    assert fq(out=None) == E_NULL
    assert fq(out=ctypes.c_void_p(0x900008)) == E_ALIGN
    assert fq(out=ctypes.c_void_p(0x100000 + 1024)) == E_ARG        # partial overlap
    assert fq(out=FAKE, dt=1, odt=0) == E_ARG                          # in place, dtypes differ
    assert fq(rows=0, w=None, out=None) == OK


# -- multi-tensor calls and the serialized layout -------------------------------------

def test_blob_layout_equals_oracle():
    shapes = [s for _, s in W.needle2_shapes()] + [(2, 3, 130), (1, 1), (0, 128)]
    for bits in (O.TERNARY, O.TERNARY_TRITS, 1, 2, 3, 4):
        for g in (8, 32, 64, 128, 256):
            po, no, total = cq.blob_layout(shapes, bits, g)
            want = O.blob_offsets(shapes, bits, g)
            assert (po, no, total) == (list(want[0]), list(want[1]), want[2])
            # model bytes, plus one pad byte after an odd-length index section
            groups = sum(int(np.prod(s[:-1])) * -(-s[-1] // g) for s in shapes)
            index_bytes = groups * O.group_bytes(bits, g)
            assert total == cq.model_bytes(shapes, bits, g) + index_bytes % 2
            assert no[0] == index_bytes + index_bytes % 2
    ex = json.load(open(os.path.join(ROOT, "tests", "golden", "hand_examples.json")))["blob_two_groups"]
    assert cq.blob_layout([(1, 128), (1, 128)], 2) == (ex["packed_offsets"], ex["norm_offsets"], ex["total"])
    assert cq.blob_layout([], 2) == ([], [], 0)


def test_blob_layout_validation():
    L = cq.lib()
    r = (ctypes.c_int64 * 2)(3, -1)
    c = (ctypes.c_int64 * 2)(128, 128)
    t = ctypes.c_int64()
    assert L.cq_blob_layout(2, r, c, 2, 128, None, None, ctypes.byref(t)) == E_ARG
    assert L.cq_blob_layout(1, None, c, 2, 128, None, None, ctypes.byref(t)) == E_NULL
    assert L.cq_blob_layout(1, r, c, 2, 4, None, None, ctypes.byref(t)) == E_ARG     # G < 8
    assert L.cq_blob_layout(1, r, c, 5, 128, None, None, ctypes.byref(t)) == E_ARG
    assert L.cq_blob_layout(1, r, c, 2, 128, None, None, None) == OK
    u = ctypes.c_uint64()
    assert L.cq_model_bytes(1, r, c, 2, 4, ctypes.byref(u)) == E_ARG


def _qdesc(w=0x100000, rows=4, cols=256, packed=0x900000, norms=0x1100000):
    return cq.QuantDesc(w, rows, cols, packed, norms)


def test_quantize_many_validation():
    L = cq.lib()
    lv, lp = _levels(4)

    def qm(descs, n=None, dt=1, bits=2, g=128, nl=4):
        arr = (cq.QuantDesc * max(len(descs), 1))(*descs)
        return L.cq_quantize_many(len(descs) if n is None else n, arr if descs else None, dt, bits, g,
                                  lp if nl == 4 else _levels(nl)[1], nl, None)

    good = _qdesc()
    assert qm([], n=0) == OK
    assert qm([good], n=-1) == E_ARG
    assert L.cq_quantize_many(1, None, 1, 2, 128, lp, 4, None) == E_NULL
    assert qm([good], dt=2) == E_ARG
    assert qm([good], g=512) == E_UNSUP
    assert qm([good], g=16) == E_UNSUP
    assert qm([good], bits=O.TERNARY_TRITS, nl=3, g=512) == E_UNSUP
    assert qm([good, _qdesc(rows=-1)], g=64) == E_ARG                  # G = 64 validates as 128 does
    assert qm([good], nl=8) == E_ARG
    assert qm([good, _qdesc(rows=-1)]) == E_ARG
    assert qm([good, _qdesc(w=0)]) == E_NULL
    assert qm([good, _qdesc(w=0x100008)]) == E_ALIGN
    assert qm([good, _qdesc(norms=0x1100001)]) == E_ALIGN
    # 4 x 256 bf16 = 2 KiB input, 8 groups: 256 B packed, 16 B norms
    assert qm([good, _qdesc(w=0x200000, packed=0x900000 + 128, norms=0x1200000)]) == E_ARG  # outputs overlap
    assert qm([good, _qdesc(w=0x200000, packed=0x100000 + 512, norms=0x1200000)]) == E_ARG  # into an input
    assert qm([_qdesc(rows=0, w=0, packed=0, norms=0), _qdesc(cols=0, w=0, packed=0, norms=0)]) == OK
    assert L.cq_last_error() is not None


def test_dequantize_many_validation():
    L = cq.lib()
    lv, lp = _levels(4)
    D = cq.DequantDesc

    def dm(descs, n=None, dt=0, bits=2, g=128):
        arr = (D * max(len(descs), 1))(*descs)
        return L.cq_dequantize_many(len(descs) if n is None else n, arr if descs else None, bits, g, lp, 4,
                                    dt, None)

    good = D(0x100000, 0x900000, 4, 256, 0x1100000)
    assert dm([], n=0) == OK
    assert dm([good], dt=5) == E_ARG
    assert dm([good], g=512) == E_UNSUP
    assert dm([good, D(0, 0x900000, 4, 256, 0x1200000)], g=256) == E_NULL
    assert dm([good, D(0, 0x900000, 4, 256, 0x1200000)]) == E_NULL
    assert dm([good, D(0x100000, 0x900000, 4, 256, 0x1200004)]) == E_ALIGN
    # 4 x 256 f32 = 4 KiB outputs
    assert dm([good, D(0x100000, 0x900000, 4, 256, 0x1100000 + 4000)]) == E_ARG        # outputs overlap
    assert dm([good, D(0x100000, 0x900000, 4, 256, 0x100000 + 16)]) == E_ARG            # out over packed
    assert dm([D(0, 0, 0, 256, 0)]) == OK


def test_gemm_validation():
    L = cq.lib()
    lv, lp = _levels(4)
    D = cq.MatvecDesc

    def gm(packed=FAKE, norms=FAKE2, n_out=8, k=256, bits=2, x=ctypes.c_void_p(0x2100000), batch=16,
           y=ctypes.c_void_p(0x3100000), g=128, nl=4):
        return L.cq_dequant_gemm(packed, norms, n_out, k, bits, g, lp, nl, x, batch, y, None)

    assert gm(k=200) == E_UNSUP
    assert gm(g=512) == E_UNSUP
    assert gm(g=64, k=192) == E_UNSUP                                 # tiles of 128 columns
    assert gm(batch=0) == E_ARG
    assert gm(bits=158, nl=4) == E_ARG
    assert gm(x=None) == E_NULL
    assert gm(y=None) == E_NULL
    assert gm(x=ctypes.c_void_p(0x2100004)) == E_ALIGN
    assert gm(y=ctypes.c_void_p(0x2100000)) == E_ARG               # y overlaps x
    assert gm(y=ctypes.c_void_p(0x100000 + 32)) == E_ARG            # y overlaps packed
    assert gm(n_out=0, packed=None, norms=None, x=None, y=None) == OK

    def many(descs, batch=16):
        arr = (D * max(len(descs), 1))(*descs)
        return L.cq_dequant_gemm_many(len(descs), arr if descs else None, 2, 128, lp, 4, batch, None)

    good = D(0x100000, 0x900000, 8, 256, 0x2100000, 0x3100000)
    assert many([]) == OK
    assert many([good], batch=-1) == E_ARG
    # the second matrix's y lands on the first one's y
    assert many([good, D(0x100000, 0x900000, 8, 256, 0x2100000, 0x3100000 + 64)]) == E_ARG
    assert many([good, D(0x100000, 0x900000, 8, 256, 0, 0x4100000)]) == E_NULL


# -- trit storage ------------------------------------------------------------------------

def test_trit_sizes_equal_oracle():
    T = O.TERNARY_TRITS
    assert cq.TERNARY_TRITS == T == 159
    assert cq.layout(300, 1000, T) == (2400, 2400 * 26)
    shapes = [s for _, s in W.needle2_shapes()] + [(2, 3, 130)]
    for g in (8, 64, 128, 256):
        assert cq.model_bytes(shapes, T, g) == O.model_bytes(shapes, T, g)
        po, no, total = cq.blob_layout(shapes, T, g)
        want = O.blob_offsets(shapes, T, g)
        assert (po, no, total) == (list(want[0]), list(want[1]), want[2])
    np.testing.assert_array_equal(cq.codebook(T), np.float32(O.TERNARY_LEVELS))


def test_trit_validation():
    L = cq.lib()
    lv, lp = _levels(3)
    T = O.TERNARY_TRITS
    # the product calls decode 2-bit fields only
    assert L.cq_dequant_matvec(FAKE, FAKE2, 8, 256, T, 128, lp, 3, ctypes.c_void_p(0x2100000), 1,
                               ctypes.c_void_p(0x3100000), None) == E_UNSUP
    assert L.cq_dequant_gemm(FAKE, FAKE2, 8, 256, T, 128, lp, 3, ctypes.c_void_p(0x2100000), 16,
                             ctypes.c_void_p(0x3100000), None) == E_UNSUP
    assert "cq_repack" in L.cq_last_error().decode()
    # quantize with trit storage validates like any width
    assert L.cq_quantize(FAKE, 0, 4, 256, T, 128, lp, 4, FAKE2, FAKE3, None) == E_ARG   # 3 levels needed
    assert L.cq_quantize(FAKE, 0, 4, 256, T, 128, lp, 3, ctypes.c_void_p(0x100000 + 16), FAKE3,
                         None) == E_ARG                                                   # packed overlaps w
    # repack
    R = L.cq_repack
    assert R(FAKE, 2, FAKE2, T, 10, 128, None) == E_ARG          # only ternary <-> trits
    assert R(FAKE, T, FAKE2, T, 10, 128, None) == E_ARG
    assert R(FAKE, O.TERNARY, FAKE2, T, -1, 128, None) == E_ARG
    assert R(FAKE, O.TERNARY, FAKE2, T, 10, 512, None) == E_UNSUP
    assert R(ctypes.c_void_p(0x100002), O.TERNARY, FAKE2, T, 10, 64, None) == E_ALIGN   # fields 4-B at 64
    assert R(None, O.TERNARY, FAKE2, T, 10, 128, None) == E_NULL
    assert R(ctypes.c_void_p(0x100008), O.TERNARY, FAKE2, T, 10, 128, None) == E_ALIGN   # fields 16-B
    assert R(FAKE, O.TERNARY, ctypes.c_void_p(0x900001), T, 10, 128, None) == E_ALIGN   # trits 2-B
    assert R(FAKE, O.TERNARY, ctypes.c_void_p(0x100000 + 300), T, 10, 128, None) == E_ARG  # overlap
    assert R(None, O.TERNARY, None, T, 0, 128, None) == OK


def test_group_size_support():
    L = cq.lib()
    lv, lp = _levels(4)
    lv3, lp3 = _levels(3)
    # codec calls: 32, 64, 128, 256; others unsupported; trit storage at 128 only
    assert quant(g=16) == E_UNSUP
    assert quant(g=1024) == E_UNSUP
    assert L.cq_quantize(FAKE, 0, 4, 256, O.TERNARY_TRITS, 16, lp3, 3, FAKE2, FAKE3, None) == E_UNSUP
    # the products take the codec sizes too; repack takes 128 only
    assert L.cq_dequant_matvec(FAKE, FAKE2, 8, 256, 2, 512, lp, 4, ctypes.c_void_p(0x2100000), 1,
                               ctypes.c_void_p(0x3100000), None) == E_UNSUP
    assert L.cq_dequant_gemm(FAKE, FAKE2, 8, 256, 2, 512, lp, 4, ctypes.c_void_p(0x2100000), 16,
                             ctypes.c_void_p(0x3100000), None) == E_UNSUP
    # the GEMM runs 128-column tiles at every group size
    assert L.cq_dequant_gemm(FAKE, FAKE2, 8, 192, 2, 64, lp, 4, ctypes.c_void_p(0x2100000), 16,
                             ctypes.c_void_p(0x3100000), None) == E_UNSUP
    assert L.cq_dequant_gemm(FAKE, FAKE2, 8, 384, 2, 256, lp, 4, ctypes.c_void_p(0x2100000), 16,
                             ctypes.c_void_p(0x3100000), None) == E_UNSUP
    assert L.cq_repack(FAKE, O.TERNARY, FAKE2, O.TERNARY_TRITS, 4, 512, None) == E_UNSUP
    # sizes for other group sizes
    assert cq.layout(3, 200, 2, 64) == (12, 12 * 16)
    assert cq.layout(3, 200, 4, 256) == (3, 3 * 128)


def test_matvec_many_noalloc_rejects_beyond_its_workspace():
    """The allocation-free product checks its workspace need (about 56 bytes
    per matrix plus batch * sum(k) * 4 bytes) against its fixed 16 MiB before
    any device work, so fake device pointers are safe here."""
    L = cq.lib()
    lv, lp = _levels(4)
    # 8 rows x k = 2^20 at batch 8: 32 MiB of rotated activations.
    k = 1 << 20
    d = (cq.MatvecDesc * 1)(cq.MatvecDesc(0x1000000, 0x9000000, 8, k, 0x20000000, 0x60000000))
    assert L.cq_dequant_matvec_many_noalloc(1, d, 2, 128, lp, 4, 8, None) == E_UNSUP
    assert b"16777216" in L.cq_last_error()
    # Argument errors come first, as for cq_dequant_matvec_many.
    assert L.cq_dequant_matvec_many_noalloc(1, d, 2, 128, lp, 4, 0, None) == E_ARG
    assert L.cq_dequant_matvec_many_noalloc(1, d, 5, 128, lp, 4, 1, None) == E_ARG
    assert L.cq_dequant_matvec_many_noalloc(0, None, 2, 128, lp, 4, 1, None) == OK
