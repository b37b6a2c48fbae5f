"""GPU parity of the multi-tensor calls (cq_quantize_many, cq_dequantize_many)
and of the serialized blob they write, through the C ABI.

Each tensor of a multi-tensor call must give exactly what the single-tensor
call gives (the same kernels' arithmetic), and the oracle's rules of
tests/parity.py hold per tensor.  Each case prints its name before it touches
the GPU.
"""

import sys
import zlib

import numpy as np
import pytest

from oracle import cq_oracle as O
from rotated_codebook_bit_amd import workloads as W
from parity import check_count, check_dequant, check_quantize

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_codebook_bit_amd as cq  # noqa: E402

DEV = "cuda"
ALL_BITS = [O.TERNARY, 2, 3, 4]


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def levels(levels32):
    # The oracle's float32 codebooks, handed to both sides.
    return {b: levels32[b] for b in ALL_BITS}


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f16_bits(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


def test_quantize_many_needle2_blob(levels):
    """The 45.5M-parameter set (fp32, 91 tensors, the last one ragged) in one
    call: per-tensor oracle parity, the blob equals the oracle's layout of
    the same per-tensor results, and every tensor equals cq_quantize."""
    lv = levels[2]
    tensors = W.needle2()
    ws = [torch.from_numpy(w).to(DEV) for _, w in tensors]
    say(f"quantize_many needle2: {len(ws)} tensors")
    blob, views = cq.quantize_many(ws, 2, lv)
    blob_h = host(blob)
    shapes = [w.shape for _, w in tensors]
    po, no, total = O.blob_offsets(shapes, 2)
    assert blob_h.size == total == 12_162_752
    mism = elems = 0
    for i, ((name, w), (pk, nm)) in enumerate(zip(tensors, views)):
        q = O.quantize(w.astype(np.float64), 2, lv)
        packed, norms = host(pk), f16_bits(nm)
        rep = check_quantize(packed, norms, q, enforce_count=False)
        mism += rep["index_mismatches"]
        elems += rep["elements"]
        # the views sit where the pages' layout puts this tensor
        assert np.array_equal(blob_h[po[i]:po[i] + packed.size], packed.ravel())
        assert np.array_equal(blob_h[no[i]:no[i] + 2 * norms.size].view(np.uint16), norms.ravel())
        if i % 15 == 0 or i == len(tensors) - 1:
            p1, n1 = cq.quantize(ws[i], 2, lv)
            assert np.array_equal(host(p1), packed) and np.array_equal(f16_bits(n1), norms), name
    say(f"quantize_many needle2: {mism} in-band mismatches in {elems} elements")
    check_count(mism, elems)


def test_dequantize_many_needle2(levels):
    """Dequantize the oracle's quantization of the 45.5M set in one call."""
    lv = levels[2]
    tensors = W.needle2()
    qs = [O.quantize(w.astype(np.float64), 2, lv) for _, w in tensors]
    items = []
    for (name, w), q in zip(tensors, qs):
        r, c = w.shape
        items.append((torch.from_numpy(q.packed.reshape(r, -1)).to(DEV),
                      torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16), r, c))
    say(f"dequantize_many needle2: {len(items)} tensors")
    outs = cq.dequantize_many(items, 2, lv)
    for (name, w), q, out in zip(tensors, qs, outs):
        r, c = w.shape
        ref = O.dequantize(q.packed, q.norm16, r, c, 2, lv)
        check_dequant(host(out), ref, q.norm16, r, c)
    # bf16 output of the ragged tensor equals the single-tensor call
    p, n, r, c = items[-1]
    o1 = cq.dequantize(p, n, r, c, 2, lv, out_dtype=torch.bfloat16)
    om = cq.dequantize_many([items[-1]], 2, lv, out_dtype=torch.bfloat16)[0]
    assert torch.equal(o1.view(torch.int16), om.view(torch.int16))


@pytest.mark.parametrize("bits", ALL_BITS)
def test_quantize_many_batch_tails(bits, levels):
    """Tensors whose full 64-group batches are not a multiple of 32 (the
    quantize kernel takes full batches 32 at a time and the rest one by one),
    with partial last batches, in one bf16 call: per-tensor oracle parity and
    bit-identity with the single-tensor call."""
    lv = levels[bits]
    shapes = [(6637, 128), (2213, 384), (4096, 512), (700, 1024), (64 * 33 + 1, 128)]
    rng = np.random.default_rng(zlib.crc32(repr(("tails", bits)).encode()))
    hb = [W.f32_to_bf16_bits((rng.standard_normal(sh) * 0.02).astype(np.float32)) for sh in shapes]
    ws = [torch.from_numpy(b.view(np.int16)).to(DEV).view(torch.bfloat16) for b in hb]
    say(f"quantize_many tails bits={bits}: {shapes}")
    blob, views = cq.quantize_many(ws, bits, lv)
    mism = elems = 0
    for sh, b, w, (pk, nm) in zip(shapes, hb, ws, views):
        q = O.quantize(W.bf16_bits_to_f32(b).astype(np.float64), bits, lv)
        packed, norms = host(pk), f16_bits(nm)
        rep = check_quantize(packed, norms, q, enforce_count=False)
        mism += rep["index_mismatches"]
        elems += rep["elements"]
        p1, n1 = cq.quantize(w, bits, lv)
        assert np.array_equal(host(p1), packed) and np.array_equal(f16_bits(n1), norms), sh
    say(f"quantize_many tails bits={bits}: {mism} in-band mismatches in {elems} elements")
    check_count(mism, elems)


@pytest.mark.parametrize("bits", ALL_BITS + ["sym2"])
def test_many_small_mixed(bits, levels, sym_levels32):
    """Many small tensors of mixed shapes (multiples of 128 and ragged,
    empty, 3-D) in one call, bf16: bit-identical to the single-tensor calls,
    and the oracle's rules on every tensor.  "sym2": 2 bits with an
    antisymmetric codebook."""
    if bits == "sym2":
        bits, lv = 2, sym_levels32
    else:
        lv = levels[bits]
    rng = np.random.default_rng(zlib.crc32(repr(("many", bits)).encode()))
    shapes = []
    for _ in range(150):
        kind = rng.integers(0, 6)
        if kind == 0:
            shapes.append((int(rng.integers(1, 40)), 128 * int(rng.integers(1, 9))))
        elif kind == 1:
            shapes.append((int(rng.integers(1, 40)), int(rng.integers(1, 700))))
        elif kind == 2:
            shapes.append((int(rng.integers(0, 3)), 0) if rng.integers(0, 2) else (0, 256))
        elif kind == 3:
            shapes.append((2, int(rng.integers(1, 5)), 128 * int(rng.integers(1, 4))))
        elif kind == 4:
            shapes.append((int(rng.integers(100, 600)), 256))  # several batches per tensor
        else:
            shapes.append((1, 1))
    bits_h = [W.f32_to_bf16_bits((rng.standard_normal(s) * 0.02).astype(np.float32)) for s in shapes]
    ws = [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(DEV).view(torch.bfloat16)
          for b in bits_h]
    say(f"quantize_many {len(ws)} mixed tensors bits={bits}")
    blob, views = cq.quantize_many(ws, bits, lv)
    mism = elems = 0
    items = []
    for s, b, w, (pk, nm) in zip(shapes, bits_h, ws, views):
        rows = int(np.prod(s[:-1])) if len(s) > 1 else 1
        cols = s[-1]
        if rows * cols == 0:
            continue
        p1, n1 = cq.quantize(w, bits, lv)
        assert np.array_equal(host(p1), host(pk)), s
        assert np.array_equal(f16_bits(n1), f16_bits(nm)), s
        q = O.quantize(W.bf16_bits_to_f32(b).astype(np.float64), bits, lv)
        rep = check_quantize(host(pk), f16_bits(nm), q, enforce_count=False)
        mism += rep["index_mismatches"]
        elems += rep["elements"]
        items.append((pk.reshape(rows, -1), nm, rows, cols))
    check_count(mism, elems)
    say(f"dequantize_many {len(items)} mixed tensors bits={bits}")
    outs = cq.dequantize_many(items, bits, lv)
    for (pk, nm, rows, cols), out in zip(items, outs):
        o1 = cq.dequantize(pk, nm, rows, cols, bits, lv)
        assert torch.equal(o1, out), (rows, cols)


# Ragged tensors of one call load and store in 16-byte pieces when every
# ragged width is a multiple of the piece (8 bf16 or 4 float32 elements),
# else element by element: sets whose widths have gcd 8, 4 and 2.
RAGGED_SETS = [[(7, 1000), (3, 200), (11, 1016)], [(5, 1004), (3, 1000), (2, 12)], [(4, 130), (6, 1000), (1, 1)]]


@pytest.mark.parametrize("bits", ALL_BITS + ["sym2"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("which", range(len(RAGGED_SETS)))
def test_many_ragged_widths(bits, dtype, which, levels, sym_levels32):
    """Only ragged tensors in one call: bit-identical to the single-tensor
    calls (each picks its own load form), and the oracle's rules.  "sym2":
    2 bits with an antisymmetric codebook."""
    if bits == "sym2":
        bits, lv = 2, sym_levels32
    else:
        lv = levels[bits]
    shapes = RAGGED_SETS[which]
    rng = np.random.default_rng(zlib.crc32(repr(("ragged", bits, dtype, which)).encode()))
    hosts = [(rng.standard_normal(s) * 0.02).astype(np.float32) for s in shapes]
    if dtype == "bf16":
        hb = [W.f32_to_bf16_bits(h) for h in hosts]
        ws = [torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(DEV).view(torch.bfloat16) for b in hb]
        w64 = [W.bf16_bits_to_f32(b).astype(np.float64) for b in hb]
    else:
        ws = [torch.from_numpy(h).to(DEV) for h in hosts]
        w64 = [h.astype(np.float64) for h in hosts]
    say(f"quantize_many ragged {shapes} {dtype} bits={bits}")
    blob, views = cq.quantize_many(ws, bits, lv)
    items, refs = [], []
    for s, w, x64, (pk, nm) in zip(shapes, ws, w64, views):
        p1, n1 = cq.quantize(w, bits, lv)
        assert np.array_equal(host(p1), host(pk)), s
        assert np.array_equal(f16_bits(n1), f16_bits(nm)), s
        q = O.quantize(x64, bits, lv)
        check_quantize(host(pk), f16_bits(nm), q)
        # Dequantize the oracle's packing, so the expected values are the
        # oracle's alone.
        items.append((torch.from_numpy(q.packed.reshape(s[0], -1)).to(DEV),
                      torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16), s[0], s[1]))
        refs.append((O.dequantize(q.packed, q.norm16, s[0], s[1], bits, lv), q.norm16))
    say(f"dequantize_many ragged {shapes} bits={bits}")
    for odt in (torch.float32, torch.bfloat16):
        outs = cq.dequantize_many(items, bits, lv, out_dtype=odt)
        for (pk, nm, rows, cols), out, (ref, n16) in zip(items, outs, refs):
            o1 = cq.dequantize(pk, nm, rows, cols, bits, lv, out_dtype=odt)
            if odt == torch.bfloat16:
                assert torch.equal(o1.view(torch.int16), out.view(torch.int16)), (rows, cols, odt)
            else:
                assert torch.equal(o1, out), (rows, cols, odt)
                check_dequant(host(out), ref, n16, rows, cols)


def test_quantize_many_shared_input(levels):
    """Two descriptors may read the same input; their outputs are equal."""
    lv = levels[2]
    w = (torch.randn((64, 512), device=DEV) * 0.02).to(torch.bfloat16)
    say("quantize_many shared input")
    blob, views = cq.quantize_many([w, w], 2, lv)
    assert torch.equal(views[0][0], views[1][0])
    assert torch.equal(views[0][1].view(torch.int16), views[1][1].view(torch.int16))


def test_many_empty_call(levels):
    blob, views = cq.quantize_many([], 2, levels[2])
    assert blob.numel() == 0 and views == []
    assert cq.dequantize_many([], 2, levels[2]) == []
