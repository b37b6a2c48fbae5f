"""GPU parity of ternary trit storage (CQ_TERNARY_TRITS, five indices per
byte) through the C ABI: quantize and dequantize against the oracle, the
multi-tensor calls, and cq_repack against the 2-bit field form.  Each case
prints its name before it touches the GPU."""

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
T = O.TERNARY_TRITS


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lv():
    # The oracle's ternary levels as float32 (the fixed three-level codebook).
    return O.runtime_levels(O.codebook(T)).astype(np.float32)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f16_bits(t):
    return host(t.contiguous().view(torch.int16)).view(np.uint16)


def make(shape, seed, dtype):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    if dtype == "bf16":
        b = W.f32_to_bf16_bits(w)
        return (W.bf16_bits_to_f32(b).astype(np.float64),
                torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(DEV).view(torch.bfloat16))
    return w.astype(np.float64), torch.from_numpy(w).to(DEV)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1000, 384), (77, 1000), (3, 1, 130), (1, 1), (4096, 256)])
def test_trit_quantize_dequantize(dtype, shape, lv):
    w64, w_dev = make(shape, zlib.crc32(repr(("trit", dtype, shape)).encode()), dtype)
    rows = int(np.prod(shape[:-1]))
    cols = shape[-1]
    say(f"trit quantize {dtype}{shape}")
    q = O.quantize(w64, T, lv)
    packed, norms = cq.quantize(w_dev, T, lv)
    assert packed.shape[-1] == 26
    check_quantize(host(packed), f16_bits(norms), q)
    say(f"trit dequantize oracle packing {shape}")
    ref = O.dequantize(q.packed, q.norm16, rows, cols, T, lv)
    out = cq.dequantize(torch.from_numpy(q.packed.reshape(rows, -1)).to(DEV),
                        torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16),
                        rows, cols, T, lv)
    check_dequant(host(out), ref, q.norm16, rows, cols)


def test_trit_equals_field_form_and_repack(lv):
    """Trit quantize equals 2-bit ternary quantize followed by cq_repack, the
    reverse repack gives the field bytes back, and dequantize agrees."""
    w64, w_dev = make((2048, 1024), 3, "bf16")
    say("trit vs field form 2048x1024")
    p2, n2 = cq.quantize(w_dev, O.TERNARY, lv)
    p3, n3 = cq.quantize(w_dev, T, lv)
    assert torch.equal(n2.view(torch.int16), n3.view(torch.int16))
    to3 = cq.repack(p2, O.TERNARY, T)
    assert torch.equal(to3, p3)
    back = cq.repack(p3, T, O.TERNARY)
    assert torch.equal(back, p2)
    d2 = cq.dequantize(p2, n2, 2048, 1024, O.TERNARY, lv)
    d3 = cq.dequantize(p3, n3, 2048, 1024, T, lv)
    assert torch.equal(d2, d3)
    # the oracle's own trit bytes for the same decisions
    q = O.quantize(w64, T, lv)
    check_quantize(host(p3), f16_bits(n3), q)


# The ragged tensors of the first set load element by element (widths 300
# and 1), those of the second in 16-byte pieces (widths 1000 and 200).
@pytest.mark.parametrize("shapes", [[(64, 128), (5, 300), (1, 1), (300, 512), (0, 128), (2, 3, 256)],
                                    [(7, 1000), (64, 128), (3, 200)]])
def test_trit_many_calls(lv, shapes):
    """Mixed shapes through cq_quantize_many / cq_dequantize_many with trit
    storage: identical to the single-tensor calls, blob offsets as laid out."""
    rng = np.random.default_rng(8 + len(shapes))
    ws = [torch.from_numpy((rng.standard_normal(s) * 0.02).astype(np.float32)).to(DEV) for s in shapes]
    say("trit quantize_many")
    blob, views = cq.quantize_many(ws, T, lv)
    po, no, total = O.blob_offsets(shapes, T)
    assert blob.numel() == total
    items = []
    for s, w, (pk, nm) in zip(shapes, ws, views):
        rows, cols = int(np.prod(s[:-1])), s[-1]
        if rows * cols == 0:
            continue
        p1, n1 = cq.quantize(w, T, lv)
        assert torch.equal(p1, pk) and torch.equal(n1.view(torch.int16), nm.view(torch.int16)), s
        items.append((pk.reshape(rows, -1), nm, rows, cols))
    say("trit dequantize_many")
    outs = cq.dequantize_many(items, T, lv, out_dtype=torch.bfloat16)
    for (pk, nm, rows, cols), out in zip(items, outs):
        o1 = cq.dequantize(pk, nm, rows, cols, T, lv, out_dtype=torch.bfloat16)
        assert torch.equal(o1.view(torch.int16), out.view(torch.int16))


def test_trit_needle2_footprint(lv):
    """The 45.5M-parameter set in trit storage: 355,328 + 2,400 groups of
    28 bytes, and oracle parity over the whole set."""
    tensors = W.needle2()
    ws = [torch.from_numpy(w).to(DEV) for _, w in tensors]
    say("trit needle2 quantize_many")
    blob, views = cq.quantize_many(ws, T, lv)
    assert blob.numel() == (355_328 + 2_400) * 28 == O.model_bytes([w.shape for _, w in tensors], T)
    mism = elems = 0
    for (name, w), (pk, nm) in zip(tensors, views):
        rep = check_quantize(host(pk), f16_bits(nm), O.quantize(w.astype(np.float64), T, lv),
                             enforce_count=False)
        mism += rep["index_mismatches"]
        elems += rep["elements"]
    check_count(mism, elems)


@pytest.mark.parametrize("g", [32, 64, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(100, 384), (7, 1000)])
def test_trit_group_sizes(g, dtype, shape, lv):
    """Trit storage at group sizes other than 128 (ceil(G/5) bytes per group):
    quantize and dequantize against the oracle, and equality with 2-bit
    ternary quantize followed by cq_repack (both directions)."""
    w64, w_dev = make(shape, zlib.crc32(repr(("trit-g", g, dtype, shape)).encode()), dtype)
    rows, cols = shape
    say(f"trit G={g} quantize {dtype}{shape}")
    q = O.quantize(w64, T, lv, g)
    packed, norms = cq.quantize(w_dev, T, lv, group_size=g)
    assert packed.shape[-1] == -(-g // 5)
    check_quantize(host(packed), f16_bits(norms), q)
    p2, n2 = cq.quantize(w_dev, O.TERNARY, lv, group_size=g)
    assert torch.equal(cq.repack(p2, O.TERNARY, T, group_size=g), packed)
    assert torch.equal(cq.repack(packed, T, O.TERNARY, group_size=g), p2)
    say(f"trit G={g} dequantize {shape}")
    ref = O.dequantize(q.packed, q.norm16, rows, cols, T, lv, g)
    out = cq.dequantize(torch.from_numpy(q.packed.reshape(rows, -1)).to(DEV),
                        torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16),
                        rows, cols, T, lv, group_size=g)
    check_dequant(host(out), ref, q.norm16, rows, cols, g)


def test_trit_many_calls_group_64(lv):
    """The multi-tensor calls with trit storage at G = 64: 13-byte groups, so
    tensors sit at odd blob offsets."""
    rng = np.random.default_rng(19)
    shapes = [(3, 64), (5, 300), (1, 1), (64, 512)]
    ws = [torch.from_numpy((rng.standard_normal(s) * 0.02).astype(np.float32)).to(DEV) for s in shapes]
    say("trit G=64 quantize_many")
    blob, views = cq.quantize_many(ws, T, lv, group_size=64)
    po, no, total = O.blob_offsets(shapes, T, 64)
    assert blob.numel() == total and any(o % 2 for o in po)
    items = []
    for s, w, (pk, nm) in zip(shapes, ws, views):
        p1, n1 = cq.quantize(w, T, lv, group_size=64)
        assert torch.equal(p1.reshape(-1), pk.reshape(-1)) and torch.equal(n1.view(torch.int16).reshape(-1),
                                                                             nm.view(torch.int16).reshape(-1)), s
        items.append((pk.reshape(s[0], -1), nm, s[0], s[1]))
    say("trit G=64 dequantize_many")
    outs = cq.dequantize_many(items, T, lv, group_size=64)
    for (pk, nm, rows, cols), out in zip(items, outs):
        assert torch.equal(cq.dequantize(pk, nm, rows, cols, T, lv, group_size=64), out)
