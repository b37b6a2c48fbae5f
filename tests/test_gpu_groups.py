"""GPU parity for group sizes other than 128 (32, 64, 256) through the C ABI:
quantize, dequantize and fake quantization against the oracle run with the
same group size.  Each case prints its name before it touches the GPU."""

import sys
import zlib

import numpy as np
import pytest

from oracle import cq_oracle as O
from rotated_codebook_bit_amd import workloads as W
from parity import check_count, check_dequant, check_fake_quant, check_quantize

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_codebook_bit_amd as cq  # noqa: E402

DEV = "cuda"
ALL_BITS = [O.TERNARY, 2, 3, 4]

# In-band index mismatches are correct results (either neighbour is); their
# count is capped at 1e-6 of the elements over the module's whole workload,
# checked by the last test.
TALLY = {"mismatches": 0, "elements": 0}


def tally(rep):
    TALLY["mismatches"] += rep["index_mismatches"]
    TALLY["elements"] += rep["elements"]


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


def make(shape, seed, dtype):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    if dtype == "bf16":
        b = W.f32_to_bf16_bits(w)
        return (W.bf16_bits_to_f32(b).astype(np.float64),
                torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).to(DEV).view(torch.bfloat16))
    return w.astype(np.float64), torch.from_numpy(w).to(DEV)


@pytest.mark.parametrize("g", [32, 64, 256])
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(300, 1000), (64, 512), (3, 1, 37)])
def test_group_size_codec(g, bits, dtype, shape, levels):
    lv = levels[bits]
    w64, w_dev = make(shape, zlib.crc32(repr(("g", g, bits, dtype, shape)).encode()), dtype)
    rows, cols = int(np.prod(shape[:-1])), shape[-1]
    say(f"G={g} quantize bits={bits} {dtype}{shape}")
    q = O.quantize(w64, bits, lv, g)
    packed, norms = cq.quantize(w_dev, bits, lv, group_size=g)
    tally(check_quantize(host(packed), f16_bits(norms), q, enforce_count=False))
    say(f"G={g} dequantize bits={bits}")
    ref = O.dequantize(q.packed, q.norm16, rows, cols, bits, lv, g)
    out = cq.dequantize(torch.from_numpy(q.packed.reshape(rows, -1)).to(DEV),
                        torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16),
                        rows, cols, bits, lv, group_size=g)
    check_dequant(host(out), ref, q.norm16, rows, cols, g)
    say(f"G={g} fake quant bits={bits}")
    fq = cq.fake_quant(w_dev, bits, lv, out_dtype=torch.float32, group_size=g)
    rep = check_fake_quant(host(fq).astype(np.float64), w64, bits, lv, enforce_count=False, g=g)
    TALLY["mismatches"] += rep.get("index_mismatches", 0)
    TALLY["elements"] += rep.get("indices_read_back", 0)


@pytest.mark.parametrize("g", [32, 64, 256])
def test_group_size_special_groups(g, levels):
    """Zero groups, constant groups and norms that overflow binary16."""
    rng = np.random.default_rng(g)
    w = np.concatenate([np.zeros((1, 2 * g)), np.full((1, 2 * g), 0.25), rng.standard_normal((1, 2 * g)),
                        np.full((1, 2 * g), 1e5)], axis=0).astype(np.float32)
    for bits in ALL_BITS:
        say(f"G={g} special groups bits={bits}")
        q = O.quantize(w.astype(np.float64), bits, levels[bits], g)
        packed, norms = cq.quantize(torch.from_numpy(w).to(DEV), bits, levels[bits], group_size=g)
        tally(check_quantize(host(packed), f16_bits(norms), q, enforce_count=False))
        n = f16_bits(norms)
        assert (n[0] == 0).all() and (n[-1] == 0x7C00).all()


@pytest.mark.parametrize("g", [32, 64, 256])
@pytest.mark.parametrize("bits", [2, 3])
def test_group_size_many_calls(g, bits, levels):
    """cq_quantize_many / cq_dequantize_many at other group sizes: the blob at
    the oracle's serialized offsets (some only 4- or 8-byte aligned),
    identical to the single-tensor calls, and parity on one tensor."""
    lv = levels[bits]
    rng = np.random.default_rng(70 + g + bits)
    shapes = [(5, 300), (64, 512), (1, 1), (0, 256), (2, 3, 2 * g), (3, 1000)]
    ws = [torch.from_numpy((rng.standard_normal(s) * 0.02).astype(np.float32)).to(DEV) for s in shapes]
    say(f"G={g} bits={bits} quantize_many")
    blob, views = cq.quantize_many(ws, bits, lv, group_size=g)
    po, no, total = O.blob_offsets(shapes, bits, g)
    assert blob.numel() == total == O.model_bytes(shapes, bits, g)
    assert list(cq.blob_layout(shapes, bits, g)[:2]) == [list(po), list(no)]
    items = []
    for s, w, (pk, nm) in zip(shapes, ws, views):
        rows, cols = int(np.prod(s[:-1])), s[-1]
        if rows * cols == 0:
            continue
        p1, n1 = cq.quantize(w, bits, lv, group_size=g)
        assert torch.equal(p1.reshape(-1), pk.reshape(-1)), s
        assert torch.equal(n1.view(torch.int16).reshape(-1), nm.view(torch.int16).reshape(-1)), s
        items.append((pk.reshape(rows, -1), nm, rows, cols))
    w64 = ws[1].double().cpu().numpy()
    tally(check_quantize(host(views[1][0]), f16_bits(views[1][1]), O.quantize(w64, bits, lv, g),
                         enforce_count=False))
    say(f"G={g} bits={bits} dequantize_many")
    outs = cq.dequantize_many(items, bits, lv, group_size=g)
    for (pk, nm, rows, cols), out in zip(items, outs):
        o1 = cq.dequantize(pk, nm, rows, cols, bits, lv, group_size=g)
        assert torch.equal(o1, out)


def test_zz_mismatch_total():
    say(f"group sizes: {TALLY['mismatches']} in-band mismatches in {TALLY['elements']} elements")
    check_count(TALLY["mismatches"], TALLY["elements"])


@pytest.mark.parametrize("g", [32, 64, 256])
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("batch", [1, 3])
def test_group_size_matvec(g, bits, batch, levels):
    """cq_dequant_matvec at other group sizes against the oracle's x @ W_hat^T
    (batch 1 of 2-bit fields takes the pair-table kernel, batch 3 the
    matrix-core kernel with 4 batch rows per block; both rotate the
    activations partly across lanes), including k not a multiple of the
    1024-column tile."""
    from parity import check_matvec
    lv = levels[bits]
    rng = np.random.default_rng(zlib.crc32(repr(("mv", g, bits, batch)).encode()))
    n_out, k = 300, 1536 if g != 256 else 1280
    q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, bits, lv, g)
    w_hat = O.dequantize(q.packed, q.norm16, n_out, k, bits, lv, g)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    say(f"G={g} matvec bits={bits} batch={batch}")
    y = cq.dequant_matvec(torch.from_numpy(q.packed.reshape(n_out, -1)).to(DEV),
                          torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16),
                          n_out, k, bits, lv, torch.from_numpy(x).to(DEV), group_size=g)
    check_matvec(host(y), x.astype(np.float64) @ w_hat.T, x, w_hat)


@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("batch", [1, 3, 12])
def test_group32_odd_width_matvec(bits, batch, levels):
    """Rows of an odd number of 32-column groups (k = 32 mod 64) take the
    per-lane-table kernel at every batch."""
    from parity import check_matvec
    lv = levels[bits]
    rng = np.random.default_rng(zlib.crc32(repr(("mv32", bits, batch)).encode()))
    n_out, k = 200, 1504
    q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, bits, lv, 32)
    w_hat = O.dequantize(q.packed, q.norm16, n_out, k, bits, lv, 32)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    say(f"G=32 odd-width matvec bits={bits} batch={batch}")
    y = cq.dequant_matvec(torch.from_numpy(q.packed.reshape(n_out, -1)).to(DEV),
                          torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16),
                          n_out, k, bits, lv, torch.from_numpy(x).to(DEV), group_size=32)
    check_matvec(host(y), x.astype(np.float64) @ w_hat.T, x, w_hat)


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("batch", [3, 8, 10])
def test_group32_odd_width_matvec_many(bits, batch, levels):
    """cq_dequant_matvec_many over matrices of an odd number of 32-column
    groups (k = 32 mod 64), which the matrix-core kernel does not take:
    the byte-table kernel runs chunks of 3, 8, and 8 + 2 batch rows."""
    from parity import check_matvec
    lv = levels[bits]
    rng = np.random.default_rng(zlib.crc32(repr(("mvm32", bits, batch)).encode()))
    items, refs = [], []
    for n_out, k in ((70, 1504), (33, 96), (260, 4128)):
        q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, bits, lv, 32)
        w_hat = O.dequantize(q.packed, q.norm16, n_out, k, bits, lv, 32)
        x = rng.standard_normal((batch, k)).astype(np.float32)
        items.append((torch.from_numpy(q.packed.reshape(n_out, -1)).to(DEV),
                      torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16),
                      n_out, k, torch.from_numpy(x).to(DEV),
                      torch.full((batch, n_out), float("nan"), dtype=torch.float32, device=DEV)))
        refs.append((x, w_hat))
    say(f"G=32 odd-width matvec_many bits={bits} batch={batch}")
    cq.dequant_matvec_many(items, bits, lv, batch, group_size=32)
    for it, (x, w_hat) in zip(items, refs):
        check_matvec(host(it[5]), x.astype(np.float64) @ w_hat.T, x, w_hat)


@pytest.mark.parametrize("g", [32, 64, 256])
@pytest.mark.parametrize("bits", ALL_BITS)
def test_group_size_matvec_two_passes(g, bits, levels):
    """The matrix-core kernel with 8 batch rows per block (batch 6: two rows
    past the batch) on rows of two 4096-column passes, where every level is
    scaled by its norm before its products."""
    from parity import check_matvec
    lv = levels[bits]
    rng = np.random.default_rng(zlib.crc32(repr(("mv2", g, bits)).encode()))
    n_out, k, batch = 100, 4352, 6
    q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, bits, lv, g)
    w_hat = O.dequantize(q.packed, q.norm16, n_out, k, bits, lv, g)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    say(f"G={g} two-pass matvec bits={bits} batch={batch}")
    y = cq.dequant_matvec(torch.from_numpy(q.packed.reshape(n_out, -1)).to(DEV),
                          torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16),
                          n_out, k, bits, lv, torch.from_numpy(x).to(DEV), group_size=g)
    check_matvec(host(y), x.astype(np.float64) @ w_hat.T, x, w_hat)


@pytest.mark.parametrize("g", [32, 64, 256])
@pytest.mark.parametrize("bits", ALL_BITS)
@pytest.mark.parametrize("batch", [16, 70])
def test_group_size_gemm(g, bits, batch, levels):
    """cq_dequant_gemm at other group sizes against the oracle (GEMM bound):
    several scaled groups per 128-column tile (32, 64) or one group over two
    tiles (256); batch 70 takes 64-row tiles where the group size allows."""
    from parity import GEMM_TOL, check_matvec
    lv = levels[bits]
    rng = np.random.default_rng(zlib.crc32(repr(("gemm", g, bits, batch)).encode()))
    n_out, k = 300, 1536
    q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, bits, lv, g)
    w_hat = O.dequantize(q.packed, q.norm16, n_out, k, bits, lv, g)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    say(f"G={g} gemm bits={bits} batch={batch}")
    y = cq.dequant_gemm(torch.from_numpy(q.packed.reshape(n_out, -1)).to(DEV),
                        torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16),
                        n_out, k, bits, lv, torch.from_numpy(x).to(DEV), group_size=g)
    check_matvec(host(y), x.astype(np.float64) @ w_hat.T, x, w_hat, tol=GEMM_TOL)


@pytest.mark.parametrize("g", [32, 64, 256])
def test_group_size_gemm_many_groups(g, levels):
    """The thread-per-unit activation rotation (at least 32,768 (group, row)
    units) and many matrices in one call at another group size."""
    from parity import GEMM_TOL, check_matvec
    lv = levels[2]
    rng = np.random.default_rng(90 + g)
    batch = 256
    items, refs = [], []
    for n_out, k in [(64, 8192), (200, 1024), (33, 2048)]:
        q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, 2, lv, g)
        w_hat = O.dequantize(q.packed, q.norm16, n_out, k, 2, lv, g)
        x = rng.standard_normal((batch, k)).astype(np.float32)
        y = torch.full((batch, n_out), float("nan"), dtype=torch.float32, device=DEV)
        items.append((torch.from_numpy(q.packed.reshape(n_out, -1)).to(DEV),
                      torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16), n_out, k,
                      torch.from_numpy(x).to(DEV), y))
        refs.append((x, w_hat))
    say(f"G={g} gemm_many batch={batch}")
    cq.dequant_gemm_many(items, 2, lv, batch, group_size=g)
    for (x, w_hat), it in zip(refs, items):
        check_matvec(host(it[5]), x.astype(np.float64) @ w_hat.T, x, w_hat, tol=GEMM_TOL)
