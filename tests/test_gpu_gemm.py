"""GPU parity of the matrix-core dequant-GEMM (cq_dequant_gemm,
cq_dequant_gemm_many) against the oracle's x @ W_hat^T in float64, through the
C ABI, under the GEMM bound of tests/parity.py (5e-5 * ||x_b|| * ||W_hat_n||,
derived from the split-bf16 arithmetic).  Batches cover one block row, several,
and ragged tails; output counts cover partial 256-column tiles.  Each case
prints its name before it touches the GPU.
"""

import sys
import zlib

import numpy as np
import pytest

from oracle import cq_oracle as O
from rotated_codebook_bit_amd import workloads as W
from parity import GEMM_TOL, MV_TOL, check_matvec

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


def dev_q(q, rows):
    return (torch.from_numpy(q.packed.reshape(rows, -1)).to(DEV),
            torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16))


@pytest.fixture(scope="module")
def weight(levels):
    """The 11008 x 4096 bf16 matrix quantized by the oracle (2-bit), and its
    oracle reconstruction."""
    lv = levels[2]
    b = W.matvec_weight_bits()
    q = O.quantize(W.bf16_bits_to_f32(b).astype(np.float64), 2, lv)
    w_hat = O.dequantize(q.packed, q.norm16, 11008, 4096, 2, lv)
    return q, w_hat


@pytest.mark.parametrize("batch", [16, 64, 100, 256, 1])
def test_gemm_weight(batch, weight, levels):
    q, w_hat = weight
    x = np.random.default_rng(zlib.crc32(repr(("gemm", batch)).encode())).standard_normal(
        (batch, 4096)).astype(np.float32)
    y_ref = x.astype(np.float64) @ w_hat.T
    p, n = dev_q(q, 11008)
    say(f"gemm 11008x4096 batch={batch}")
    y = host(cq.dequant_gemm(p, n, 11008, 4096, 2, levels[2], torch.from_numpy(x).to(DEV)))
    rep = check_matvec(y, y_ref, x, w_hat, tol=GEMM_TOL)
    say(f"gemm batch={batch}: {rep.line()}")


@pytest.mark.parametrize("bits", [O.TERNARY, 3, 4])
@pytest.mark.parametrize("n_out,k", [(300, 384), (37, 11008), (513, 128)])
def test_gemm_bits_shapes(bits, n_out, k, levels):
    lv = levels[bits]
    rng = np.random.default_rng(zlib.crc32(repr(("gemm", bits, n_out, k)).encode()))
    w = rng.standard_normal((n_out, k)) * 0.02
    q = O.quantize(w, bits, lv)
    w_hat = O.dequantize(q.packed, q.norm16, n_out, k, bits, lv)
    x = rng.standard_normal((70, k)).astype(np.float32)
    y_ref = x.astype(np.float64) @ w_hat.T
    p, n = dev_q(q, n_out)
    say(f"gemm bits={bits} {n_out}x{k} batch=70")
    y = host(cq.dequant_gemm(p, n, n_out, k, bits, lv, torch.from_numpy(x).to(DEV)))
    rep = check_matvec(y, y_ref, x, w_hat, tol=GEMM_TOL)
    say(f"gemm bits={bits}: {rep.line()}")


def test_gemm_many(levels):
    """Several matrices in one call, two of them reading the same x, one with
    k = 0 (an empty sum: zeros)."""
    lv = levels[2]
    rng = np.random.default_rng(21)
    batch = 33
    shapes = [(256, 512), (300, 512), (1000, 256), (64, 1024), (7, 0)]
    xs = {512: rng.standard_normal((batch, 512)).astype(np.float32)}
    items, refs = [], []
    for n_out, k in shapes:
        if k not in xs:
            xs[k] = rng.standard_normal((batch, k)).astype(np.float32)
        if k:
            q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, 2, lv)
            w_hat = O.dequantize(q.packed, q.norm16, n_out, k, 2, lv)
            p, n = dev_q(q, n_out)
        else:
            w_hat = np.zeros((n_out, 0))
            p = torch.zeros((n_out, 0), dtype=torch.uint8, device=DEV)
            n = torch.zeros((n_out, 0), dtype=torch.float16, device=DEV)
        y = torch.full((batch, n_out), float("nan"), dtype=torch.float32, device=DEV)
        items.append((p, n, n_out, k, torch.from_numpy(xs[k]).to(DEV), y))
        refs.append((xs[k], w_hat))
    say(f"gemm_many {len(items)} matrices batch={batch}")
    ys = cq.dequant_gemm_many(items, 2, lv, batch)
    for (x, w_hat), y in zip(refs, ys):
        yh = host(y)
        if w_hat.shape[1] == 0:
            assert not yh.any()
        else:
            check_matvec(yh, x.astype(np.float64) @ w_hat.T, x, w_hat, tol=GEMM_TOL)


def test_gemm_deterministic_and_close_to_matvec(weight, levels):
    """Two runs are bit-identical; the GEMM agrees with the exact-fp32 matvec
    within the two bounds combined."""
    q, w_hat = weight
    x = np.random.default_rng(5).standard_normal((40, 4096)).astype(np.float32)
    p, n = dev_q(q, 11008)
    xd = torch.from_numpy(x).to(DEV)
    say("gemm determinism")
    a = host(cq.dequant_gemm(p, n, 11008, 4096, 2, levels[2], xd))
    b = host(cq.dequant_gemm(p, n, 11008, 4096, 2, levels[2], xd))
    assert np.array_equal(a, b)
    m = host(cq.dequant_matvec(p, n, 11008, 4096, 2, levels[2], xd))
    check_matvec(a, m.astype(np.float64), x, w_hat, tol=GEMM_TOL + MV_TOL)


@pytest.mark.parametrize("batch", [32, 64, 3])
@pytest.mark.parametrize("n_out,k", [(512, 16384), (256, 128)])
def test_gemm_and_matvec_edges(batch, n_out, k, levels):
    """Tile boundaries (batch 32 / 64, outputs a multiple of 256), a long row
    (k = 16384: 128 groups, 4 matvec passes) and a single-group row, through
    both product calls."""
    lv = levels[2]
    rng = np.random.default_rng(zlib.crc32(repr(("edge", batch, n_out, k)).encode()))
    q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, 2, lv)
    w_hat = O.dequantize(q.packed, q.norm16, n_out, k, 2, lv)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    y_ref = x.astype(np.float64) @ w_hat.T
    p, n = dev_q(q, n_out)
    xd = torch.from_numpy(x).to(DEV)
    say(f"edges gemm+matvec {n_out}x{k} batch={batch}")
    check_matvec(host(cq.dequant_gemm(p, n, n_out, k, 2, lv, xd)), y_ref, x, w_hat, tol=GEMM_TOL)
    check_matvec(host(cq.dequant_matvec(p, n, n_out, k, 2, lv, xd)), y_ref, x, w_hat, tol=MV_TOL)


def test_gemm_and_matvec_many_groups(levels):
    """k = 16384 at batch 256: 32,768 (group, row) units, where both products
    rotate the activations with one thread per unit instead of one wave."""
    lv = levels[2]
    rng = np.random.default_rng(61)
    n_out, k, batch = 64, 16384, 256
    q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, 2, lv)
    w_hat = O.dequantize(q.packed, q.norm16, n_out, k, 2, lv)
    x = rng.standard_normal((batch, k)).astype(np.float32)
    y_ref = x.astype(np.float64) @ w_hat.T
    p, n = dev_q(q, n_out)
    xd = torch.from_numpy(x).to(DEV)
    say(f"gemm+matvec {n_out}x{k} batch={batch} (thread-per-unit rotation)")
    check_matvec(host(cq.dequant_gemm(p, n, n_out, k, 2, lv, xd)), y_ref, x, w_hat, tol=GEMM_TOL)
    check_matvec(host(cq.dequant_matvec(p, n, n_out, k, 2, lv, xd)), y_ref, x, w_hat, tol=MV_TOL)
