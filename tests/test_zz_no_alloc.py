"""cq_dequant_matvec_many_noalloc (the allocation-free product, workspace in
the library's fixed device array) against cq_dequant_matvec_many on the same
inputs: bit-identical outputs, on two calls in a row, the second smaller,
through the C ABI; both also checked against the oracle's product."""

import sys
import zlib

import numpy as np
import pytest

from oracle import cq_oracle as O
from parity import check_matvec

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rotated_codebook_bit_amd as cq  # noqa: E402

DEV = "cuda"


def say(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def _set(shapes, batch, bits, lv, seed):
    rng = np.random.default_rng(seed)
    mats = []
    for n_out, k in shapes:
        if k:
            q = O.quantize(rng.standard_normal((n_out, k)) * 0.02, bits, lv)
            w_hat = O.dequantize(q.packed, q.norm16, n_out, k, bits, lv)
            p = torch.from_numpy(q.packed.reshape(n_out, -1)).to(DEV)
            nv = torch.from_numpy(q.norm16.view(np.int16)).to(DEV).view(torch.float16)
        else:
            w_hat = np.zeros((n_out, 0))
            p = torch.zeros((n_out, 0), dtype=torch.uint8, device=DEV)
            nv = torch.zeros((n_out, 0), dtype=torch.float16, device=DEV)
        x = rng.standard_normal((batch, k)).astype(np.float32)
        mats.append((p, nv, n_out, k, torch.from_numpy(x).to(DEV), x, w_hat))
    return mats


def _run(mats, bits, lv, batch, fn):
    items = [(p, nv, n_out, k, xd, torch.full((batch, n_out), float("nan"), dtype=torch.float32, device=DEV))
             for p, nv, n_out, k, xd, _, _ in mats]
    fn(items, bits, lv, batch)
    torch.cuda.synchronize()
    return [it[5].cpu().numpy() for it in items]


@pytest.mark.parametrize("bits", [2, 4])
def test_noalloc_equals_stream_ordered_workspace(bits, levels32):
    lv = levels32[bits]
    # First call: mixed shapes, one k = 0 matrix, batch 3 (matrix-core kernel).
    big = [(1000, 4096), (37, 11008), (64, 128), (5, 0), (300, 384), (2048, 1024)]
    # Second call, smaller: fewer matrices, smaller k, batch 1 (pair kernel
    # for 2-bit fields) -- the workspace keeps the first call's contents.
    small = [(77, 256), (513, 512)]
    for name, shapes, batch in (("first", big, 3), ("second", small, 1)):
        mats = _set(shapes, batch, bits, lv, zlib.crc32(repr((name, bits)).encode()))
        say(f"noalloc {name} call bits={bits}: {len(shapes)} matrices, batch {batch}")
        got = _run(mats, bits, lv, batch, cq.dequant_matvec_many_noalloc)
        want = _run(mats, bits, lv, batch, cq.dequant_matvec_many)
        for (_, _, n_out, k, _, x, w_hat), a, b in zip(mats, got, want):
            assert np.array_equal(a, b), f"{n_out}x{k}: outputs differ from the stream-ordered call"
            if k:
                check_matvec(a, x.astype(np.float64) @ w_hat.T, x, w_hat)
            else:
                assert not a.any()
