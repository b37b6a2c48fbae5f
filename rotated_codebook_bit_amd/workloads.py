"""Seeded synthetic inputs for the CQ quantizer.

This module only draws random numbers and converts dtypes; it holds none of
the quantizer's arithmetic.  Both the oracle tests and the GPU tests / bench
take their inputs from here, so the two sides see identical data.

Workloads (shapes and distributions follow the pages' own workloads, which
are "random matrices", a 45M-parameter model and 7B-parameter models; no
dataset or trained weights are used):

* ``small``      fp32 256x512, N(0, 0.02^2), numpy default_rng(0).
* ``needle2``    the 45.5M-parameter set: embedding 8192x512, then 15 layers of
                 q 512x512, k 512x128, v 512x128, o 512x512, up 512x2048,
                 down 2048x512, then one 300x1000 tensor that needs padding;
                 fp32 N(0, 0.02^2), one default_rng(0) stream drawn in order.
* ``sweep``      bf16 4096x4096: Student-t (3 dof) * 0.02, then 0.1% of the
                 entries (16,777 positions, no repeats) multiplied by 20.
* ``llama7b``    bf16 N(0, 0.02^2): 32 layers of 4x(4096x4096), 2x(4096x11008),
                 1x(11008x4096), then the 32000x4096 embedding, back to back in
                 one flat buffer.  Drawn on the device with torch's seeded
                 generator (tensor i uses seed i) because 6.6G host draws take
                 minutes; the oracle reads back the groups it checks.
* ``matvec``     W = bf16(N(0, 0.02^2)) 11008x4096 from default_rng(0);
                 x = N(0, 1) fp32 [batch, 4096] from default_rng(1).

The Lloyd-Max training samples are 400,000 standard-normal draws from NumPy's
legacy ``RandomState(seed)`` generator, seed 0, as the codebook-training page
describes them.
"""

from __future__ import annotations

import numpy as np

LLOYD_SEED = 0
LLOYD_SAMPLES = 400_000


def lloyd_samples(seed: int = LLOYD_SEED, n: int = LLOYD_SAMPLES) -> np.ndarray:
    """Standard-normal training samples for the Lloyd-Max codebook."""
    return np.random.RandomState(seed).randn(n)


# ---------------------------------------------------------------------------
# dtype helpers (input preparation only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns.  NaN is not expected in these workloads."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 value (as float32)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

def small(seed: int = 0) -> np.ndarray:
    """fp32 256x512, N(0, 0.02^2)."""
    return (np.random.default_rng(seed).standard_normal((256, 512)) * 0.02).astype(np.float32)


def needle2_shapes() -> list[tuple[str, tuple[int, int]]]:
    """Tensor names and shapes of the 45.5M-parameter set plus the padding case."""
    out = [("embed", (8192, 512))]
    for layer in range(15):
        for name, shape in (("q", (512, 512)), ("k", (512, 128)), ("v", (512, 128)),
                            ("o", (512, 512)), ("up", (512, 2048)), ("down", (2048, 512))):
            out.append((f"l{layer}.{name}", shape))
    out.append(("pad", (300, 1000)))
    return out


def needle2(seed: int = 0) -> list[tuple[str, np.ndarray]]:
    """The 45.5M-parameter set, fp32 N(0, 0.02^2), one stream drawn in order."""
    rng = np.random.default_rng(seed)
    return [(name, (rng.standard_normal(shape) * 0.02).astype(np.float32))
            for name, shape in needle2_shapes()]


def sweep_bits(seed: int = 0, n: int = 4096) -> np.ndarray:
    """bf16 bit patterns of the n x n heavy-tailed matrix with 0.1% outliers."""
    rng = np.random.default_rng(seed)
    w = rng.standard_t(3, (n, n)) * 0.02
    count = (n * n) // 1000
    pos = rng.choice(n * n, count, replace=False)
    w.flat[pos] *= 20.0
    return f32_to_bf16_bits(w.astype(np.float32))


def llama7b_shapes() -> list[tuple[int, int]]:
    """Shapes of the 7B-parameter tensor list, in buffer order."""
    layer = [(4096, 4096)] * 4 + [(4096, 11008)] * 2 + [(11008, 4096)]
    return layer * 32 + [(32000, 4096)]


def llama7b_device(device="cuda", scale: float = 0.02):
    """Allocate and fill the flat bf16 7B-shaped buffer on the device.

    Returns (buffer, offsets) where offsets[i] is tensor i's element offset.
    Tensor i is drawn in float32 with a torch generator seeded with i, then
    rounded to bf16."""
    import torch

    shapes = llama7b_shapes()
    sizes = [r * c for r, c in shapes]
    offsets = np.concatenate(([0], np.cumsum(sizes)))
    buf = torch.empty(int(offsets[-1]), dtype=torch.bfloat16, device=device)
    gen = torch.Generator(device=device)
    for i, (r, c) in enumerate(shapes):
        gen.manual_seed(i)
        t = torch.randn((r, c), generator=gen, device=device, dtype=torch.float32)
        buf[int(offsets[i]):int(offsets[i + 1])].copy_(t.mul_(scale).view(-1))
        del t
    return buf, offsets


def matvec_weight_bits(seed: int = 0, n_out: int = 11008, k: int = 4096) -> np.ndarray:
    """bf16 bit patterns of the n_out x k matvec weight, N(0, 0.02^2)."""
    w = np.random.default_rng(seed).standard_normal((n_out, k)) * 0.02
    return f32_to_bf16_bits(w.astype(np.float32))


def matvec_x(batch: int, seed: int = 1, k: int = 4096) -> np.ndarray:
    """fp32 activations [batch, k], N(0, 1)."""
    return np.random.default_rng(seed).standard_normal((batch, k)).astype(np.float32)
