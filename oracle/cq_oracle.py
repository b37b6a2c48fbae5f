"""CPU oracle for the Cactus-Quants (CQ) rotated-codebook quantizer.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow reference the HIP
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU baseline legs of ``bench.py`` (``cpu_baseline``,
``cpu_baseline_configs``) may import it; the product path
(``rotated_codebook_bit_amd``) never does, and this module imports nothing from
the product path.  It shares no code, table or constant generator with the
HIP library.

Everything is computed in float64 NumPy, step by step in the order the pages
describe, with dense matrices where the pages use dense matrices.  Sources
(page title, then section):

* "Cactus Quants CQ2-bit Quantization: Extreme Compression for Edge LLMs"
  (called *CQ2 overview* below): §Group-wise Weight Partitioning,
  §Hadamard Rotation, §Optimized Codebook Design,
  §The CQ2-bit Implementation Pipeline.
* "How CQ2-bit Quantization Contributes to Needle 2's Small Footprint"
  (*Footprint*): §Hadamard Rotation, §Static Codebook Quantization,
  §Per-Group Storage Breakdown, §Binary Serialization.
* "Performance Differences Between 2-Bit and 4-Bit Quantization in Needle"
  (*2-bit vs 4-bit*): §Quantization Error and Accuracy Impact,
  §Practical Code Comparison.
* "How Quantization Codebooks Are Trained in Cactus Quants: Lloyd-Max on
  Gaussian Data" (*Codebook training*): §Gaussian Sampling and
  Initialization, §Iterative Refinement of Quantization Levels,
  §Ternary Special Case Handling, §Production Codebook Generation and Caching.

Where the pages are silent or ambiguous, the reading taken is stated next to
the code it affects.

Parity pins: every public function here is pinned by ``tests/test_oracle_*.py``
against closed forms, textbook values, brute force or hand-worked examples;
the tolerance helpers ``threshold_distance`` and ``admissible_indices`` by
hand-worked values on a codebook whose thresholds are exact
(``tests/test_oracle_band.py``); ``normalised_groups`` by the norm invariant,
an independent in-lane transform and an exact-cancellation example
(``tests/test_oracle_transform.py``, ``tests/test_oracle_quantize.py``).
"""

from __future__ import annotations

import math

import numpy as np

# Ternary case: the pages give the 3-level codebook explicitly instead of
# training it (*Codebook training*, §Ternary Special Case Handling).
TERNARY = 158  # bit-width code for the "1.58-bit" three-level codebook
TERNARY_TRITS = 159  # the same codebook stored five trits per byte
TERNARY_LEVELS = (-1.2240064, 0.0, 1.2240064)

GROUP = 128  # default group size (*CQ2 overview*, §Group-wise Weight Partitioning)
LLOYD_SAMPLES = 400_000  # (*Codebook training*, §Gaussian Sampling and Initialization)
LLOYD_ITERS = 200  # (*Codebook training*, §Iterative Refinement of Quantization Levels)


# ---------------------------------------------------------------------------
# Codebook
# ---------------------------------------------------------------------------

def n_levels(bits: int) -> int:
    """Number of codebook levels: 3 for the ternary code, else 2**bits."""
    if bits in (TERNARY, TERNARY_TRITS):
        return 3
    if bits not in (1, 2, 3, 4):
        raise ValueError(f"unsupported bit-width {bits}")
    return 1 << bits


def storage_bits(bits: int) -> int:
    """Bits stored per index.  The three ternary codes use a 2-bit field
    (reading: the pages describe no trit packing).  Trit storage has no bit
    fields (see :func:`pack_trits`)."""
    if bits == TERNARY_TRITS:
        raise ValueError("trit storage has no fixed-width fields")
    return 2 if bits == TERNARY else n_levels(bits).bit_length() - 1


def group_bytes(bits: int, g: int = GROUP) -> int:
    """Bytes of packed indices per group: g*sbits/8, or ceil(g/5) for trit
    storage (26 at g = 128, the 1.6-bit form of the "1.58-bit" ternary
    code; *Codebook training* §Ternary Special Case Handling)."""
    if bits == TERNARY_TRITS:
        return -(-g // 5)
    return g * storage_bits(bits) // 8


def lloyd_max(samples: np.ndarray, levels: int, iters: int = LLOYD_ITERS) -> np.ndarray:
    """1-D Lloyd-Max (k-means) on a sample set, as *Codebook training*
    §Gaussian Sampling and Initialization and §Iterative Refinement of
    Quantization Levels describe it.

    * The samples are sorted; the initial level k is the sample at the
      quantile position floor((k + 1/2) * n / L) of the sorted array.
    * Each iteration puts the decision boundaries at the midpoints of
      neighbouring levels, gives every sample to the cell whose lower
      boundary it strictly exceeds (a sample equal to a boundary stays in the
      lower cell), and moves every level to the mean of its cell.
    * A cell left empty keeps its previous level (reading: the pages do not
      say; it never happens for L <= 16 with this initialisation).
    * The levels are returned sorted ascending.
    """
    x = np.sort(np.asarray(samples, dtype=np.float64).ravel())
    n = x.size
    if n < levels:
        raise ValueError("need at least as many samples as levels")
    pos = ((2 * np.arange(levels, dtype=np.int64) + 1) * n) // (2 * levels)
    c = x[pos].copy()
    for _ in range(iters):
        edges = 0.5 * (c[:-1] + c[1:])
        # Cell k holds the sorted samples in [start[k], start[k+1]).  A sample
        # belongs to cell #{edges < sample}, so cell k starts after the last
        # sample that is <= edges[k-1].
        start = np.concatenate(([0], np.searchsorted(x, edges, side="right"), [n]))
        for k in range(levels):
            lo, hi = start[k], start[k + 1]
            if hi > lo:
                c[k] = x[lo:hi].mean()
    return np.sort(c)


def codebook(bits: int, samples: np.ndarray | None = None,
             iters: int = LLOYD_ITERS) -> np.ndarray:
    """Codebook levels in N(0,1) units (float64), before any group scaling.

    Ternary returns the fixed three levels; every other width runs
    :func:`lloyd_max` on ``samples`` (the caller draws them: the pages use
    400,000 standard-normal draws from a seeded generator).
    """
    if bits in (TERNARY, TERNARY_TRITS):
        return np.array(TERNARY_LEVELS, dtype=np.float64)
    if samples is None:
        raise ValueError("Lloyd-Max codebooks need the Gaussian samples")
    return lloyd_max(samples, n_levels(bits), iters)


def runtime_levels(levels: np.ndarray) -> np.ndarray:
    """The levels as the quantizer uses them at run time: rounded to float32
    (the pages turn the NumPy table into a device array, *Footprint*
    §Hadamard Rotation), returned as exact float64 copies of those floats."""
    return np.asarray(levels, dtype=np.float64).astype(np.float32).astype(np.float64)


def thresholds(levels32: np.ndarray) -> np.ndarray:
    """Decision thresholds: midpoints of neighbouring levels (*Codebook
    training* §Iterative Refinement).  Exact in float64 for float32 levels."""
    c = np.asarray(levels32, dtype=np.float64)
    return 0.5 * (c[:-1] + c[1:])


# ---------------------------------------------------------------------------
# Hadamard rotation
# ---------------------------------------------------------------------------

def sylvester(g: int) -> np.ndarray:
    """The +-1 Sylvester-Hadamard matrix of order g (a power of two), built by
    repeated Kronecker doubling [[H, H], [H, -H]]."""
    if g < 1 or g & (g - 1):
        raise ValueError("group size must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < g:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard(g: int) -> np.ndarray:
    """Orthonormal Walsh-Hadamard matrix H/sqrt(g) (*CQ2 overview* §Hadamard
    Rotation; *Footprint* §Hadamard Rotation).  Reading: Sylvester natural
    order.  It is symmetric and its own inverse."""
    return sylvester(g) / math.sqrt(g)


def normalised_groups(x: np.ndarray, g: int) -> tuple[np.ndarray, np.ndarray]:
    """Group norms n and normalised rotated values z = sqrt(g) * y / n of the
    rows of x, y = x H/sqrt(g) the orthonormal rotation (z = 0 for a zero
    group).

    Computed from the +-1 product hx = x H: y = hx / sqrt(g), so
    sqrt(g) * y = hx, ||y||^2 = sum(hx^2) / g and z = hx / n.  The +-1 sums
    of float32 or bf16 inputs are exact in float64, so a component that
    cancels exactly is exactly 0 and a tie at a threshold of 0 is decided by
    the tie rule (multiplying by the rounded entries 1/sqrt(g) first leaves
    ~1e-17 there, i.e. rounding noise decides); the division by g = 2^k is
    exact, so a norm that is a float64 number comes out exactly."""
    hx = np.asarray(x, dtype=np.float64) @ sylvester(g)
    n = np.sqrt(np.sum(hx * hx, axis=1) / g)
    z = np.zeros_like(hx)
    nz = n > 0
    z[nz] = hx[nz] / n[nz, None]
    return n, z


# ---------------------------------------------------------------------------
# Quantize / dequantize
# ---------------------------------------------------------------------------

def to_groups(w: np.ndarray, g: int = GROUP) -> tuple[np.ndarray, int, int]:
    """Zero-pad the last axis to a multiple of g and cut it into groups
    (*CQ2 overview* §The CQ2-bit Implementation Pipeline, step 1).

    Returns (X, R, D): X has shape (R * ceil(D/g), g) in row-major group
    order, R is the product of the leading dimensions, D the last dimension.
    """
    w = np.asarray(w, dtype=np.float64)
    if w.ndim == 0:
        raise ValueError("need at least one dimension")
    d = w.shape[-1]
    r = int(np.prod(w.shape[:-1], dtype=np.int64)) if w.ndim > 1 else 1
    w2 = w.reshape(r, d)
    ng = -(-d // g)
    padded = np.zeros((r, ng * g), dtype=np.float64)
    padded[:, :d] = w2
    return padded.reshape(r * ng, g), r, d


class Quantized:
    """Result of :func:`quantize` (all arrays in row-major group order).

    idx    int64  [R, ng, g]   codebook index per element
    z      f64    [R, ng, g]   normalised rotated value the index was chosen from
    norm   f64    [R, ng]      unrounded group L2 norm
    norm16 uint16 [R, ng]      IEEE binary16 bits of the stored norm
    """

    def __init__(self, idx, z, norm, norm16, rows, cols, bits, g, levels32):
        self.idx, self.z, self.norm, self.norm16 = idx, z, norm, norm16
        self.rows, self.cols, self.bits, self.g = rows, cols, bits, g
        self.levels32 = levels32

    @property
    def packed(self) -> np.ndarray:
        return pack_indices(self.idx, self.bits)


def fp16_bits(x: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit pattern of float64 values, round-to-nearest-even,
    converted directly from float64 (NumPy's double->half conversion)."""
    with np.errstate(over="ignore"):  # norms above 65504 store +Inf
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def quantize(w: np.ndarray, bits: int, levels: np.ndarray, g: int = GROUP) -> Quantized:
    """CQ quantize, following *CQ2 overview* §The CQ2-bit Implementation
    Pipeline (steps 1-4) and *Footprint* §Per-Group Storage Breakdown.

    1. pad the last axis with zeros to a multiple of g, cut into groups;
    2. rotate every group by the orthonormal Hadamard matrix (dense product;
       :func:`normalised_groups` does steps 2 and 3);
    3. take the group's L2 norm n and normalise: z = sqrt(g) * y / n
       (equivalently unit-norm components against levels / sqrt(g),
       *Codebook training* §Production Codebook Generation and Caching);
       a zero group gives z = 0 (reading: the pages do not say);
    4. index = number of thresholds strictly below z (nearest level; an exact
       tie goes to the lower level);
    5. store the index and the norm rounded to binary16.

    ``levels`` are in N(0,1) units; they are rounded to float32 first
    (:func:`runtime_levels`).
    """
    levels32 = runtime_levels(levels)
    if levels32.size != n_levels(bits):
        raise ValueError("codebook size does not match the bit-width")
    t = thresholds(levels32)
    x, r, d = to_groups(w, g)
    n, z = normalised_groups(x, g)
    idx = np.searchsorted(t, z, side="left").astype(np.int64)
    ng = x.shape[0] // r if r else 0
    shape3 = (r, ng, g)
    return Quantized(idx.reshape(shape3), z.reshape(shape3), n.reshape(r, ng),
                     fp16_bits(n).reshape(r, ng), r, d, bits, g, levels32)


def dequantize_groups(idx: np.ndarray, norm16: np.ndarray, levels: np.ndarray,
                      g: int = GROUP) -> np.ndarray:
    """Reconstructed groups (float64, shape [..., g]) from indices and stored
    binary16 norms: look up the float32 levels, scale by norm/sqrt(g), rotate
    back by the Hadamard matrix (*CQ2 overview* §The CQ2-bit Implementation
    Pipeline, steps 4-5)."""
    levels32 = runtime_levels(levels)
    idx = np.asarray(idx, dtype=np.int64)
    n = np.asarray(norm16, dtype=np.uint16).view(np.float16).astype(np.float64)
    q = levels32[idx] * (n[..., None] / math.sqrt(g))
    return q @ hadamard(g)


def dequantize(packed: np.ndarray, norm16: np.ndarray, rows: int, cols: int,
               bits: int, levels: np.ndarray, g: int = GROUP) -> np.ndarray:
    """Dequantize packed storage to a float64 [rows, cols] matrix; the pad
    columns are dropped (*CQ2 overview* §The CQ2-bit Implementation Pipeline,
    step 6)."""
    ng = -(-cols // g)
    idx = unpack_indices(packed, bits, g).reshape(rows, ng, g)
    xh = dequantize_groups(idx, np.asarray(norm16).reshape(rows, ng), levels, g)
    return xh.reshape(rows, ng * g)[:, :cols]


# ---------------------------------------------------------------------------
# Packing
# ---------------------------------------------------------------------------

def pack(idx: np.ndarray, sbits: int) -> np.ndarray:
    """Pack indices into bytes: within each group, index j occupies bits
    [sbits*j, sbits*j + sbits) of a little-endian bit stream (least
    significant bit first).  Reading of *Footprint* §Binary Serialization,
    which says only that consecutive weights are packed into bytes.

    idx has shape [..., g]; the result has shape [..., g * sbits / 8]."""
    idx = np.asarray(idx, dtype=np.int64)
    g = idx.shape[-1]
    if (g * sbits) % 8:
        raise ValueError("group does not fill whole bytes")
    bits = (idx[..., :, None] >> np.arange(sbits)) & 1  # [..., g, sbits]
    stream = bits.reshape(idx.shape[:-1] + (g * sbits,)).astype(np.uint8)
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack(packed: np.ndarray, sbits: int, g: int = GROUP) -> np.ndarray:
    """Inverse of :func:`pack`: bytes [..., g*sbits/8] -> indices [..., g]."""
    packed = np.asarray(packed, dtype=np.uint8)
    nbytes = g * sbits // 8
    flat = packed.reshape(-1, nbytes)
    stream = np.unpackbits(flat, axis=-1, bitorder="little").astype(np.int64)
    stream = stream.reshape(flat.shape[0], g, sbits)
    idx = np.sum(stream << np.arange(sbits), axis=-1)
    return idx.reshape(packed.shape[:-1] + (g,)) if packed.ndim > 1 else idx.reshape(g)


def pack_trits(idx: np.ndarray) -> np.ndarray:
    """Five ternary indices per byte, base 3, least significant digit first:
    within each group, index j is digit j % 5 of byte j // 5; the last byte
    holds the g mod 5 remaining indices (upper digits zero).  Reading: the
    pages name the 1.58-bit ternary code but no trit layout.  [..., g] ->
    [..., ceil(g/5)]."""
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size and (idx.min() < 0 or idx.max() > 2):
        raise ValueError("ternary indices are 0, 1 or 2")
    g = idx.shape[-1]
    nb = -(-g // 5)
    padded = np.zeros(idx.shape[:-1] + (nb * 5,), dtype=np.int64)
    padded[..., :g] = idx
    digits = padded.reshape(idx.shape[:-1] + (nb, 5))
    weights = 3 ** np.arange(5)
    return np.sum(digits * weights, axis=-1).astype(np.uint8)


def unpack_trits(packed: np.ndarray, g: int = GROUP) -> np.ndarray:
    """Inverse of :func:`pack_trits`: bytes [..., ceil(g/5)] -> indices [..., g]."""
    packed = np.asarray(packed, dtype=np.uint8)
    nb = -(-g // 5)
    flat = packed.reshape(-1, nb).astype(np.int64)
    digits = (flat[..., None] // (3 ** np.arange(5))) % 3
    idx = digits.reshape(flat.shape[0], nb * 5)[:, :g]
    return idx.reshape(packed.shape[:-1] + (g,)) if packed.ndim > 1 else idx.reshape(g)


def pack_indices(idx: np.ndarray, bits: int) -> np.ndarray:
    """Packed storage of indices for a bit-width code (bit fields, or trits)."""
    if bits == TERNARY_TRITS:
        return pack_trits(idx)
    return pack(idx, storage_bits(bits))


def unpack_indices(packed: np.ndarray, bits: int, g: int = GROUP) -> np.ndarray:
    """Inverse of :func:`pack_indices`."""
    if bits == TERNARY_TRITS:
        return unpack_trits(packed, g)
    return unpack(packed, storage_bits(bits), g)


# ---------------------------------------------------------------------------
# Dequantize-matvec
# ---------------------------------------------------------------------------

def matvec(packed: np.ndarray, norm16: np.ndarray, n_out: int, k: int, bits: int,
           levels: np.ndarray, x: np.ndarray, g: int = GROUP) -> np.ndarray:
    """y = x . W_hat^T in float64, with W_hat the dequantized [n_out, k]
    matrix (the forward product of *2-bit vs 4-bit* §Practical Code
    Comparison applied to quantized weights).  x is [batch, k]."""
    w_hat = dequantize(packed, norm16, n_out, k, bits, levels, g)
    return np.asarray(x, dtype=np.float64) @ w_hat.T


def matvec_rotated(packed: np.ndarray, norm16: np.ndarray, n_out: int, k: int,
                   bits: int, levels: np.ndarray, x: np.ndarray,
                   g: int = GROUP) -> np.ndarray:
    """Second route to the same product, used to check :func:`matvec`:
    because the orthonormal Hadamard matrix is symmetric and its own inverse,
    x_g . W_hat_g = (norm/sqrt(g)) * <x_g H, levels[idx]> for every group.
    Requires k to be a multiple of g."""
    if k % g:
        raise ValueError("k must be a multiple of the group size")
    ng = k // g
    levels32 = runtime_levels(levels)
    idx = unpack_indices(packed, bits, g).reshape(n_out, ng, g)
    n = np.asarray(norm16, dtype=np.uint16).reshape(n_out, ng).view(np.float16)
    q = levels32[idx] * (n.astype(np.float64)[..., None] / math.sqrt(g))
    xr = np.asarray(x, dtype=np.float64).reshape(-1, ng, g) @ hadamard(g)
    return np.einsum("bgj,rgj->br", xr, q)


# ---------------------------------------------------------------------------
# Size accounting and error reports
# ---------------------------------------------------------------------------

def model_bytes(shapes, bits: int, g: int = GROUP) -> int:
    """Storage size of a set of tensors: per group, g*sbits/8 bytes of packed
    indices plus one binary16 norm, nothing else (*Footprint* §Per-Group
    Storage Breakdown).  A tensor of shape (..., D) has prod(leading) *
    ceil(D/g) groups; padded groups count in full."""
    per_group = group_bytes(bits, g) + 2
    total = 0
    for shape in shapes:
        shape = tuple(int(s) for s in shape)
        d = shape[-1]
        r = int(np.prod(shape[:-1], dtype=np.int64)) if len(shape) > 1 else 1
        groups = r * (-(-d // g))
        total += groups * per_group
    return total


def serialize(quantized) -> np.ndarray:
    """Serialized weights of a sequence of quantized tensors, in the order of
    *Footprint* §Binary Serialization: the packed indices of every tensor,
    tensor after tensor, followed by every tensor's binary16 norms
    (little-endian), in the same tensor order.  No header (reading: the
    norms of all tensors follow all the indices).  Trit storage can leave the
    indices an odd number of bytes (7- or 13-byte groups at g = 32, 64); then
    one zero byte follows them, so the binary16 norms start at an even
    offset (reading: the pages give no trit layout at these group sizes)."""
    parts = [np.asarray(q.packed, dtype=np.uint8).ravel() for q in quantized]
    if sum(p.size for p in parts) % 2:
        parts.append(np.zeros(1, dtype=np.uint8))
    parts += [np.asarray(q.norm16, dtype=np.uint16).astype("<u2").view(np.uint8).ravel()
              for q in quantized]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.uint8)


def blob_offsets(shapes, bits: int, g: int = GROUP):
    """(packed_offsets, norm_offsets, total) of :func:`serialize`'s output for
    tensors of the given shapes: byte offsets of each tensor's indices and
    norms, and the total size (which equals :func:`model_bytes`, plus the pad
    byte after an odd-length index section)."""
    gb = group_bytes(bits, g)
    packed, norms = [], []
    for shape in shapes:
        shape = tuple(int(s) for s in shape)
        r = int(np.prod(shape[:-1], dtype=np.int64)) if len(shape) > 1 else 1
        groups = r * (-(-shape[-1] // g))
        packed.append(groups * gb)
        norms.append(groups * 2)
    p_off = [sum(packed[:i]) for i in range(len(packed))]
    n0 = sum(packed) + sum(packed) % 2
    n_off = [n0 + sum(norms[:i]) for i in range(len(norms))]
    return p_off, n_off, n0 + sum(norms)


def relative_mse(w: np.ndarray, w_hat: np.ndarray) -> float:
    """||W - W_hat||_F^2 / ||W||_F^2 (the distortion measure of *2-bit vs
    4-bit* §Quantization Error and Accuracy Impact, read as a mean-square
    ratio)."""
    w = np.asarray(w, dtype=np.float64)
    e = w - np.asarray(w_hat, dtype=np.float64)
    return float(np.sum(e * e) / np.sum(w * w))


def fake_quant(w: np.ndarray, bits: int, levels: np.ndarray, g: int = GROUP,
               rotate: bool = True) -> np.ndarray:
    """Quantize then reconstruct with the unrounded norm, as the pages'
    quantizer returns its result (*CQ2 overview* §The CQ2-bit Implementation
    Pipeline).  ``rotate=False`` replaces the Hadamard matrix by the identity
    (the no-rotation ablation used to show the rotation's effect)."""
    levels32 = runtime_levels(levels)
    t = thresholds(levels32)
    x, r, d = to_groups(w, g)
    h = hadamard(g) if rotate else np.eye(g)
    if rotate:
        n, z = normalised_groups(x, g)
    else:
        n = np.sqrt(np.sum(x * x, axis=1))
        z = np.zeros_like(x)
        nz = n > 0
        z[nz] = math.sqrt(g) * x[nz] / n[nz, None]
    idx = np.searchsorted(t, z, side="left")
    xh = (levels32[idx] * (n[:, None] / math.sqrt(g))) @ h.T
    ng = x.shape[0] // r
    return xh.reshape(r, ng * g)[:, :d].reshape(np.shape(w))


def threshold_distance(z: np.ndarray, levels: np.ndarray) -> np.ndarray:
    """Distance (z units) from each normalised value to its nearest decision
    threshold (the midpoints of *Codebook training* §Iterative Refinement),
    element by element, same shape as z."""
    t = thresholds(runtime_levels(levels))
    z = np.asarray(z, dtype=np.float64)
    return np.min(np.abs(z[..., None] - t), axis=-1)


def admissible_indices(z: np.ndarray, levels: np.ndarray, band: float):
    """Indices a quantizer may return for the normalised value z when its own
    value of z can be off by up to ``band`` (z units): every index the
    nearest-level rule gives to some z' in [z - band, z + band].  The rule is
    monotone in z', so these are the integers from the index of z - band to
    the index of z + band.  Returns (lo, hi), each shaped like z."""
    t = thresholds(runtime_levels(levels))
    z = np.asarray(z, dtype=np.float64)
    lo = np.searchsorted(t, z - band, side="left").astype(np.int64)
    hi = np.searchsorted(t, z + band, side="left").astype(np.int64)
    return lo, hi
