"""Comparison rules between libcq (GPU) results and the oracle.

* Indices: bit-exact, except elements whose normalised value lies within
  BAND = 1e-5 (z units, oracle float64) of a decision threshold; there the
  index on the far side of that threshold is also correct (any index the
  nearest-level rule gives to a value within BAND of the oracle's z).  Such
  mismatches are counted and must number at most MAX_FRAC = 1e-6 of the
  elements checked.
* Norms (binary16): bit-exact, except where the oracle's float64 norm lies
  within 1e-6 relative of a binary16 rounding midpoint; there either
  neighbour is correct (the GPU rounds its float32 norm).
* Dequantized values: |x_gpu - x_ref| <= 1e-5 * RMS_g per element, with
  RMS_g = norm16 / sqrt(G) of the element's group.
* Matvec: |y_gpu - y_ref| <= 1e-5 * ||x_b|| * ||W_hat_r|| per element.
* Dequant-GEMM (split-bf16 MFMA): |y_gpu - y_ref| <= 5e-5 * ||x_b|| * ||W_hat_n||.
  Derived from its arithmetic: every operand v is taken as hi + lo with
  hi = bf16(v), lo = bf16(v - hi), so |v - hi - lo| <= 2^-16 |v|; the product
  drops lo*lo (<= 2^-16 relative) and carries both operands' split errors,
  <= 3 * 2^-16 = 4.6e-5 relative per product; summed with Cauchy-Schwarz over
  the groups (scaled by norm/G) this is <= 4.6e-5 * ||x_b|| * ||W_hat_n||.
* Fake quantization: the GPU's indices are read back from its output
  (H x_hat * sqrt(G) / n recovers levels[idx] for full groups) and checked
  under the index rule; values |x_gpu - x_ref| <= 1e-5 * n / sqrt(G) per
  element, plus (n / G) * (largest level gap) for each in-band element of the
  group (one flipped index moves every element of its group by exactly
  (n / G) * gap), plus one bf16 rounding for bf16 output.

The oracle is only ever given inputs that came from the seeded generators or
from the oracle itself, never from the GPU.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import cq_oracle as O

BAND = 1e-5
MAX_FRAC = 1e-6
NORM_REL = 1e-6
DEQ_TOL = 1e-5
MV_TOL = 1e-5
GEMM_TOL = 5e-5


class Report(dict):
    def line(self) -> str:
        return " ".join(f"{k}={v}" for k, v in self.items())


def _fp16_value(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def check_indices(idx_gpu: np.ndarray, q: O.Quantized, enforce_count: bool = True) -> Report:
    """Every mismatch must be admissible (check_admissible); with
    enforce_count the number of mismatches is capped here, else the caller
    applies the cap to a whole workload (see check_count)."""
    idx_gpu = np.asarray(idx_gpu).reshape(q.idx.shape)
    mism = idx_gpu != q.idx
    n = int(mism.sum())
    total = q.idx.size
    rep = Report(elements=total, index_mismatches=n)
    if n:
        check_admissible(idx_gpu[mism], q.z[mism], q.levels32)
        rep["max_band_dist"] = float(O.threshold_distance(q.z[mism], q.levels32).max())
    if enforce_count:
        check_count(n, total)
    return rep


def check_admissible(idx_gpu: np.ndarray, z: np.ndarray, levels32: np.ndarray) -> None:
    """Every GPU index must be one the nearest-level rule gives to some value
    within BAND of the oracle's z: near a threshold, the oracle's index or
    the one on the far side of that threshold, nothing else."""
    lo, hi = O.admissible_indices(z, levels32, BAND)
    ok = (idx_gpu >= lo) & (idx_gpu <= hi)
    if not ok.all():
        dist = O.threshold_distance(z[~ok], levels32)
        raise AssertionError(f"{int((~ok).sum())} index mismatches not admissible within the band "
                             f"(nearest threshold at {dist.min():.3g} .. {dist.max():.3g})")


def check_count(mismatches: int, elements: int) -> None:
    allowed = math.floor(MAX_FRAC * elements)
    assert mismatches <= allowed, (f"{mismatches} in-band mismatches > {allowed} allowed "
                                   f"({MAX_FRAC:g} of {elements})")


def check_norms(norm16_gpu: np.ndarray, q: O.Quantized) -> Report:
    g = np.asarray(norm16_gpu).view(np.uint16).reshape(q.norm16.shape)
    diff = g != q.norm16
    n = int(diff.sum())
    rep = Report(groups=q.norm16.size, norm_mismatches=n)
    if n:
        ref = q.norm[diff]
        a = _fp16_value(g[diff])
        b = _fp16_value(q.norm16[diff])
        # The two values must be binary16 neighbours and the exact norm must
        # sit within NORM_REL of their midpoint.
        step = np.abs(g[diff].astype(np.int64) - q.norm16[diff].astype(np.int64))
        assert np.all(step == 1), "norms differ by more than one binary16 step"
        mid = 0.5 * (a + b)
        assert np.all(np.abs(ref - mid) <= NORM_REL * ref), "norm mismatch away from a rounding midpoint"
    return rep


def check_quantize(packed_gpu: np.ndarray, norms_gpu: np.ndarray, q: O.Quantized,
                   enforce_count: bool = True) -> Report:
    gb = O.group_bytes(q.bits, q.g)
    idx = O.unpack_indices(np.asarray(packed_gpu).reshape(-1, gb), q.bits, q.g)
    rep = check_indices(idx, q, enforce_count)
    rep.update(check_norms(norms_gpu, q))
    return rep


def check_dequant(out_gpu: np.ndarray, ref: np.ndarray, norm16: np.ndarray, rows: int, cols: int,
                  g: int = O.GROUP) -> Report:
    """out_gpu and ref are [rows, cols]; norm16 [rows, ceil(cols/g)]."""
    out = np.asarray(out_gpu, dtype=np.float64).reshape(rows, cols)
    ng = -(-cols // g)
    rms = _fp16_value(norm16).reshape(rows, ng) / math.sqrt(g)
    tol = np.repeat(rms, g, axis=1)[:, :cols] * DEQ_TOL
    err = np.abs(out - ref)
    bad = err > tol
    assert not bad.any(), (f"{int(bad.sum())} dequantized values off by more than 1e-5 RMS; worst "
                           f"{float((err / np.maximum(tol / DEQ_TOL, 1e-300)).max()):.3g} RMS")
    scaled = err / np.where(tol > 0, tol / DEQ_TOL, 1.0)
    return Report(values=out.size, max_err_rms=float(scaled.max()) if out.size else 0.0)


def check_matvec(y_gpu: np.ndarray, y_ref: np.ndarray, x: np.ndarray, w_hat: np.ndarray,
                 tol: float = MV_TOL) -> Report:
    x = np.asarray(x, dtype=np.float64)
    scale = np.linalg.norm(x, axis=1)[:, None] * np.linalg.norm(w_hat, axis=1)[None, :]
    err = np.abs(np.asarray(y_gpu, dtype=np.float64) - y_ref)
    rel = err / np.where(scale > 0, scale, 1.0)
    assert np.all(err <= tol * scale), f"product error {rel.max():.3g} of ||x|| ||w|| > {tol:g}"
    return Report(outputs=err.size, max_err_scaled=float(rel.max()))


def check_fake_quant(out_gpu: np.ndarray, w64: np.ndarray, bits: int, levels: np.ndarray,
                     out_bf16: bool = False, enforce_count: bool = True, g: int = O.GROUP) -> Report:
    """out_gpu: the GPU reconstruction of w64 (any shape, w64's size)."""
    w2 = np.asarray(w64, dtype=np.float64).reshape(-1, np.shape(w64)[-1])
    rows, cols = w2.shape
    ng = -(-cols // g)
    ref = O.fake_quant(w2, bits, levels, g)
    q = O.quantize(w2, bits, levels, g)
    lv32 = O.runtime_levels(levels)
    out = np.asarray(out_gpu, dtype=np.float64).reshape(rows, cols)
    n = q.norm
    inband = (O.threshold_distance(q.z, lv32) <= BAND).sum(-1)
    gap = float(np.max(np.diff(lv32)))

    def by_group(a):
        full = np.zeros((rows, ng * g))
        full[:, :cols] = a
        return full.reshape(rows, ng, g)

    err = by_group(np.abs(out - ref)).max(-1)
    tol = DEQ_TOL * n / math.sqrt(g) + inband * (n / g) * gap
    if out_bf16:
        tol = tol * (1 + 2.0 ** -8) + 2.0 ** -8 * by_group(np.abs(ref)).max(-1)
    bad = err > tol
    assert not bad.any(), (f"{int(bad.sum())} groups off by more than the bound; worst "
                           f"{float((err / np.maximum(tol, 1e-300)).max()):.3g}x")
    zero = n == 0
    assert not by_group(out)[zero].any(), "a zero group must reconstruct to zeros"
    rep = Report(values=out.size, groups_with_band=int((inband > 0).sum()))

    nfull = ng if cols % g == 0 else ng - 1
    if nfull > 0:
        xg = out[:, :nfull * g].reshape(rows, nfull, g)
        nn = n[:, :nfull]
        c_hat = (xg @ O.hadamard(g)) * (math.sqrt(g) / np.where(nn > 0, nn, 1.0))[..., None]
        idx_ref = q.idx[:, :nfull]
        idx_gpu = np.argmin(np.abs(c_hat[..., None] - lv32), axis=-1)
        idx_gpu[zero[:, :nfull]] = idx_ref[zero[:, :nfull]]
        mism = idx_gpu != idx_ref
        m = int(mism.sum())
        if m:
            check_admissible(idx_gpu[mism], q.z[:, :nfull][mism], lv32)
        rep["index_mismatches"] = m
        rep["indices_read_back"] = int(idx_ref.size)
        if enforce_count:
            check_count(m, idx_ref.size)
    return rep
