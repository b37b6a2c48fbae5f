"""Python binding of libcq, the CQ rotated-codebook quantizer for MI355X.

Thin ctypes marshalling over the C ABI declared in ``include/libcq.h``: the
names match the C entry points without the ``cq_`` prefix.  Every step of the
computation runs in libcq's HIP kernels; PyTorch only provides device memory
and the current stream.  There is no fallback: if ``libcq.so`` is missing or
a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "TERNARY", "TERNARY_TRITS", "GROUP", "group_bytes", "repack", "CQError", "lib", "storage_bits", "n_levels", "layout",
    "model_bytes", "codebook", "codebook_train", "quantize", "dequantize", "dequant_matvec", "dequant_matvec_many",
    "dequant_matvec_many_noalloc",
    "fake_quant", "blob_layout", "quantize_many", "dequantize_many", "dequant_gemm",
    "dequant_gemm_many",
]

TERNARY = 158
TERNARY_TRITS = 159  # the ternary code stored five indices per byte
GROUP = 128
F32, BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcq.so")
_lib = None


class CQError(RuntimeError):
    """A libcq call returned an error status."""

    def __init__(self, func: str, status: int, detail: str):
        super().__init__(f"{func}: {detail} (status {status})")
        self.status = status


class QuantDesc(ctypes.Structure):
    """cq_quant_desc: one tensor of cq_quantize_many."""
    _fields_ = [("w", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("packed", ctypes.c_void_p), ("norms", ctypes.c_void_p)]


class DequantDesc(ctypes.Structure):
    """cq_dequant_desc: one tensor of cq_dequantize_many."""
    _fields_ = [("packed", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("out", ctypes.c_void_p)]


class MatvecDesc(ctypes.Structure):
    """cq_matvec_desc: one matrix of cq_dequant_matvec_many."""
    _fields_ = [("packed", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("n_out", ctypes.c_int64),
                ("k", ctypes.c_int64), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    """Load libcq.so (built in place by ``rotated_codebook_bit_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m rotated_codebook_bit_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.cq_layout.argtypes = [i64, i64, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.cq_model_bytes.argtypes = [i32, ctypes.POINTER(i64), ctypes.POINTER(i64), i32, i32,
                                     ctypes.POINTER(ctypes.c_uint64)]
        L.cq_codebook.argtypes = [i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
        L.cq_codebook_train.argtypes = [i32, ctypes.POINTER(ctypes.c_double), i64, i32,
                                        ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
        L.cq_quantize.argtypes = [vp, i32, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_float), i32,
                                  vp, vp, vp]
        L.cq_dequantize.argtypes = [vp, vp, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_float), i32,
                                    vp, i32, vp]
        L.cq_blob_layout.argtypes = [i32, ctypes.POINTER(i64), ctypes.POINTER(i64), i32, i32,
                                     ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.cq_quantize_many.argtypes = [i32, ctypes.POINTER(QuantDesc), i32, i32, i32,
                                       ctypes.POINTER(ctypes.c_float), i32, vp]
        L.cq_dequantize_many.argtypes = [i32, ctypes.POINTER(DequantDesc), i32, i32,
                                         ctypes.POINTER(ctypes.c_float), i32, i32, vp]
        L.cq_dequant_gemm.argtypes = [vp, vp, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_float),
                                      i32, vp, i64, vp, vp]
        L.cq_dequant_gemm_many.argtypes = [i32, ctypes.POINTER(MatvecDesc), i32, i32,
                                           ctypes.POINTER(ctypes.c_float), i32, i64, vp]
        L.cq_repack.argtypes = [vp, i32, vp, i32, i64, i32, vp]
        L.cq_fake_quant.argtypes = [vp, i32, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_float), i32,
                                    vp, i32, vp]
        L.cq_dequant_matvec.argtypes = [vp, vp, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_float),
                                        i32, vp, i64, vp, vp]
        L.cq_dequant_matvec_many.argtypes = [i32, ctypes.POINTER(MatvecDesc), i32, i32,
                                             ctypes.POINTER(ctypes.c_float), i32, i64, vp]
        L.cq_dequant_matvec_many_noalloc.argtypes = L.cq_dequant_matvec_many.argtypes
        for name in ("cq_layout", "cq_model_bytes", "cq_codebook", "cq_codebook_train", "cq_quantize", "cq_dequantize",
                     "cq_fake_quant", "cq_dequant_matvec", "cq_dequant_matvec_many",
                     "cq_dequant_matvec_many_noalloc", "cq_blob_layout",
                     "cq_quantize_many", "cq_dequantize_many", "cq_dequant_gemm",
                     "cq_dequant_gemm_many", "cq_repack"):
            getattr(L, name).restype = i32
        L.cq_status_str.argtypes = [i32]
        L.cq_status_str.restype = ctypes.c_char_p
        L.cq_last_error.argtypes = []
        L.cq_last_error.restype = ctypes.c_char_p
        L.cq_version.argtypes = []
        L.cq_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(func: str, status: int) -> None:
    if status != 0:
        L = lib()
        detail = L.cq_last_error().decode() or L.cq_status_str(status).decode()
        raise CQError(func, status, detail)


def storage_bits(bits: int) -> int:
    return 2 if bits in (TERNARY, TERNARY_TRITS) else int(bits)


def group_bytes(bits: int, group_size: int = GROUP) -> int:
    """Packed bytes per group (ceil(G/5) for trit storage)."""
    if bits == TERNARY_TRITS:
        return -(-group_size // 5)
    return group_size * storage_bits(bits) // 8


def n_levels(bits: int) -> int:
    return 3 if bits in (TERNARY, TERNARY_TRITS) else 1 << int(bits)


def _levels_arg(levels) -> tuple[np.ndarray | None, ctypes.POINTER(ctypes.c_float)]:
    """(kept-alive array, pointer) for a levels argument; None passes NULL,
    which selects the library's built-in table."""
    if levels is None:
        return None, ctypes.POINTER(ctypes.c_float)()
    arr = np.ascontiguousarray(np.asarray(levels, dtype=np.float32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _nlev(arr) -> int:
    return 0 if arr is None else int(arr.size)


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


# -- host-only calls ------------------------------------------------------------

def layout(rows: int, cols: int, bits: int, group_size: int = GROUP) -> tuple[int, int]:
    """(n_groups, packed_bytes) of a rows x cols tensor."""
    ng, pb = ctypes.c_int64(), ctypes.c_int64()
    _check("cq_layout", lib().cq_layout(rows, cols, bits, group_size, ctypes.byref(ng),
                                        ctypes.byref(pb)))
    return ng.value, pb.value


def model_bytes(shapes, bits: int, group_size: int = GROUP) -> int:
    """Storage bytes of a list of tensor shapes (last axis is the grouped one)."""
    rows, cols = [], []
    for shape in shapes:
        shape = tuple(int(s) for s in shape)
        cols.append(shape[-1])
        rows.append(int(np.prod(shape[:-1], dtype=np.int64)) if len(shape) > 1 else 1)
    n = len(rows)
    r = (ctypes.c_int64 * max(n, 1))(*rows)
    c = (ctypes.c_int64 * max(n, 1))(*cols)
    out = ctypes.c_uint64()
    _check("cq_model_bytes", lib().cq_model_bytes(n, r, c, bits, group_size, ctypes.byref(out)))
    return out.value


def codebook(bits: int) -> np.ndarray:
    """The built-in float32 codebook of a width (N(0,1) units): the table
    every call uses when its levels argument is None."""
    out = (ctypes.c_float * 16)()
    n = ctypes.c_int()
    _check("cq_codebook", lib().cq_codebook(bits, out, ctypes.byref(n)))
    return np.array(out[:n.value], dtype=np.float32)


def codebook_train(bits: int, samples, iters: int = 200) -> np.ndarray:
    """float32 Lloyd-Max codebook (N(0,1) units) trained by the library on the
    given float64 samples."""
    s = np.ascontiguousarray(np.zeros(0) if samples is None else samples, dtype=np.float64)
    out = (ctypes.c_float * 16)()
    n = ctypes.c_int()
    _check("cq_codebook_train", lib().cq_codebook_train(
        bits, s.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), s.size, iters, out, ctypes.byref(n)))
    return np.array(out[:n.value], dtype=np.float32)


# -- device calls ---------------------------------------------------------------

def _rows_cols(shape) -> tuple[int, int]:
    rows = 1
    for d in shape[:-1]:
        rows *= int(d)
    return rows, int(shape[-1])


def _desc_array(cls, columns):
    """A ctypes array of the descriptor struct `cls`, field i taken from the
    sequence columns[i].  It is filled through a NumPy record array of the
    same layout (every field is 8 bytes), one vectorised assignment per field
    instead of one ctypes construction per element."""
    n = len(columns[0])
    dt = np.dtype([(name, "<u8" if typ is ctypes.c_void_p else "<i8") for name, typ in cls._fields_])
    assert dt.itemsize == ctypes.sizeof(cls)
    rec = np.zeros(max(n, 1), dt)
    if n:
        for (name, _), col in zip(cls._fields_, columns):
            rec[name] = col
    return (cls * max(n, 1)).from_buffer(rec)


def _ptr_or_0(t) -> int:
    return t.data_ptr() if t.numel() else 0


def quantize(w, bits: int, levels, group_size: int = GROUP, packed=None, norms=None, stream=None):
    """Quantize a CUDA tensor (float32 or bfloat16, any rank; the last axis is
    grouped).  Returns (packed uint8 [rows, ngroups, G*sbits/8],
    norms float16 [rows, ngroups]) on w's device."""
    import torch
    if w.dtype == torch.float32:
        dt = F32
    elif w.dtype == torch.bfloat16:
        dt = BF16
    else:
        raise TypeError(f"unsupported dtype {w.dtype}")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    rows, cols = _rows_cols(w.shape)
    ng = -(-cols // group_size) if cols else 0
    pb = group_bytes(bits, group_size)
    if packed is None:
        packed = torch.empty((rows, ng, pb), dtype=torch.uint8, device=w.device)
    if norms is None:
        norms = torch.empty((rows, ng), dtype=torch.float16, device=w.device)
    lv, lvp = _levels_arg(levels)
    _check("cq_quantize", lib().cq_quantize(_ptr(w), dt, rows, cols, bits, group_size, lvp, _nlev(lv),
                                            _ptr(packed), _ptr(norms), _stream_ptr(stream)))
    return packed, norms


def dequantize(packed, norms, rows: int, cols: int, bits: int, levels, out_dtype=None,
               group_size: int = GROUP, out=None, stream=None):
    """Dequantize to a [rows, cols] CUDA tensor (float32 by default, or
    bfloat16)."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    dt = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    if out is None:
        out = torch.empty((rows, cols), dtype=out_dtype, device=packed.device)
    lv, lvp = _levels_arg(levels)
    _check("cq_dequantize", lib().cq_dequantize(_ptr(packed), _ptr(norms), rows, cols, bits,
                                                group_size, lvp, _nlev(lv), _ptr(out), dt,
                                                _stream_ptr(stream)))
    return out


def fake_quant(w, bits: int, levels, out_dtype=None, group_size: int = GROUP, out=None,
               stream=None):
    """Quantize and reconstruct a CUDA tensor in one pass (float32 or
    bfloat16 in, float32 or bfloat16 out, w's shape; default out dtype = w's).
    ``out=w`` fake-quantizes in place."""
    import torch
    dts = {torch.float32: F32, torch.bfloat16: BF16}
    if w.dtype not in dts:
        raise TypeError(f"unsupported dtype {w.dtype}")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    if out is None:
        out = torch.empty(w.shape, dtype=w.dtype if out_dtype is None else out_dtype, device=w.device)
    if out.dtype not in dts or not out.is_contiguous() or out.numel() != w.numel():
        raise ValueError("out must be a contiguous float32/bfloat16 tensor of w's size")
    rows, cols = _rows_cols(w.shape)
    lv, lvp = _levels_arg(levels)
    _check("cq_fake_quant", lib().cq_fake_quant(_ptr(w), dts[w.dtype], rows, cols, bits, group_size,
                                                lvp, _nlev(lv), _ptr(out), dts[out.dtype],
                                                _stream_ptr(stream)))
    return out


def dequant_matvec(packed, norms, n_out: int, k: int, bits: int, levels, x, group_size: int = GROUP,
                   y=None, stream=None):
    """y = x . W_hat^T with W the quantized n_out x k matrix; x float32
    [batch, k] on the device.  Returns float32 [batch, n_out]."""
    import torch
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 tensor")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [batch, {k}], got {tuple(x.shape)}")
    x2 = x
    batch = x2.shape[0]
    if y is None:
        y = torch.empty((batch, n_out), dtype=torch.float32, device=x.device)
    lv, lvp = _levels_arg(levels)
    _check("cq_dequant_matvec", lib().cq_dequant_matvec(_ptr(packed), _ptr(norms), n_out, k, bits,
                                                        group_size, lvp, _nlev(lv), _ptr(x2), batch,
                                                        _ptr(y), _stream_ptr(stream)))
    return y


def _matvec_descs(items):
    return _desc_array(MatvecDesc, (
        [_ptr_or_0(it[0]) for it in items], [_ptr_or_0(it[1]) for it in items],
        [it[2] for it in items], [it[3] for it in items],
        [_ptr_or_0(it[4]) for it in items], [_ptr_or_0(it[5]) for it in items]))


def dequant_matvec_many(items, bits: int, levels, batch: int, group_size: int = GROUP, stream=None):
    """Run y = x . W_hat^T for every (packed, norms, n_out, k, x, y) in items
    as one call (the y tensors, float32 [batch, n_out], are written in place).
    Returns the list of y tensors."""
    n = len(items)
    arr = _matvec_descs(items)
    lv, lvp = _levels_arg(levels)
    _check("cq_dequant_matvec_many", lib().cq_dequant_matvec_many(n, arr, bits, group_size, lvp, _nlev(lv),
                                                                  batch, _stream_ptr(stream)))
    return [it[5] for it in items]


def dequant_matvec_many_noalloc(items, bits: int, levels, batch: int, group_size: int = GROUP, stream=None):
    """dequant_matvec_many with the library's fixed 16 MiB workspace instead of
    memory allocated per call (cq_dequant_matvec_many_noalloc).  Calls that
    overlap on one GPU race on that workspace."""
    n = len(items)
    arr = _matvec_descs(items)
    lv, lvp = _levels_arg(levels)
    _check("cq_dequant_matvec_many_noalloc",
           lib().cq_dequant_matvec_many_noalloc(n, arr, bits, group_size, lvp, _nlev(lv), batch,
                                                _stream_ptr(stream)))
    return [it[5] for it in items]


def blob_layout(shapes, bits: int, group_size: int = GROUP):
    """Offsets of the serialized form (all packed indices, then all norms) of
    tensors with the given shapes: (packed_offsets, norm_offsets, total)."""
    dims = [_rows_cols(tuple(sh)) for sh in shapes]
    n = len(dims)
    rc = np.zeros((2, max(n, 1)), np.int64)
    if n:
        rc[:, :n] = np.array(dims, np.int64).T
    out = np.zeros((2, max(n, 1)), np.int64)
    p64 = ctypes.POINTER(ctypes.c_int64)
    total = ctypes.c_int64()
    _check("cq_blob_layout", lib().cq_blob_layout(n, rc[0].ctypes.data_as(p64), rc[1].ctypes.data_as(p64), bits,
                                                  group_size, out[0].ctypes.data_as(p64),
                                                  out[1].ctypes.data_as(p64), ctypes.byref(total)))
    return out[0, :n].tolist(), out[1, :n].tolist(), total.value


def quantize_many(ws, bits: int, levels, blob=None, group_size: int = GROUP, stream=None,
                  views: bool = True):
    """Quantize a list of CUDA tensors (all float32 or all bfloat16) in one
    call, writing the serialized blob (uint8, all packed indices then all
    norms).  Returns (blob, [(packed [rows, ng, G*sbits/8], norms float16
    [rows, ng]) views into the blob, one per tensor]); with views=False the
    list is empty (blob_layout gives the offsets)."""
    import torch
    if not ws:
        return torch.zeros(0, dtype=torch.uint8), []
    dt = {torch.float32: F32, torch.bfloat16: BF16}.get(ws[0].dtype)
    if dt is None or any(w.dtype != ws[0].dtype for w in ws):
        raise TypeError("all tensors must be float32, or all bfloat16")
    if any(not w.is_contiguous() for w in ws):
        raise ValueError("tensors must be contiguous")
    po, no, total = blob_layout([tuple(w.shape) for w in ws], bits, group_size)
    if blob is None:
        blob = torch.empty(total, dtype=torch.uint8, device=ws[0].device)
        # An odd-length index section is followed by a pad byte the library
        # does not write: zero it, so the blob is fully defined.
        packed_end = group_bytes(bits, group_size) * sum(
            r * -(-c // group_size) for r, c in (_rows_cols(tuple(w.shape)) for w in ws))
        if packed_end % 2:
            blob[packed_end:packed_end + 1].zero_()
    if blob.dtype != torch.uint8 or blob.numel() != total or not blob.is_contiguous():
        raise ValueError(f"blob must be a contiguous uint8 tensor of {total} bytes")
    pb = group_bytes(bits, group_size)
    base = blob.data_ptr() if total else 0
    dims = [_rows_cols(tuple(w.shape)) for w in ws]
    live = [r * c != 0 for r, c in dims]
    arr = _desc_array(QuantDesc, (
        [w.data_ptr() if a else 0 for w, a in zip(ws, live)], [r for r, _ in dims], [c for _, c in dims],
        [base + o if a else 0 for o, a in zip(po, live)], [base + o if a else 0 for o, a in zip(no, live)]))
    out_views = []
    if views:
        for i, (rows, cols) in enumerate(dims):
            ng = -(-cols // group_size) if cols else 0
            pk = blob[po[i]:po[i] + rows * ng * pb].view(rows, ng, pb)
            nm = blob[no[i]:no[i] + 2 * rows * ng].view(torch.float16).view(rows, ng)
            out_views.append((pk, nm))
    lv, lvp = _levels_arg(levels)
    _check("cq_quantize_many", lib().cq_quantize_many(len(ws), arr, dt, bits, group_size, lvp, _nlev(lv),
                                                      _stream_ptr(stream)))
    return blob, out_views


def dequantize_many(items, bits: int, levels, out_dtype=None, outs=None, group_size: int = GROUP,
                    stream=None):
    """Dequantize every (packed, norms, rows, cols) of items in one call.
    Returns the list of [rows, cols] outputs (float32 by default, or
    bfloat16; ``outs`` supplies them)."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    dt = {torch.float32: F32, torch.bfloat16: BF16}[out_dtype]
    if outs is None:
        dev = items[0][0].device if items else "cpu"
        outs = [torch.empty((r, c), dtype=out_dtype, device=dev) for _, _, r, c in items]
    for i, ((_, _, rows, cols), out) in enumerate(zip(items, outs)):
        if out.dtype != out_dtype or out.numel() != rows * cols or not out.is_contiguous():
            raise ValueError(f"outs[{i}] must be a contiguous {out_dtype} tensor of {rows}x{cols}")
    arr = _desc_array(DequantDesc, (
        [_ptr_or_0(it[0]) for it in items], [_ptr_or_0(it[1]) for it in items], [it[2] for it in items],
        [it[3] for it in items], [_ptr_or_0(o) for o in outs]))
    lv, lvp = _levels_arg(levels)
    _check("cq_dequantize_many", lib().cq_dequantize_many(len(items), arr, bits, group_size, lvp,
                                                          _nlev(lv), dt, _stream_ptr(stream)))
    return outs


def dequant_gemm(packed, norms, n_out: int, k: int, bits: int, levels, x, group_size: int = GROUP,
                 y=None, stream=None):
    """y = x . W_hat^T on the matrix cores (split-bf16 MFMA, see
    cq_dequant_gemm); x float32 [batch, k].  Returns float32 [batch, n_out]."""
    import torch
    if x.dtype != torch.float32 or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 tensor")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [batch, {k}], got {tuple(x.shape)}")
    batch = x.shape[0]
    if y is None:
        y = torch.empty((batch, n_out), dtype=torch.float32, device=x.device)
    lv, lvp = _levels_arg(levels)
    _check("cq_dequant_gemm", lib().cq_dequant_gemm(_ptr(packed), _ptr(norms), n_out, k, bits, group_size,
                                                    lvp, _nlev(lv), _ptr(x), batch, _ptr(y),
                                                    _stream_ptr(stream)))
    return y


def dequant_gemm_many(items, bits: int, levels, batch: int, group_size: int = GROUP, stream=None):
    """dequant_gemm for every (packed, norms, n_out, k, x, y) in items as one
    call (y float32 [batch, n_out] written in place).  Returns the y list."""
    n = len(items)
    arr = _matvec_descs(items)
    lv, lvp = _levels_arg(levels)
    _check("cq_dequant_gemm_many", lib().cq_dequant_gemm_many(n, arr, bits, group_size, lvp, _nlev(lv), batch,
                                                              _stream_ptr(stream)))
    return [it[5] for it in items]


def repack(src, src_bits: int, dst_bits: int, dst=None, group_size: int = GROUP, stream=None):
    """Convert packed ternary indices between 2-bit fields (TERNARY) and trit
    storage (TERNARY_TRITS).  src: uint8 CUDA tensor whose last dimension is
    one group's bytes ([..., 32] or [..., 26]).  Returns dst ([..., 26] or
    [..., 32])."""
    import torch
    sb, db = group_bytes(src_bits, group_size), group_bytes(dst_bits, group_size)
    if src.dtype != torch.uint8 or src.shape[-1] != sb or not src.is_contiguous():
        raise ValueError(f"src must be a contiguous uint8 tensor [..., {sb}]")
    n_groups = src.numel() // sb
    if dst is None:
        dst = torch.empty(tuple(src.shape[:-1]) + (db,), dtype=torch.uint8, device=src.device)
    _check("cq_repack", lib().cq_repack(_ptr(src), src_bits, _ptr(dst), dst_bits, n_groups, group_size,
                                        _stream_ptr(stream)))
    return dst
