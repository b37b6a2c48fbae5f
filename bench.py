"""Benchmark of the CQ hot path on one MI355X.

One step is one pass of the whole path over the 7B-shaped model (bf16,
6,607,077,376 parameters in one flat device buffer, 2-bit codebook, G=128):

  1. quantize the whole model in one launch (bf16 -> packed 2-bit + fp16 norms);
  2. dequantize the whole model in one launch (-> float32);
  3. dequant-matvec at batch 1 through every packed matrix (one
     cq_dequant_matvec_many call over the 225 matrices: one rotation launch,
     one product launch).

Extra phases after the step (in `phases`, not part of it): fused fake
quantization, the batch-256 dequant-GEMM, quantize as 225 calls and as one
multi-tensor call, the 11008x4096 product at batch 1 and 8 (one
cq_dequant_matvec call each, warm and cold, fraction of the binding roof),
and the 92-tensor Needle-2-sized set through cq_quantize_many and
cq_dequantize_many (warm and cold).

Prints one JSON line.  `value` is model parameters per second over the whole
step (wall clock, inputs resident in HBM).  Per-kernel times come from HIP
events recorded on the stream the kernels run on.  The CPU oracle is timed on
a bounded sample (one transformer layer and the embedding, 333M params,
through the same three steps).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
       python bench.py --copy-only   (plain 4 GiB device copy, for calibrating the byte counters)
       python bench.py --hbm-probe   (torch's read / write / copy kernels on 4 GiB: what this HBM delivers)
       python bench.py --matvec-sweep   (cq_dequant_matvec_many at batch 2 / 4 / 8 over the 7B-shaped
                                         model's matrices: all 225, the first layer, one 11008x4096)
       python bench.py --configs     (the small configurations: one JSON report line)
       python bench.py --trace-summary DIR   (per-kernel, per-grid table of a rocprofv3 kernel trace)
       python bench.py --counter-summary DIR (per-kernel table of a rocprofv3 --pmc run of COUNTERS)
       python bench.py --traffic-summary DIR (profiles/traffic_llama7b.{json,md} from FETCH_SIZE /
                                              WRITE_SIZE runs under DIR/{fetch,write,copy_fetch,copy_write})

--configs times, per configuration, single calls with HIP events (3 warm-up
calls, median of 15), warm (inputs cache-resident after the previous call)
and cold (a 1 GiB device write before each timed call evicts L2 and the
256 MB last-level cache):
  C1  fp32 256x512, 2 bits: quantize and dequantize latency;
  C2  the 45.8M-parameter Needle-2-sized set (fp32, 92 tensors, one 300x1000
      tensor padded): one cq_quantize_many / cq_dequantize_many call, and the
      same quantize as 92 per-tensor calls;
  C3  bf16 4096x4096 heavy-tailed matrix, ternary / 2 / 3 / 4 bits: quantize,
      dequantize and the relative reconstruction error;
  C5  the 11008x4096 matrix at batch 1 and 8: dequant-matvec (and the GEMM at
      batch 8) against the binding roof max(HBM time, fp32 VALU time);
and the CPU oracle on C1, C2, C3 (each width) and C5, in full.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CQ2 quantize+dequantize Gparams/s and % of HBM peak GB/s (1×MI355X)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16 matrix peak
BITS = 2
G = 128
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama7b.json")
KERNEL_SOURCES = ["rotated_codebook_bit_amd/csrc/quantize.hip",
                  "rotated_codebook_bit_amd/csrc/dequantize.hip",
                  "rotated_codebook_bit_amd/csrc/matvec.hip"]
# The source file of each measured phase's kernel: a traffic entry is valid
# while that file is unchanged.
PHASE_SOURCE = {"quantize": "rotated_codebook_bit_amd/csrc/quantize.hip",
                "dequantize_f32": "rotated_codebook_bit_amd/csrc/dequantize.hip",
                "matvec_pass_b1": "rotated_codebook_bit_amd/csrc/matvec.hip",
                "fake_quant_bf16_extra": "rotated_codebook_bit_amd/csrc/quantize.hip"}


def file_digest(rel: str) -> str:
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def sources_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-only", action="store_true", help="only run a plain 4 GiB device copy")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="time torch's read, write and copy kernels on 4 GiB buffers (one JSON line)")
    ap.add_argument("--configs", action="store_true", help="report the small configurations instead")
    ap.add_argument("--matvec-sweep", action="store_true",
                    help="time cq_dequant_matvec_many at batch 2/4/8 on model subsets (one JSON line)")
    ap.add_argument("--counter-summary", metavar="DIR",
                    help="per-kernel SQ counter table of a rocprofv3 --pmc run (the counters of COUNTERS)")
    ap.add_argument("--traffic-summary", metavar="DIR",
                    help="write profiles/traffic_llama7b.{json,md} from rocprofv3 counter runs under DIR")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print a per-kernel, per-grid table of a rocprofv3 kernel trace directory and exit")
    return ap.parse_args()


def matvec_sweep(torch):
    """cq_dequant_matvec_many over the 7B-shaped model's 2-bit matrices at
    batch 2, 4 and 8: all 225 matrices, the first layer (7) and one
    11008x4096 matrix; median of 15 back-to-back calls (HIP events around
    each call, the call's launches included)."""
    import rotated_codebook_bit_amd as cq
    from rotated_codebook_bit_amd import workloads as W
    buf, offsets = W.llama7b_device("cuda")
    shapes = W.llama7b_shapes()
    ng = buf.numel() // 128
    packed = torch.empty((ng, 32), dtype=torch.uint8, device="cuda")
    norms = torch.empty((ng,), dtype=torch.float16, device="cuda")
    cq.quantize(buf.view(ng, 128), 2, None, packed=packed.view(ng, 1, -1), norms=norms.view(ng, 1))
    del buf
    kmax = max(c for _, c in shapes)
    res = {}
    for batch in (2, 4, 8):
        gen = torch.Generator(device="cuda").manual_seed(batch)
        x = torch.randn((batch, kmax), generator=gen, device="cuda")
        xs = {c: x[:, :c].contiguous() for _, c in shapes}
        items = []
        for i, (r, c) in enumerate(shapes):
            g0, g1 = int(offsets[i]) // 128, int(offsets[i + 1]) // 128
            items.append((packed[g0:g1], norms[g0:g1], r, c, xs[c], torch.empty((batch, r), device="cuda")))
        one = [it for it in items if it[2] == 11008][:1]
        for name, sel in (("all_225", items), ("first_layer", items[:7]), ("one_11008x4096", one)):
            for _ in range(3):
                cq.dequant_matvec_many(sel, 2, None, batch)
            torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(16)]
            for i in range(15):
                ev[i].record()
                cq.dequant_matvec_many(sel, 2, None, batch)
            ev[15].record()
            torch.cuda.synchronize()
            ts = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(15))
            res[f"batch{batch}_{name}_us"] = round(ts[7], 1)
        del items, xs, x
    print(json.dumps({"matvec_sweep": res}), flush=True)


def copy_only(torch):
    n = 1 << 30  # 4 GiB of float32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    print(json.dumps({"copy_bytes_each_way": 4 * n, "ms": ms,
                      "GBps_read_plus_write": 2 * 4 * n / ms / 1e6}), flush=True)


def hbm_probe(torch):
    """What this HBM delivers to plain torch kernels on 4 GiB buffers: a read
    (sum of a float32 vector), a write (fill_) and a copy, each the median of
    10 timed calls after 3 untimed ones (HIP events on the current stream)."""
    n = 1 << 30  # 4 GiB of float32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    ops = {"read": (lambda: torch.sum(a, dim=0, out=acc), 4 * n),
           "write": (lambda: b.fill_(1.0), 4 * n),
           "copy": (lambda: b.copy_(a), 8 * n)}
    res = {}
    for name, (fn, nbytes) in ops.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(10):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        res[name] = {"bytes": nbytes, "ms": round(ms, 4), "TBps": round(nbytes / ms / 1e9, 3),
                     "frac_of_8TBps": round(nbytes / ms / 1e9 / 8.0, 4)}
    print(json.dumps({"hbm_probe": res, "device": torch.cuda.get_device_name(0)}), flush=True)


# fp32 FMA rate without packed instructions (which this build does not use):
# 256 CUs x 64 lanes x 2 flops x 2.4 GHz.
VALU_F32_PEAK_TFS = 78.6
MFMA_F32_PEAK_TFS = 157.3  # dense fp32 matrix peak


def call_times(torch, fn, scrub=None, n=15, warm=3) -> float:
    """Median milliseconds of n single calls timed with HIP events on the
    current stream, after `warm` untimed calls.  With `scrub`, the tensor is
    overwritten before each timed call (outside the events)."""
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        fn()
    times = []
    for _ in range(n):
        if scrub is not None:
            scrub.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    return float(np.median(times))


def warm_cold(torch, fn, scrub, nbytes=None) -> dict:
    w, c = call_times(torch, fn), call_times(torch, fn, scrub)
    r = {"warm_us": round(1e3 * w, 2), "cold_us": round(1e3 * c, 2)}
    if nbytes:
        r["warm_GBps"] = round(nbytes / w / 1e6, 1)
        r["cold_GBps"] = round(nbytes / c / 1e6, 1)
    return r


def configs_report(torch) -> dict:
    import rotated_codebook_bit_amd as cq
    from rotated_codebook_bit_amd import workloads as W
    dev = "cuda"
    scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    rep = {"report": "configs", "timing": "HIP events around single calls; median of 15 after 3 warm-up "
                                          "calls; cold = a 1 GiB device write before each timed call"}

    # C1: latency of the smallest case.  Every GPU call here passes NULL
    # levels: the library's built-in codebook.
    lv2 = None
    w = torch.from_numpy(W.small()).to(dev)
    pk, nm = cq.quantize(w, 2, lv2)
    out = torch.empty_like(w)
    nb = w.numel() * 4 + pk.numel() + nm.numel() * 2
    rep["C1"] = {"shape": [256, 512], "dtype": "f32", "bits": 2, "algorithmic_bytes": nb,
                 "quantize": warm_cold(torch, lambda: cq.quantize(w, 2, lv2, packed=pk, norms=nm), scrub, nb),
                 "dequantize": warm_cold(torch, lambda: cq.dequantize(pk, nm, 256, 512, 2, lv2, out=out), scrub, nb)}

    # C2: the Needle-2-sized parameter set.
    tensors = [torch.from_numpy(a).to(dev) for _, a in W.needle2()]
    params = sum(t.numel() for t in tensors)
    blob, views = cq.quantize_many(tensors, 2, lv2)
    nbq = params * 4 + blob.numel()
    items = [(p.reshape(t.shape[0], -1), n, t.shape[0], t.shape[1]) for t, (p, n) in zip(tensors, views)]
    outs = [torch.empty_like(t) for t in tensors]
    singles = [cq.quantize(t, 2, lv2) for t in tensors]

    def per_tensor():
        for t, (p, n) in zip(tensors, singles):
            cq.quantize(t, 2, lv2, packed=p, norms=n)

    rep["C2"] = {"tensors": len(tensors), "params": params, "model_bytes": blob.numel(),
                 "quantize_many_1_call": warm_cold(torch, lambda: cq.quantize_many(tensors, 2, lv2, blob=blob,
                                                                                    views=False), scrub, nbq),
                 "dequantize_many_1_call": warm_cold(torch, lambda: cq.dequantize_many(items, 2, lv2, outs=outs),
                                                     scrub, nbq),
                 "quantize_per_tensor_calls": warm_cold(torch, per_tensor, scrub, nbq)}
    del tensors, blob, views, items, outs, singles

    # C3: every width on the heavy-tailed 4096x4096 bf16 matrix.
    b = W.sweep_bits()
    wb = torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)
    w64 = wb.double()
    rep["C3"] = {}
    for bits, name in ((cq.TERNARY, "ternary"), (2, "2"), (3, "3"), (4, "4")):
        lv = None
        pk, nm = cq.quantize(wb, bits, lv)
        o = cq.dequantize(pk, nm, 4096, 4096, bits, lv)
        nbq = wb.numel() * 2 + pk.numel() + nm.numel() * 2
        nbd = pk.numel() + nm.numel() * 2 + o.numel() * 4
        err = float(torch.linalg.vector_norm(w64 - o.double()) / torch.linalg.vector_norm(w64))
        rep["C3"][name] = {"relative_error": round(err, 4),
                           "quantize": warm_cold(torch, lambda: cq.quantize(wb, bits, lv, packed=pk, norms=nm),
                                                 scrub, nbq),
                           "dequantize": warm_cold(torch, lambda: cq.dequantize(pk, nm, 4096, 4096, bits, lv,
                                                                                out=o), scrub, nbd)}
    del wb, w64

    # C5: the 11008x4096 product at batch 1 and 8.
    wm = torch.from_numpy(W.matvec_weight_bits().view(np.int16)).to(dev).view(torch.bfloat16)
    pk, nm = cq.quantize(wm, 2, lv2)
    rep["C5"] = {}
    for batch in (1, 8):
        x = torch.from_numpy(W.matvec_x(batch)).to(dev)
        y = torch.empty((batch, 11008), dtype=torch.float32, device=dev)
        nbm = pk.numel() + nm.numel() * 2 + x.numel() * 4 + y.numel() * 4
        flops = 2 * batch * 11008 * 4096
        t_hbm = nbm / (HBM_PEAK_GBS * 1e9) * 1e6
        # Batch 1 runs on the VALU (pair tables), larger batches on the fp32 matrix cores.
        t_cmp = flops / ((VALU_F32_PEAK_TFS if batch == 1 else MFMA_F32_PEAK_TFS) * 1e12) * 1e6
        roof = max(t_hbm, t_cmp)
        r = {"algorithmic_bytes": nbm, "flops": flops, "t_hbm_us": round(t_hbm, 3),
             "t_compute_us": round(t_cmp, 3),
             "binding": "hbm" if t_hbm >= t_cmp else ("valu (fp32)" if batch == 1 else "mfma (fp32)")}
        mv = warm_cold(torch, lambda: cq.dequant_matvec(pk, nm, 11008, 4096, 2, lv2, x, y=y), scrub)
        mv["frac_of_roof_warm"] = round(roof / mv["warm_us"], 3)
        mv["frac_of_roof_cold"] = round(roof / mv["cold_us"], 3)
        r["matvec"] = mv
        if batch >= 8:
            gm = warm_cold(torch, lambda: cq.dequant_gemm(pk, nm, 11008, 4096, 2, lv2, x, y=y), scrub)
            gm["frac_of_roof_warm"] = round(roof / gm["warm_us"], 3)
            r["gemm"] = gm
        rep["C5"][f"batch{batch}"] = r
    rep["notes"] = ("C1, C3 and C5 take a few microseconds of kernel time, so launch latency and the "
                    "per-call descriptor and rotation launches dominate their call times")
    return rep


def c5_phases(torch, cq, W, scrub) -> dict:
    """cq_dequant_matvec on the 11008x4096 2-bit matrix at batch 1 and 8:
    median call time (HIP events around one call, launch included), warm and
    cold, and its fraction of the binding roof."""
    wm = torch.from_numpy(W.matvec_weight_bits().view(np.int16)).to("cuda").view(torch.bfloat16)
    pk, nm = cq.quantize(wm, 2, None)
    del wm
    out = {}
    for batch in (1, 8):
        x = torch.from_numpy(W.matvec_x(batch)).to("cuda")
        y = torch.empty((batch, 11008), dtype=torch.float32, device="cuda")
        nbm = pk.numel() + nm.numel() * 2 + x.numel() * 4 + y.numel() * 4
        flops = 2 * batch * 11008 * 4096
        t_hbm = nbm / (HBM_PEAK_GBS * 1e9) * 1e6
        # Batch 1 runs on the VALU (pair tables), larger batches on the fp32 matrix cores.
        t_cmp = flops / ((VALU_F32_PEAK_TFS if batch == 1 else MFMA_F32_PEAK_TFS) * 1e12) * 1e6
        roof = max(t_hbm, t_cmp)
        r = warm_cold(torch, lambda: cq.dequant_matvec(pk, nm, 11008, 4096, 2, None, x, y=y), scrub)
        r.update({"algorithmic_bytes": nbm, "flops": flops, "roof_us": round(roof, 3),
                  "binding": "hbm" if t_hbm >= t_cmp else ("valu (fp32)" if batch == 1 else "mfma (fp32)"),
                  "frac_of_roof_warm": round(roof / r["warm_us"], 4),
                  "frac_of_roof_cold": round(roof / r["cold_us"], 4)})
        out[f"batch{batch}"] = r
    out["note"] = ("call times include the launch; kernel times are in the rocprofv3 trace "
                   "(profiles/kernel_trace_configs.md)")
    return out


def c2_phases(torch, cq, W, scrub) -> dict:
    """The 92-tensor Needle-2-sized set (fp32) through one cq_quantize_many
    call (writing the blob) and one cq_dequantize_many call: call times warm
    and cold, GB/s of algorithmic bytes."""
    tensors = [torch.from_numpy(a).to("cuda") for _, a in W.needle2()]
    params = sum(t.numel() for t in tensors)
    blob, views = cq.quantize_many(tensors, 2, None)
    nb = params * 4 + blob.numel()
    items = [(p.reshape(t.shape[0], -1), n, t.shape[0], t.shape[1]) for t, (p, n) in zip(tensors, views)]
    outs = [torch.empty_like(t) for t in tensors]
    r = {"tensors": len(tensors), "params": params, "model_bytes": blob.numel(), "algorithmic_bytes": nb,
         "quantize_many": warm_cold(torch, lambda: cq.quantize_many(tensors, 2, None, blob=blob, views=False),
                                    scrub, nb),
         "dequantize_many": warm_cold(torch, lambda: cq.dequantize_many(items, 2, None, outs=outs), scrub, nb)}
    del tensors, blob, views, items, outs
    return r


def trace_summary(path: str) -> None:
    """Per (kernel, grid) dispatch counts and durations of the library's
    kernels from the kernel-trace CSV files of a rocprofv3 output directory
    (one markdown table)."""
    import csv
    import glob
    import statistics
    rows = {}
    for f in glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
                if "cq::" not in name:  # the library's kernels only, not torch's input generation
                    continue
                key = (name, r.get("Grid_Size_X", r.get("Grid_Size", "")),
                       r.get("Grid_Size_Y", "1"), r.get("Workgroup_Size_X", r.get("Workgroup_Size", "")))
                rows.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print("| kernel | grid x | grid y | block | launches | median us | mean us | min us | total us |")
    print("|---|---|---|---|---|---|---|---|---|")
    for (name, gx, gy, wg), ds in sorted(rows.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{name}` | {gx} | {gy} | {wg} | {len(ds)} | {statistics.median(ds):.2f} | "
              f"{statistics.mean(ds):.2f} | {min(ds):.2f} | {sum(ds):.1f} |")


# Kernels of the traffic profile: phase -> kernel name (the largest dispatch
# of that name is the whole-model launch).
TRAFFIC_KERNELS = {"quantize": "cq::kq::quantize_contig<4, true, false, false>",
                   "dequantize_f32": "cq::kd::dequantize_quad_contig<2, false, false, false>",
                   "matvec_pass_b1": "cq::km::matvec_pair_kernel<",
                   "fake_quant_bf16_extra": "cq::kq::fakequant_contig<4, true, true>"}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 4 << 30  # copy_only: 4 GiB read and 4 GiB written


def traffic_summary(path: str) -> None:
    """Writes profiles/traffic_llama7b.{json,md} from four rocprofv3 --pmc
    runs under `path` (CSV output): fetch/ and write/ (FETCH_SIZE or
    WRITE_SIZE of `bench.py --steps 1 --warmup 0 --no-cpu`), copy_fetch/ and
    copy_write/ (the same counters of `bench.py --copy-only`).  Each counter
    is scaled by what it reports for the copy, whose bytes are known."""
    import csv
    import glob
    from rotated_codebook_bit_amd import workloads as W

    def largest(sub, counter, name_prefix):
        best = None
        for f in glob.glob(os.path.join(path, sub, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    name = r["Kernel_Name"].replace("(anonymous namespace)::", "")
                    if r["Counter_Name"] != counter or not (name.startswith(name_prefix)
                                                           or name.startswith("void " + name_prefix)):
                        continue
                    key = (int(r["Grid_Size"]), float(r["Counter_Value"]))
                    if best is None or key > best:
                        best = key
        if best is None:
            raise SystemExit(f"no {counter} dispatch of {name_prefix} under {path}/{sub}")
        return best[1] * 1024.0  # KiB -> bytes

    fs = COPY_BYTES / largest("copy_fetch", "FETCH_SIZE", COPY_KERNEL)
    ws = COPY_BYTES / largest("copy_write", "WRITE_SIZE", COPY_KERNEL)
    shapes = W.llama7b_shapes()
    params = sum(r * c for r, c in shapes)
    ng = params // G
    alg = {"quantize": params * 2 + ng * (G * BITS // 8) + ng * 2,
           "dequantize_f32": ng * (G * BITS // 8) + ng * 2 + params * 4,
           "matvec_pass_b1": ng * (G * BITS // 8 + 2) + sum(c * 4 + r * 4 for r, c in shapes),
           "fake_quant_bf16_extra": params * 4}
    kernels = {}
    for phase, kname in TRAFFIC_KERNELS.items():
        fb = round(largest("fetch", "FETCH_SIZE", kname) * fs)
        wb = round(largest("write", "WRITE_SIZE", kname) * ws)
        kernels[phase] = {"kernel": kname.replace("cq::", "").rstrip("<"), "fetch_bytes": fb, "write_bytes": wb,
                          "hbm_bytes_per_launch": fb + wb, "algorithmic_bytes": alg[phase],
                          "source": PHASE_SOURCE[phase], "source_digest": file_digest(PHASE_SOURCE[phase])}
    cmd = "cd /tmp && export TMPDIR=/tmp && timeout -s KILL 240 rocprofv3 --pmc {c} --output-format csv -d $R/{d} -o run -- python3 $R/bench.py {a}"
    out = {"what": ("HBM bytes per launch on the 7B-shaped model (bf16, 2-bit, G=128), from rocprofv3 FETCH_SIZE "
                    "and WRITE_SIZE (KiB per dispatch, the largest dispatch of each kernel), each scaled by what the "
                    f"same counter reports for a plain 4 GiB device copy ({COPY_KERNEL}): scale {fs:.3f} for "
                    f"FETCH_SIZE, {ws:.3f} for WRITE_SIZE."),
           "commands": [cmd.format(c="FETCH_SIZE", d=f"{path}/fetch", a="--steps 1 --warmup 0 --no-cpu"),
                        cmd.format(c="WRITE_SIZE", d=f"{path}/write", a="--steps 1 --warmup 0 --no-cpu"),
                        cmd.format(c="FETCH_SIZE", d=f"{path}/copy_fetch", a="--copy-only"),
                        cmd.format(c="WRITE_SIZE", d=f"{path}/copy_write", a="--copy-only"),
                        f"python3 bench.py --traffic-summary {path}"],
           "kernels": kernels,
           "note": ("each entry holds the digest of its kernel's source file as measured; bench.py reports an "
                    "entry only while that file is unchanged")}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    lines = ["# HBM traffic per launch: 7B-shaped model (bf16, 2-bit, G=128)", "",
             "Counters: rocprofv3 `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch), one pass each, "
             "`python3 bench.py --steps 1 --warmup 0 --no-cpu`; per kernel the largest dispatch (the whole-model "
             "launch); the commands are in `traffic_llama7b.json`, which `python3 bench.py --traffic-summary DIR` "
             "writes together with this file.",
             f"Calibration: a plain 4 GiB device copy (`bench.py --copy-only`, kernel `{COPY_KERNEL}`); scale "
             f"{fs:.3f} for `FETCH_SIZE`, {ws:.3f} for `WRITE_SIZE`.", "",
             "| kernel | read (scaled) | written (scaled) | total | algorithmic | ratio |", "|---|---|---|---|---|---|"]
    for phase, k in kernels.items():
        lines.append(f"| {k['kernel']} | {k['fetch_bytes'] / 1e9:.3f} GB | {k['write_bytes'] / 1e9:.3f} GB | "
                     f"{k['hbm_bytes_per_launch'] / 1e9:.3f} GB | {k['algorithmic_bytes'] / 1e9:.3f} GB | "
                     f"{k['hbm_bytes_per_launch'] / k['algorithmic_bytes']:.4f} |")
    lines += ["", "Each kernel's source digest at measurement is in `traffic_llama7b.json`."]
    with open(TRAFFIC_FILE.replace(".json", ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(open(TRAFFIC_FILE.replace(".json", ".md")).read())


COUNTERS = ["GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU", "SQ_BUSY_CU_CYCLES",
            "SQ_INSTS_LDS", "SQ_ACTIVE_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_VALU_MFMA_BUSY_CYCLES"]


def counter_summary(path: str) -> None:
    """Per (kernel, grid) medians of the SQ counters of one rocprofv3 --pmc
    run under `path` (CSV output; the counters of COUNTERS), library kernels
    only, as a markdown table.  Units as this GPU reports them:
    GRBM_GUI_ACTIVE is GPU cycles summed over the 8 XCDs; SQ_BUSY_CU_CYCLES,
    SQ_ACTIVE_INST_VALU and SQ_ACTIVE_INST_LDS are quad-cycles summed over the
    SIMDs; SQ_LDS_BANK_CONFLICT and SQ_VALU_MFMA_BUSY_CYCLES are cycles summed
    over the SIMDs.  Derived columns: clock = GRBM_GUI_ACTIVE / 8 / the
    dispatch's duration (its timestamps in the same run); VALU busy =
    SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES (above 1 where two waves issue a
    VALU instruction each in one quad-cycle); LDS conflict =
    SQ_LDS_BANK_CONFLICT / (4 SQ_ACTIVE_INST_LDS), the share of LDS-active
    cycles lost to bank conflicts; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /
    (4 SQ_BUSY_CU_CYCLES)."""
    import csv
    import glob
    import statistics
    vals = {}
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
                if "cq::" not in name:
                    continue
                key = (name.replace("void ", ""), r["Grid_Size"])
                d = vals.setdefault(key, {}).setdefault(r["Dispatch_Id"], {})
                d[r["Counter_Name"]] = float(r["Counter_Value"])
                d["ns"] = float(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("| kernel | grid | dispatches | " + " | ".join(c for c in COUNTERS) +
          " | us | clock GHz | VALU busy | LDS conflict | MFMA busy |")
    print("|---|---|---|" + "---|" * (len(COUNTERS) + 5))
    order = sorted(vals.items(), key=lambda kv: -statistics.median(
        d.get("GRBM_GUI_ACTIVE", 0.0) for d in kv[1].values()))
    for (name, grid), disp in order:
        med = {c: statistics.median(d.get(c, 0.0) for d in disp.values()) for c in COUNTERS + ["ns"]}
        busy = med["SQ_BUSY_CU_CYCLES"]
        valu = med["SQ_ACTIVE_INST_VALU"] / busy if busy else 0.0
        lds = med["SQ_LDS_BANK_CONFLICT"] / (4 * med["SQ_ACTIVE_INST_LDS"]) if med["SQ_ACTIVE_INST_LDS"] else 0.0
        mfma = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (4 * busy) if busy else 0.0
        clock = med["GRBM_GUI_ACTIVE"] / 8 / med["ns"] if med["ns"] else 0.0
        print(f"| `{name}` | {grid} | {len(disp)} | " + " | ".join(f"{med[c]:.4g}" for c in COUNTERS) +
              f" | {med['ns'] / 1e3:.1f} | {clock:.2f} | {valu:.3f} | {lds:.3f} | {mfma:.3f} |")


def cpu_baseline_configs() -> dict:
    """The oracle on C1, C2, C3 (each width) and C5 in full: quantize +
    dequantize (C5: dequantize + the float64 product), params/s."""
    from oracle import cq_oracle as O
    from rotated_codebook_bit_amd import workloads as W
    import rotated_codebook_bit_amd as cq
    res = {}

    samples = W.lloyd_samples()

    def run(name, ws, bits, extra=None):
        lv = O.runtime_levels(O.codebook(bits, samples)).astype(np.float32)
        t0 = time.perf_counter()
        n = 0
        for w in ws:
            q = O.quantize(w, bits, lv)
            wh = O.dequantize(q.packed, q.norm16, w.shape[0], w.shape[1], bits, lv)
            if extra is not None:
                extra(wh)
            n += w.size
        dt = time.perf_counter() - t0
        res[name] = {"s": round(dt, 3), "Mparams_per_s": round(n / dt / 1e6, 3)}

    run("C1", [W.small().astype(np.float64)], 2)
    run("C2", [a.astype(np.float64) for _, a in W.needle2()], 2)
    w3 = W.bf16_bits_to_f32(W.sweep_bits()).astype(np.float64)
    for bits, name in ((cq.TERNARY, "ternary"), (2, "2"), (3, "3"), (4, "4")):
        run(f"C3_{name}", [w3], bits)
    wm = W.bf16_bits_to_f32(W.matvec_weight_bits()).astype(np.float64)
    for batch in (1, 8):
        x = W.matvec_x(batch).astype(np.float64)
        run(f"C5_batch{batch}", [wm], 2, extra=lambda wh: x @ wh.T)
    res["note"] = "float64 NumPy oracle; C5 includes quantizing W (its input is the float matrix)"
    res["cpu_count"] = os.cpu_count()
    return res


def cpu_baseline() -> dict:
    """The oracle as it stands, on one transformer layer of the 7B-shaped
    model plus its embedding (4 x 4096x4096, 2 x 4096x11008, 11008x4096,
    32000x4096 = 333,447,168 params): quantize, dequantize and a batch-1
    matvec per tensor, the per-tensor work of one step."""
    from oracle import cq_oracle as O
    from rotated_codebook_bit_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count() or 1
    levels = O.runtime_levels(O.codebook(BITS, W.lloyd_samples())).astype(np.float32)
    rng = np.random.default_rng(0)
    shapes = W.llama7b_shapes()
    layer = shapes[:7] + shapes[-1:]
    params = 0
    dt = 0.0
    for r, c in layer:
        w = W.bf16_round((rng.standard_normal((r, c)) * 0.02).astype(np.float32)).astype(np.float64)
        x = rng.standard_normal((1, c))
        t0 = time.perf_counter()
        q = O.quantize(w, BITS, levels)
        w_hat = O.dequantize(q.packed, q.norm16, r, c, BITS, levels)
        _ = x @ w_hat.T
        dt += time.perf_counter() - t0
        params += w.size
        del w, q, w_hat
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(params / dt / 1e9, 6), "unit": "Gparams/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"one 7B-shaped transformer layer + the embedding ({params:,} bf16-valued "
                      f"params, 8 tensors) "
                      f"through quantize, dequantize and a batch-1 matvec, float64 NumPy, "
                      f"{dt:.1f} s timed; host {model}, cpu_count={os.cpu_count()}, "
                      f"BLAS threads={blas_threads}"}


def main():
    args = parse()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.hbm_probe:
        hbm_probe(torch)
        return
    if args.matvec_sweep:
        matvec_sweep(torch)
        return
    if args.copy_only:
        copy_only(torch)
        return
    if args.configs:
        rep = configs_report(torch)
        if not args.no_cpu:
            log("CPU oracle on the small configurations")
            rep["cpu_oracle"] = cpu_baseline_configs()
        print(json.dumps(rep), flush=True)
        return

    import rotated_codebook_bit_amd as cq
    from rotated_codebook_bit_amd import workloads as W

    levels = None  # the library's built-in codebook
    shapes = W.llama7b_shapes()
    log("generating the 7B-shaped bf16 model on the device")
    buf, offsets = W.llama7b_device("cuda")
    params = buf.numel()
    n_groups = params // G
    w2 = buf.view(n_groups, G)
    packed = torch.empty((n_groups, G * BITS // 8), dtype=torch.uint8, device="cuda")
    norms = torch.empty((n_groups,), dtype=torch.float16, device="cuda")
    out = torch.empty((n_groups, G), dtype=torch.float32, device="cuda")
    kmax = max(c for _, c in shapes)
    nmax = max(r for r, _ in shapes)
    xg = torch.Generator(device="cuda")
    xg.manual_seed(1)
    x = torch.randn((1, kmax), generator=xg, device="cuda", dtype=torch.float32)
    # One y row per matrix (y[i, :rows_i]); row slices of a contiguous
    # matrix are contiguous.
    y_all = torch.empty((len(shapes), nmax), dtype=torch.float32, device="cuda")
    # Per-tensor views of the packed model (groups never straddle tensors:
    # every column count is a multiple of 128).
    views = []
    for i, (r, c) in enumerate(shapes):
        g0, g1 = int(offsets[i]) // G, int(offsets[i + 1]) // G
        views.append((packed[g0:g1], norms[g0:g1], r, c))
    stream = torch.cuda.current_stream()

    # x[:, :c] for each column count: the activations, contiguous.
    xs = {c: x[:, :c].contiguous() for _, c in shapes}
    items = [(p, nv, r, c, xs[c], y_all[i:i + 1, :r]) for i, (p, nv, r, c) in enumerate(views)]

    def step2(ev=None):
        if ev:
            ev[0].record(stream)
        cq.quantize(w2, BITS, levels, packed=packed.view(n_groups, 1, -1),
                    norms=norms.view(n_groups, 1))
        if ev:
            ev[1].record(stream)
        cq.dequantize(packed, norms, n_groups, G, BITS, levels, out=out)
        if ev:
            ev[2].record(stream)
        cq.dequant_matvec_many(items, BITS, levels, 1)
        if ev:
            ev[3].record(stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step2()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step2(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    tq = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    tdq = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    tmv = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))

    sb = BITS
    q_bytes = params * 2 + n_groups * (G * sb // 8) + n_groups * 2
    dq_bytes = n_groups * (G * sb // 8) + n_groups * 2 + params * 4
    mv_bytes = n_groups * (G * sb // 8 + 2) + sum(c * 4 + r * 4 for r, c in shapes)

    def gbs(b, ms):
        return b / (ms * 1e-3) / 1e9

    phases = {
        "quantize": {"ms": round(tq, 4), "Gparams_per_s": round(params / tq / 1e6, 1),
                     "GB_per_s": round(gbs(q_bytes, tq), 1), "bytes": q_bytes,
                     "frac_hbm_peak": round(gbs(q_bytes, tq) / HBM_PEAK_GBS, 4)},
        "dequantize_f32": {"ms": round(tdq, 4), "Gparams_per_s": round(params / tdq / 1e6, 1),
                           "GB_per_s": round(gbs(dq_bytes, tdq), 1), "bytes": dq_bytes,
                           "frac_hbm_peak": round(gbs(dq_bytes, tdq) / HBM_PEAK_GBS, 4)},
        "matvec_pass_b1": {"ms": round(tmv, 4), "matrices": len(shapes),
                           "GB_per_s": round(gbs(mv_bytes, tmv), 1), "bytes": mv_bytes},
        "quantize_plus_dequantize_Gparams_per_s": round(params / (tq + tdq) / 1e6, 1),
    }
    # Fused fake quantization (quantize + reconstruct, bf16 -> bf16, one
    # launch over the whole model), timed on its own after the step.
    fq_out = torch.empty_like(buf)
    for _ in range(2):
        cq.fake_quant(buf, BITS, levels, out=fq_out)
    fe = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in fe:
        e[0].record(stream)
        cq.fake_quant(buf, BITS, levels, out=fq_out)
        e[1].record(stream)
    torch.cuda.synchronize()
    tfq = float(np.mean([e[0].elapsed_time(e[1]) for e in fe]))
    fq_bytes = params * 2 * 2
    del fq_out
    phases["fake_quant_bf16_extra"] = {
        "ms": round(tfq, 4), "Gparams_per_s": round(params / tfq / 1e6, 1),
        "GB_per_s": round(gbs(fq_bytes, tfq), 1), "bytes": fq_bytes,
        "frac_hbm_peak": round(gbs(fq_bytes, tfq) / HBM_PEAK_GBS, 4),
        "note": "not part of the step; bf16 in, bf16 out, one launch"}
    # Prefill-style batched product through all 225 matrices on the matrix
    # cores (split-bf16 MFMA, three MFMAs per product), batch 256.
    GB_ = 256
    gx = {c: torch.randn((GB_, c), generator=xg, device="cuda", dtype=torch.float32)
          for c in sorted({c for _, c in shapes})}
    gy = [torch.empty((GB_, r), dtype=torch.float32, device="cuda") for r, _ in shapes]
    gitems = [(p_, nv, r, c, gx[c], gy[i]) for i, (p_, nv, r, c) in enumerate(views)]
    cq.dequant_gemm_many(gitems, BITS, levels, GB_)
    torch.cuda.synchronize()
    ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ge[0].record(stream)
    for _ in range(3):
        cq.dequant_gemm_many(gitems, BITS, levels, GB_)
    ge[1].record(stream)
    torch.cuda.synchronize()
    tg = ge[0].elapsed_time(ge[1]) / 3
    alg_tf = 2 * GB_ * params / (tg * 1e-3) / 1e12
    phases["dequant_gemm_b256_extra"] = {
        "ms": round(tg, 4), "alg_TFLOP_per_s": round(alg_tf, 1),
        "mfma_bf16_TFLOP_per_s_executed": round(3 * alg_tf, 1),
        "frac_bf16_mfma_peak_executed": round(3 * alg_tf / MFMA_BF16_PEAK_TFS, 4),
        "note": "batch-256 product through all 225 matrices (one cq_dequant_gemm_many call: rotation + "
                "MFMA launch); fp32-grade split-bf16 arithmetic, 3 MFMAs per product; not part of the step"}
    del gx, gy, gitems

    # Quantize as 225 back-to-back per-tensor calls on one stream (launch
    # gaps and small-tensor tails), against the one flat launch above.
    def per_tensor():
        for i, (r, c) in enumerate(shapes):
            o0, o1 = int(offsets[i]), int(offsets[i + 1])
            g0, g1 = o0 // G, o1 // G
            cq.quantize(buf[o0:o1].view(r, c), BITS, levels, packed=packed[g0:g1].view(r, c // G, -1),
                        norms=norms[g0:g1].view(r, c // G))
    per_tensor()
    torch.cuda.synchronize()
    pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    reps = 3
    pe[0].record(stream)
    for _ in range(reps):
        per_tensor()
    pe[1].record(stream)
    torch.cuda.synchronize()
    tpt = pe[0].elapsed_time(pe[1]) / reps
    phases["quantize_225_calls_extra"] = {
        "ms": round(tpt, 4), "GB_per_s": round(gbs(q_bytes, tpt), 1),
        "note": "the same quantize as 225 per-tensor calls; not part of the step"}

    # The same 225 tensors through one multi-tensor call, writing the
    # serialized blob (all packed indices, then all norms).
    tviews = [buf[int(offsets[i]):int(offsets[i + 1])].view(r, c) for i, (r, c) in enumerate(shapes)]
    blob, _ = cq.quantize_many(tviews, BITS, levels)
    torch.cuda.synchronize()
    pe[0].record(stream)
    for _ in range(reps):
        cq.quantize_many(tviews, BITS, levels, blob=blob, views=False)
    pe[1].record(stream)
    torch.cuda.synchronize()
    tqm = pe[0].elapsed_time(pe[1]) / reps
    phases["quantize_many_1_call_extra"] = {
        "ms": round(tqm, 4), "GB_per_s": round(gbs(q_bytes, tqm), 1),
        "note": "the same quantize as one cq_quantize_many call over the 225 tensors, writing the "
                "serialized blob; not part of the step"}
    del blob

    # The 11008x4096 product (one cq_dequant_matvec call: one launch, no
    # workspace) at batch 1 and 8, warm and cold (a 1 GiB device write before
    # each timed call), against its binding roof max(HBM time, fp32 VALU time).
    del out
    torch.cuda.empty_cache()
    scrub = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    phases["matvec_11008x4096_extra"] = c5_phases(torch, cq, W, scrub)
    # The 45.8M-parameter Needle-2-sized set: 92 fp32 tensors (one 300x1000,
    # padded) through one cq_quantize_many call writing the serialized blob
    # and one cq_dequantize_many call back to fp32, warm and cold.
    phases["needle2_92_tensors_extra"] = c2_phases(torch, cq, W, scrub)
    del scrub

    dom = "dequantize_f32" if tdq >= tq else "quantize"
    dom_kernel = {"dequantize_f32": "dequantize_quad_contig<2, false, false, false>",
                  "quantize": "quantize_contig<4, true, false, false>"}
    ach = gbs(phases[dom]["bytes"], phases[dom]["ms"])
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            t = json.load(open(TRAFFIC_FILE))
            entry = t.get("kernels", {}).get(dom, {})
            if entry.get("source_digest") == file_digest(PHASE_SOURCE[dom]):
                traffic = entry["hbm_bytes_per_launch"]
        except Exception:
            traffic = None
    roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dom_kernel[dom], "bytes_per_launch": phases[dom]["bytes"]}
    result = {
        "metric": METRIC,
        "value": round(params / (ms_step * 1e-3) / 1e9, 2),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "llama7b-shaped: 32x[4x(4096x4096), 2x(4096x11008), 11008x4096] + "
                               "32000x4096, bf16 N(0,0.02^2), 6,607,077,376 params, bits=2, G=128",
                   "step": "quantize (1 launch) + dequantize to f32 (1 launch) + batch-1 "
                           "dequant-matvec through all 225 matrices (1 call)",
                   "parallelism": "single GPU"},
        "phases": phases,
        "roofline": roofline,
        "sources_digest": sources_digest(),
    }
    del buf
    torch.cuda.empty_cache()
    if not args.no_cpu:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
