// CQ dequantize kernels for gfx950.
//
// Method (web pages, by title and section):
//   "Cactus Quants CQ2-bit Quantization: Extreme Compression for Edge LLMs",
//     The CQ2-bit Implementation Pipeline: look the levels up, rescale by the
//     group norm, rotate back with the (self-inverse) orthonormal Hadamard
//     matrix, drop the padding;
//   "How CQ2-bit Quantization Contributes to Needle 2's Small Footprint",
//     Per-Group Storage Breakdown: packed indices + one fp16 norm per group.
//
// x_hat = (norm/sqrt(G)) * levels[idx] * Hn with Hn = H/sqrt(G) (H the +-1
// Sylvester matrix), i.e. x_hat = (norm / G) * H levels[idx]; 1/G = 2^-7 is
// exact.
//
// Kernels:
//   dequantize_quad_contig  whole-group tensors (cols % 128 == 0): 2-, 3- or
//                           4-bit fields or trit storage, a quad of lanes
//                           per group, 16-group steps per wave, stores of
//                           whole kilobytes;
//   dequantize_ragged       rows whose length is not a multiple of 128 (a
//                           quad of lanes per group, padding dropped).

#include "cq_internal.h"

namespace cq {
namespace kd {

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Byte table: a packed byte holds E = 8 / SB consecutive indices (E = 4 at 2
// bits, 2 at 4 bits).  Entry b is the unnormalised E-point Walsh-Hadamard
// transform of the levels its indices select, so one table read replaces E
// lookups and the first log2(E) butterfly stages.  The adds are the same
// float32 operations, in the same order, as running those stages in
// registers.
template <int SB>
struct ByteTable {
  static constexpr int E = 8 / SB;
  static __device__ __forceinline__ void fill(float* tab, const LevelTable& lv, int t) {
    if (t >= 256) return;
    float q[4];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = (t >> (SB * e)) & ((1 << SB) - 1);
      q[e] = level_at(lv, i);
    }
    if constexpr (E == 4) {
      const float a0 = q[0] + q[1], a1 = q[0] - q[1], a2 = q[2] + q[3], a3 = q[2] - q[3];
      const float v0 = a0 + a2, v1 = a1 + a3, v2 = a0 - a2, v3 = a1 - a3;
      tab[4 * t] = v0;
      tab[4 * t + 1] = v1;
      tab[4 * t + 2] = v2;
      tab[4 * t + 3] = v3;
      wait_lds_writes();
      hold_values(v0, v1, v2, v3);
    } else {
      const float v0 = q[0] + q[1], v1 = q[0] - q[1];
      tab[2 * t] = v0;
      tab[2 * t + 1] = v1;
      wait_lds_writes();
      hold_values(v0, v1);
    }
  }
};

template <int SB>
struct TableSize {
  static constexpr int floats = SB == 3 ? kMaxLevels : 256 * (8 / SB);
};

template <int SB>
__device__ __forceinline__ void fill_table(float* tab, const LevelTable& lv, int t) {
  if constexpr (SB == 3) {
    if (t < kMaxLevels) {
      const float v = level_at(lv, t);
      tab[t] = v;
      wait_lds_writes();
      hold_values(v);
    }
  } else {
    ByteTable<SB>::fill(tab, lv, t);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ void fill_trit_table(uint16_t* ttab, int t) {
  if (t < 256) {
    const uint32_t v = trit_table_entry(static_cast<uint32_t>(t));
    ttab[t] = static_cast<uint16_t>(v);
    wait_lds_writes();
    hold_values(v);
  }
}

// Cache policy of the output stores (the buffer instruction's aux bits:
// 2 = nt, 16 = sc1): "nt sc1", streaming, for both output types.  On the
// 7B-shaped model it took the one-lane-per-group kernel this library had
// first from 5.18 to 4.92 ms for float32 output (nt or sc1 alone: 5.05, sc0
// sc1: 5.05); with the quad kernel nt alone, sc1 alone and the default
// policy were 1-3% slower for float32, and the default 3-9% slower for bf16
// (3.03 against 2.78-2.80 ms in 4-wave blocks).
[[maybe_unused]] constexpr int kStoreStream = 2 | 16;  // used in device code only

template <int AUX>
__device__ __forceinline__ void store16(const uint4& v, __amdgpu_buffer_rsrc_t dst, uint32_t voff,
                                        uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, dst, voff, soff, AUX);
#endif
}

// One launch of the quad kernel: one tensor (MANY = false: packed, norms,
// out, n_groups) or a table of tensors whose column counts are multiples of
// 128 (MANY = true: t and the total of their 64-group batches, each tensor's
// batches numbered consecutively).
struct DequantJob {
  const uint8_t* packed;
  const uint16_t* norms;
  uint8_t* out;
  int64_t n_groups;
  TensorTable<DequantDesc> t;
  int64_t n_batches;
};

// General path: rows whose length is not a multiple of 128, in quad form
// (see quad_load / quad_butterfly_across): lane q of a quad reads the
// quarter of its group's packed bytes that codes elements 32q .. 32q+31,
// looks them up (the byte table also runs the first butterfly stages), runs
// the remaining stages in its registers and across the quad, scales by
// norm / 128 and writes its existing elements.  One-wave blocks take 16
// groups per step of a grid-stride loop.  With MANY, unit u is group u of
// the concatenation of the table's tensors and the plain arguments are
// ignored.
template <int SB, bool BF16OUT, bool MANY, bool TRITS, bool WIDE>
__global__ void __launch_bounds__(kWave)
dequantize_ragged(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                  int64_t rows, int64_t cols, LevelTable lv, uint8_t* __restrict__ out,
                  TensorTable<DequantDesc> t, int64_t total) {
  __shared__ __attribute__((aligned(16))) float tab[TableSize<SB>::floats];
  __shared__ uint16_t ttab[TRITS ? 256 : 1];
#pragma unroll
  for (int i = 0; i < 256; i += kWave) {
    if constexpr (TRITS) fill_trit_table(ttab, i + threadIdx.x);
    fill_table<SB>(tab, lv, i + threadIdx.x);
  }
  __syncthreads();
  constexpr int PB = 16 * SB;  // packed bytes per group (2-bit fields for trits)
  const int q = threadIdx.x & 3;
  const int64_t n_units = MANY ? total : rows * ((cols + kGroup - 1) / kGroup);
  const int64_t n_steps = (n_units + kQuadGroups - 1) / kQuadGroups;
  for (int64_t s = blockIdx.x; s < n_steps; s += gridDim.x) {
    int64_t u = s * kQuadGroups + (threadIdx.x >> 2);
    const bool live = u < n_units;
    if (!live) u = n_units - 1;  // the quad computes on a real group and stores nothing
    const uint8_t* pk = packed;
    const uint16_t* nm = norms;
    uint8_t* o = out;
    int64_t c = cols, gl = u;
    if constexpr (MANY) {
      const int d = find_unit(t.start, 0, t.n, u);
      const DequantDesc* qd = t.desc + d;
      pk = load_const(&qd->packed);
      nm = load_const(&qd->norms);
      o = load_const(&qd->out);
      c = load_const(&qd->cols);
      gl = u - load_const(t.start + d);
    }
    const QuadPlace pl = quad_place(gl, c);
    uint32_t words[SB];
    if constexpr (TRITS) {
      uint32_t tr[13], all[8];
      const uint16_t* src = reinterpret_cast<const uint16_t*>(pk + gl * kTritBytes);
#pragma unroll
      for (int k = 0; k < 13; ++k) tr[k] = src[k];
      trits_to_fields(tr, ttab, all);
      words[0] = q == 0 ? all[0] : q == 1 ? all[2] : q == 2 ? all[4] : all[6];
      words[1] = q == 0 ? all[1] : q == 1 ? all[3] : q == 2 ? all[5] : all[7];
    } else {
      const uint8_t* src = pk + gl * PB + q * (4 * SB);
      if constexpr (SB == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(src);
        words[0] = v.x;
        words[1] = v.y;
      } else if constexpr (SB == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(src);
        words[0] = v.x;
        words[1] = v.y;
        words[2] = v.z;
        words[3] = v.w;
      } else {
#pragma unroll
        for (int i = 0; i < SB; ++i) words[i] = reinterpret_cast<const uint32_t*>(src)[i];
      }
    }
    const uint16_t n16 = nm[gl];
    float y[kQuadElems];
    if constexpr (SB == 3) {
      // Element m's field at bit 3m of the lane's 96 bits.
#pragma unroll
      for (int m = 0; m < kQuadElems; ++m) {
        const int pos = 3 * m, wd = pos >> 5, off = pos & 31;
        uint32_t v = words[wd] >> off;
        if (off > 29) v |= words[wd + 1] << (32 - off);
        y[m] = tab[v & 7u];
      }
      quad_butterfly_in_lane<1>(y);
    } else {
      constexpr int E = ByteTable<SB>::E;
#pragma unroll
      for (int k = 0; k < kQuadElems / E; ++k) {
        const uint32_t b = (words[k >> 2] >> (8 * (k & 3))) & 0xFFu;
        if constexpr (E == 4) {
          const float4 v = *reinterpret_cast<const float4*>(tab + 4 * b);
          y[4 * k] = v.x;
          y[4 * k + 1] = v.y;
          y[4 * k + 2] = v.z;
          y[4 * k + 3] = v.w;
        } else {
          const float2 v = *reinterpret_cast<const float2*>(tab + 2 * b);
          y[2 * k] = v.x;
          y[2 * k + 1] = v.y;
        }
      }
      quad_butterfly_in_lane<E>(y);
    }
    quad_butterfly_across<1>(y, q);
    quad_butterfly_across<2>(y, q);
    const float sc = half_to_float(n16) * (1.0f / kGroup);
#pragma unroll
    for (int j = 0; j < kQuadElems; ++j) y[j] *= sc;
    if (live) quad_store<BF16OUT, WIDE>(o, pl.first, pl.valid, q, y);
  }
}

// Quad form for whole-group tensors (cols % 128 == 0), 2-, 3- or 4-bit
// fields, float32 or bf16 output.  A wave takes a step of 16 consecutive
// groups of one tensor: lane 4i + q holds elements 32q .. 32q+31 of the
// step's group i,
// i.e. output bytes LB * lane .. LB * lane + LB - 1 of the step (LB = 128 for
// float32, 64 for bf16).  Its codes are the lane's 4 * SB bytes at offset
// 4 * SB * lane of the step's packed bytes (one coalesced load for the wave),
// stages 1-2 (2-bit) or 1 (4-bit) come from the byte table (3-bit fields:
// one lookup per element in an 8-entry table, no stage), the remaining
// in-lane stages run in registers and stages 6-7 across the quad
// (quad_butterfly_across).  These are the float32 operations, in the same
// order, of the seven butterfly stages run over one lane's 128 values.
//
// The step's output (8 or 4 KiB) is transposed through a wave-private LDS
// buffer so that store k writes bytes 1024k .. 1024k+1023 of the step:
// consecutive lanes, consecutive 16 bytes, whole 128-byte lines.  (Each lane
// storing its own bytes in 16-byte pieces leaves every instruction with 64
// partial lines, and under the streaming policy of these stores that
// ran 16 times slower.)  Chunk c of lane l sits at slot c ^ swz(l) of the
// lane's LB bytes, so eight consecutive lanes touch eight different 16-byte
// bank groups on both sides of the transpose.
//
// One step per wave, in blocks of 16 KiB of output: two waves for float32,
// four for bf16.  On the 7B-shaped model (26.4 GB of float32 output)
// 4.60-4.65 ms against 4.76 for a kernel with one lane per group and 32 KiB
// per wave; blocks of 3 or 4 waves took 4.83-4.88 ms, two steps per wave
// 4.94, one-wave blocks 5.7, a capped grid looping over steps 5.65.  bf16
// output: 2.78-2.80 ms in 4-wave blocks, 2.95-2.97 in 2-wave ones.  For
// float32 the LDS (20 KiB per block) sets the occupancy at 16 waves per CU.
//
// MANY: a table of tensors whose 64-group batches are numbered consecutively
// (the numbering quantize's multi-tensor launch uses too); step s is quarter
// s % 4 of batch s / 4, and quarters past a tensor's last group are skipped.
// Waves per block: 16 KiB of output per block (two 8 KiB float32 steps or
// four 4 KiB bf16 steps) was the fastest shape for both output types.
constexpr int quad_waves(bool bf16out) { return bf16out ? 4 : 2; }
// Grid cap of the quad kernel; larger calls loop (grid-stride).
constexpr int64_t kMaxGridBlocks = int64_t{1} << 30;

template <int SB, bool BF16OUT, bool MANY, bool TRITS = false>
__global__ void __launch_bounds__(quad_waves(BF16OUT) * kWave)
dequantize_quad_contig(DequantJob job, LevelTable lv) {
  static_assert(SB >= 2 && SB <= 4, "2-, 3- and 4-bit fields");
  static_assert(!TRITS || SB == 2, "trit storage decodes to 2-bit fields");
#if defined(__HIP_DEVICE_COMPILE__)  // buffer builtins exist only for the GPU target
  constexpr int E = SB == 3 ? 1 : ByteTable<SB>::E;  // elements per table read
  constexpr int QB = 4 * SB;                 // packed bytes per lane
  constexpr int OB = BF16OUT ? 2 : 4;        // output bytes per element
  constexpr int LB = kQuadElems * OB;        // output bytes per lane
  constexpr int CPL = LB / 16;               // 16-byte chunks per lane
  constexpr int STEP = kWave * LB;           // output bytes per step
  constexpr int NS = STEP / 1024;            // store instructions per step
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ __attribute__((aligned(16))) float tab[TableSize<SB>::floats];
  constexpr int W = quad_waves(BF16OUT);
  __shared__ __attribute__((aligned(16))) uint8_t stage[W * STEP];
  __shared__ uint16_t ttab[TRITS ? 256 : 1];
  for (int t = threadIdx.x; t < 256; t += blockDim.x) {
    if constexpr (TRITS) fill_trit_table(ttab, t);
    fill_table<SB>(tab, lv, t);
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), q = lane & 3;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  uint8_t* const buf = stage + wave * STEP;
  // Bank-group swizzle of a lane's chunks (see above).
  auto swz = [](int l) __attribute__((always_inline)) { return BF16OUT ? (l >> 2) & 3 : l & 7; };
  const int64_t n_steps = MANY ? 4 * job.n_batches : (job.n_groups + kQuadGroups - 1) / kQuadGroups;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * W;
  for (int64_t step = static_cast<int64_t>(blockIdx.x) * W + wave; step < n_steps;
       step += stride) {
    const uint8_t* pk = job.packed;
    const uint16_t* nm = job.norms;
    uint8_t* o = job.out;
    int64_t g0 = step * kQuadGroups, ng = job.n_groups;
    if constexpr (MANY) {
      const int64_t b = step >> 2;
      const int d = find_unit(job.t.start, 0, job.t.n, b);
      const DequantDesc* qd = job.t.desc + d;  // field by field: scalar loads
      pk = load_const(&qd->packed);
      nm = load_const(&qd->norms);
      o = load_const(&qd->out);
      ng = load_const(&qd->rows) * (load_const(&qd->cols) / kGroup);
      g0 = (b - load_const(job.t.start + d)) * kWave + (step & 3) * kQuadGroups;
      if (g0 >= ng) continue;  // a quarter past the tensor's partial last batch
    }
    const int64_t left = ng - g0;
    const int nv = left < kQuadGroups ? static_cast<int>(left) : kQuadGroups;
    // Lanes of groups past the end read zeros (outside the buffer resource)
    // and their stores are dropped.
    uint32_t words[SB];
    if constexpr (TRITS) {
      // Trit storage (26 bytes per group, 2-byte aligned): every lane of the
      // quad converts its group's 26 bytes to the 256 bits of 2-bit fields
      // and keeps the 64 bits of its quarter.
      const auto src = make_rsrc(pk + g0 * kTritBytes, nv * kTritBytes);
      uint32_t tr[13], all[8];
#pragma unroll
      for (int k = 0; k < 13; ++k) tr[k] = __builtin_amdgcn_raw_buffer_load_b16(src, (lane >> 2) * kTritBytes + 2 * k, 0, 0);
      trits_to_fields(tr, ttab, all);
      words[0] = q == 0 ? all[0] : q == 1 ? all[2] : q == 2 ? all[4] : all[6];
      words[1] = q == 0 ? all[1] : q == 1 ? all[3] : q == 2 ? all[5] : all[7];
    } else if constexpr (SB == 2) {
      const auto src = make_rsrc(pk + g0 * (16 * SB), nv * (16 * SB));
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(src, lane * QB, 0, 0);
      words[0] = v.x;
      words[1] = v.y;
    } else if constexpr (SB == 3) {
      const auto src = make_rsrc(pk + g0 * (16 * SB), nv * (16 * SB));
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(src, lane * QB, 0, 0);
      words[0] = v.x;
      words[1] = v.y;
      words[2] = v.z;
    } else {
      const auto src = make_rsrc(pk + g0 * (16 * SB), nv * (16 * SB));
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(src, lane * QB, 0, 0);
      words[0] = v.x;
      words[1] = v.y;
      words[2] = v.z;
      words[3] = v.w;
    }
    const auto nsrc = make_rsrc(nm + g0, nv * 2);
    const uint16_t n16 = __builtin_amdgcn_raw_buffer_load_b16(nsrc, (lane >> 2) * 2, 0, 0);
    float y[kQuadElems];
#pragma unroll
    for (int k = 0; k < kQuadElems / E; ++k) {
      if constexpr (SB == 3) {  // element k's field at bit 3k of the lane's 96 bits; an 8-entry table
        const int pos = 3 * k, wd = pos >> 5, off = pos & 31;
        uint32_t v = words[wd] >> off;
        if (off > 29) v |= words[wd + 1] << (32 - off);
        y[k] = tab[v & 7u];
        continue;
      }
      const uint32_t b = (words[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      if constexpr (E == 4) {
        const float4 v = *reinterpret_cast<const float4*>(tab + 4 * b);
        y[4 * k] = v.x;
        y[4 * k + 1] = v.y;
        y[4 * k + 2] = v.z;
        y[4 * k + 3] = v.w;
      } else {
        const float2 v = *reinterpret_cast<const float2*>(tab + 2 * b);
        y[2 * k] = v.x;
        y[2 * k + 1] = v.y;
      }
    }
    quad_butterfly_in_lane<E>(y);
    quad_butterfly_across<1>(y, q);
    quad_butterfly_across<2>(y, q);
    const float sc = half_to_float(n16) * (1.0f / kGroup);
    uint4 ch[CPL];
    if constexpr (BF16OUT) {
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w[i] = f32_to_bf16_rne(y[8 * c + 2 * i] * sc) | (f32_to_bf16_rne(y[8 * c + 2 * i + 1] * sc) << 16);
        ch[c] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        ch[c] = make_uint4(__builtin_bit_cast(uint32_t, y[4 * c] * sc), __builtin_bit_cast(uint32_t, y[4 * c + 1] * sc),
                           __builtin_bit_cast(uint32_t, y[4 * c + 2] * sc),
                           __builtin_bit_cast(uint32_t, y[4 * c + 3] * sc));
    }
    const auto dst = make_rsrc(o + g0 * (kGroup * OB), nv * (kGroup * OB));
    const int sw = swz(lane);
#pragma unroll
    for (int c = 0; c < CPL; ++c) *reinterpret_cast<uint4*>(buf + lane * LB + 16 * (c ^ sw)) = ch[c];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int sl = (1024 * k + 16 * lane) / LB, cl = lane % CPL;  // source lane and chunk
      const uint4 v = *reinterpret_cast<const uint4*>(buf + sl * LB + 16 * (cl ^ swz(sl)));
      store16<kStoreStream>(v, dst, static_cast<uint32_t>(16 * lane), static_cast<uint32_t>(1024 * k));
    }
    // The next step's LDS writes come after these reads in the wave's LDS
    // order; the wait only keeps the written registers live (see
    // hold_until_lds_written).
    hold_until_lds_written(ch);
  }
#endif
}

// Blocks of the quad kernel for n_steps steps: one step per wave.
inline int quad_grid(int64_t n_steps, bool bf16out) {
  const int w = quad_waves(bf16out);
  const int64_t want = (n_steps + w - 1) / w;
  return static_cast<int>(want < 1 ? 1 : want < kMaxGridBlocks ? want : kMaxGridBlocks);
}

template <int SB, bool BF16OUT, bool TRITS>
hipError_t launch_sb(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols,
                     const LevelTable& lv, void* out, hipStream_t s) {
  uint8_t* ob = static_cast<uint8_t*>(out);
  if (cols % kGroup == 0) {
    const int64_t n_groups = rows * (cols / kGroup);
    const int64_t n_steps = (n_groups + kQuadGroups - 1) / kQuadGroups;
    const DequantJob job{packed, norms, ob, n_groups, TensorTable<DequantDesc>{nullptr, nullptr, 0}, 0};
    hipLaunchKernelGGL((dequantize_quad_contig<SB, BF16OUT, false, TRITS>), dim3(quad_grid(n_steps, BF16OUT)),
                       dim3(quad_waves(BF16OUT) * kWave), 0, s, job, lv);
  } else {
    const int blocks = quad_blocks(rows * ((cols + kGroup - 1) / kGroup));
    const TensorTable<DequantDesc> none{nullptr, nullptr, 0};
    if (cols % wide_elems(BF16OUT) == 0)  // whole 16-byte pieces (the output is 16-byte aligned)
      hipLaunchKernelGGL((dequantize_ragged<SB, BF16OUT, false, TRITS, true>), dim3(blocks), dim3(kWave), 0, s,
                         packed, norms, rows, cols, lv, ob, none, int64_t{0});
    else
      hipLaunchKernelGGL((dequantize_ragged<SB, BF16OUT, false, TRITS, false>), dim3(blocks), dim3(kWave), 0, s,
                         packed, norms, rows, cols, lv, ob, none, int64_t{0});
  }
  return hipGetLastError();
}

template <int SB, bool BF16OUT, bool TRITS>
hipError_t launch_many_sb(const LevelTable& lv, TensorTable<DequantDesc> contig, int64_t contig_batches,
                          TensorTable<DequantDesc> ragged, int64_t ragged_groups, int64_t ragged_cols_gcd,
                          hipStream_t s) {
  if (contig_batches > 0) {
    const DequantJob job{nullptr, nullptr, nullptr, 0, contig, contig_batches};
    hipLaunchKernelGGL((dequantize_quad_contig<SB, BF16OUT, true, TRITS>), dim3(quad_grid(4 * contig_batches, BF16OUT)),
                       dim3(quad_waves(BF16OUT) * kWave), 0, s, job, lv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ragged_groups > 0) {
    const int blocks = quad_blocks(ragged_groups);
    if (ragged_cols_gcd % wide_elems(BF16OUT) == 0)  // every ragged width, so their gcd
      hipLaunchKernelGGL((dequantize_ragged<SB, BF16OUT, true, TRITS, true>), dim3(blocks), dim3(kWave), 0, s,
                         nullptr, nullptr, int64_t{0}, int64_t{0}, lv, nullptr, ragged, ragged_groups);
    else
      hipLaunchKernelGGL((dequantize_ragged<SB, BF16OUT, true, TRITS, false>), dim3(blocks), dim3(kWave), 0, s,
                         nullptr, nullptr, int64_t{0}, int64_t{0}, lv, nullptr, ragged, ragged_groups);
  }
  return hipGetLastError();
}

template <int SB, bool TRITS = false>
hipError_t launch_many_out(const LevelTable& lv, bool bf16_out, TensorTable<DequantDesc> contig,
                           int64_t contig_batches, TensorTable<DequantDesc> ragged, int64_t ragged_groups,
                           int64_t ragged_cols_gcd, hipStream_t s) {
  return bf16_out
             ? launch_many_sb<SB, true, TRITS>(lv, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, s)
             : launch_many_sb<SB, false, TRITS>(lv, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, s);
}

template <int SB, bool TRITS = false>
hipError_t launch_out(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols,
                      const LevelTable& lv, void* out, bool bf16_out, hipStream_t s) {
  return bf16_out ? launch_sb<SB, true, TRITS>(packed, norms, rows, cols, lv, out, s)
                  : launch_sb<SB, false, TRITS>(packed, norms, rows, cols, lv, out, s);
}

}  // namespace kd

// sbits: 2, 3 or 4; kTritStorage: five ternary indices per byte.
hipError_t launch_dequantize(const uint8_t* packed, const uint16_t* norms, int64_t rows,
                             int64_t cols, int sbits, const LevelTable& lv, void* out,
                             bool bf16_out, hipStream_t stream) {
  switch (sbits) {
    case 2: return kd::launch_out<2>(packed, norms, rows, cols, lv, out, bf16_out, stream);
    case 3: return kd::launch_out<3>(packed, norms, rows, cols, lv, out, bf16_out, stream);
    case 4: return kd::launch_out<4>(packed, norms, rows, cols, lv, out, bf16_out, stream);
    case kTritStorage: return kd::launch_out<2, true>(packed, norms, rows, cols, lv, out, bf16_out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequantize_many(int sbits, const LevelTable& lv, bool bf16_out,
                                  TensorTable<DequantDesc> contig, int64_t contig_batches,
                                  TensorTable<DequantDesc> ragged, int64_t ragged_groups,
                                  int64_t ragged_cols_gcd, hipStream_t stream) {
  switch (sbits) {
    case 2: return kd::launch_many_out<2>(lv, bf16_out, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd,
                                         stream);
    case 3: return kd::launch_many_out<3>(lv, bf16_out, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd,
                                         stream);
    case 4: return kd::launch_many_out<4>(lv, bf16_out, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd,
                                         stream);
    case kTritStorage:
      return kd::launch_many_out<2, true>(lv, bf16_out, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd,
                                         stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cq
