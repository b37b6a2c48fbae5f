// Internal interface between the host library (libcq_host.cpp) and the
// kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/libcq.h"

namespace cq {

constexpr int kGroup = 128;       // elements per group
constexpr int kWave = 64;         // lanes per wavefront (gfx950)
constexpr int kMaxLevels = 16;

// Per-call constants of the quantize kernels, derived on the host from the
// float32 levels.  Thresholds are midpoints of neighbouring float32 levels,
// computed in double and rounded once to float32.  They are in z units
// (z = rotated value / group norm * sqrt(G) = unnormalised butterfly output /
// group norm), so the kernels compare the unnormalised butterfly output Y
// against threshold * norm.
struct QuantParams {
  float thr[kMaxLevels - 1];  // L-1 thresholds (binary-search widths: L = 8, 16)
  // Two-compare decision for L = 3 and L = 4 (see quantize.hip):
  float mu;     // centre of the outer pair of thresholds
  float delta;  // half distance between the outer pair
  float hmid;   // L = 4: middle threshold minus mu; L = 3: delta
  int n_levels;
  // Symmetric decisions (quantize.hip, shift_in_pair): 1 when the middle
  // threshold is the centre of the outer pair (three levels always; four
  // levels when hmid == 0), with neg2_over_delta = -2 / delta.
  int sym;
  float neg2_over_delta;
};

struct LevelTable {
  float c[kMaxLevels];  // float32 levels in N(0,1) units; entries >= n_levels are 0
  int n_levels;
};

// lv.c[i] for a per-thread index i, by an unrolled select over constant
// indices: the levels stay in scalar registers (a dynamic index into the
// kernel-argument struct would become serialized memory loads).
__device__ __forceinline__ float level_at(const LevelTable& lv, int i) {
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxLevels; ++j) v = (i == j) ? lv.c[j] : v;
  return v;
}

// ---- Ternary trit storage ------------------------------------------------------
//
// A 128-group of ternary indices (0, 1, 2) is stored in 26 bytes: index j is
// base-3 digit j % 5 of byte j / 5, least significant digit first (the last
// byte holds indices 125..127).  In registers the same group is either eight
// dwords of 2-bit fields (index j at bits 2 (j % 16) of word j / 16, the
// layout of the 2-bit kernels) or 13 dwords holding two trit bytes each in
// their low 16 bits.
constexpr int kTritBytes = 26;
constexpr int kTritStorage = 5;  // storage code of the dequantize launchers for trits

// 2-bit fields -> trit bytes (13 values of two bytes; Horner from the top
// digit, all positions compile-time).
__device__ __forceinline__ void fields_to_trits(const uint32_t (&w)[8], uint32_t (&t)[13]) {
#pragma unroll
  for (int k = 0; k < 13; ++k) {
    uint32_t pair = 0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int b = 2 * k + half;
      uint32_t v = 0;
#pragma unroll
      for (int i = 4; i >= 0; --i) {
        const int j = 5 * b + i;
        if (j < kGroup) v = v * 3u + ((w[j / 16] >> (2 * (j % 16))) & 3u);
      }
      pair |= v << (8 * half);
    }
    t[k] = pair;
  }
}

// Entry b of the 256-entry trit table: the five base-3 digits of b as 2-bit
// fields (digit i at bits 2i).  Bytes above 242 never come from a
// quantizer; they map to some in-range fields.
__device__ __forceinline__ uint32_t trit_table_entry(uint32_t b) {
  uint32_t f = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    f |= (b % 3u) << (2 * i);
    b /= 3u;
  }
  return f;
}

// Trit bytes -> 2-bit fields through the LDS table `tab`.  Byte b's fields
// land at bit 10 b of the group's 256-bit field stream.
__device__ __forceinline__ void trits_to_fields(const uint32_t (&t)[13], const uint16_t* tab,
                                                uint32_t (&w)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = 0u;
#pragma unroll
  for (int b = 0; b < kTritBytes; ++b) {
    const uint32_t f = tab[(t[b / 2] >> (8 * (b % 2))) & 0xFFu];
    const int pos = 10 * b, wi = pos / 32, sh = pos % 32;
    w[wi] |= f << sh;
    if (sh > 22 && wi + 1 < 8) w[wi + 1] |= f >> (32 - sh);
  }
}

// Ternary 2-bit fields <-> trit storage for n_groups groups of group_size
// (32, 64, 128, 256) indices (to_trits: src holds fields).
hipError_t launch_repack(const uint8_t* src, bool to_trits, uint8_t* dst, int64_t n_groups, int group_size,
                         hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

// Chunks a wave has just stored to LDS (a ds_write_b128 each) keep their
// registers until the LDS has taken them.  Measured on gfx950: with the bf16
// output of dequantize at 3 bits, the compiler reused the first data
// register of each ds_write_b128 in the very next instruction, and the store
// now and then took the new value (zeros in the first dword of some 16-byte
// chunks, different ones from run to run).  Waiting for the wave's LDS
// operations (lgkmcnt(0)), with the registers named as inputs of asm
// statements placed after the wait, rules that out: the registers cannot be
// reused before the wait, and after it the writes are done.
template <int N>
__device__ __forceinline__ void hold_until_lds_written(const uint4 (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"v"(v[i].x), "v"(v[i].y), "v"(v[i].z), "v"(v[i].w));
}

// The same for 32-bit values (table fills): wait for the wave's LDS writes,
// then name the stored values, so their registers outlive the writes.
__device__ __forceinline__ void wait_lds_writes() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <typename T>
__device__ __forceinline__ void hold_value(const T& v) {
  asm volatile("" ::"v"(v));
}
template <typename... T>
__device__ __forceinline__ void hold_values(const T&... v) {
  (hold_value(v), ...);
}

// Blocks of a launch are handed to the 8 XCDs in turn (block b runs on XCD
// b % 8, each XCD with its own L2).  xcd_block renumbers the blocks of the
// complete rounds of 8 so that consecutive numbers run on one XCD: XCD x
// takes numbers x * n8 .. x * n8 + n8 - 1 (n8 = blocks / 8, rounded down);
// the last blocks keep their numbers.  A kernel that hands out work by this
// number keeps neighbouring work units in one L2.
__device__ __forceinline__ int xcd_block(int b, int n) {
  const int full = n & ~7;
  if (b >= full) return b;
  return (b & 7) * (full >> 3) + (b >> 3);
}

// ---- Ragged rows: one group over a quad of lanes ---------------------------------
//
// Where a row's length is not a multiple of 128, groups start anywhere and
// the last group of each row is partial (zero-padded on input, its padding
// dropped on output: "Cactus Quants CQ2-bit Quantization: Extreme
// Compression for Edge LLMs", section Group-wise Weight Partitioning).  The
// kernels for such tensors give a group to a quad of four consecutive
// lanes: lane q of the quad holds elements 32q .. 32q+31.  Butterfly stages
// with pair distances 1..16 then stay inside a lane's registers, and the
// stages with distances 32 and 64 pair lane q with lanes q^1 and q^2 of the
// same quad (DPP quad permutes, no LDS).  A wave covers 16 groups, so a
// small tensor spreads over four times as many waves as with one lane per
// group, each doing a quarter of the arithmetic.

constexpr int kQuadElems = kGroup / 4;  // elements per lane
constexpr int kQuadGroups = kWave / 4;  // groups per wave

// Value of lane (lane ^ X) of the same quad, X = 1 or 2: DPP quad_perm
// [1,0,3,2] (0xB1) or [2,3,0,1] (0x4E).  Every lane of the quad must be active.
// bound_ctrl: a lane whose source is inactive would read 0, so the move needs
// no old value (which would cost a register clear per exchange); within an
// active quad every source lane exists.
template <int X>
__device__ __forceinline__ float quad_xor(float v) {
  static_assert(X == 1 || X == 2, "quad lanes differ in bit 0 or bit 1");
  constexpr int kCtrl = X == 1 ? 0xB1 : 0x4E;
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}

// Word held by lane K of the quad (quad_perm [K,K,K,K]).
template <int K>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x55 * K, 0xF, 0xF, false));
}

// Butterfly stages with pair distances H0, 2 H0, ..., 16 over a lane's 32
// elements.
template <int H0>
__device__ __forceinline__ void quad_butterfly_in_lane(float (&y)[kQuadElems]) {
#pragma unroll
  for (int h = H0; h < kQuadElems; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kQuadElems; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
    }
  }
}

// Butterfly stage of pair distance 32 X across the quad.  The lane with bit
// X of q clear holds a and takes a + b; its partner holds b and takes a - b
// (fma(-1, b, a) is the rounded a - b), the same operations as in one lane.
template <int X>
__device__ __forceinline__ void quad_butterfly_across(float (&y)[kQuadElems], int q) {
  const float sgn = (q & X) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < kQuadElems; ++j) y[j] = __builtin_fmaf(sgn, y[j], quad_xor<X>(y[j]));
}

// Sum of v over the quad, the same value (bit for bit) in all four lanes:
// (v0 + v1) + (v2 + v3) in every lane, as float addition commutes.
__device__ __forceinline__ float quad_sum(float v) {
  v += quad_xor<1>(v);
  return v + quad_xor<2>(v);
}

// Group gl of a tensor with `cols` columns: index of its first element and
// how many of its 128 elements exist (1..128).
struct QuadPlace {
  int64_t first;
  int valid;
};
__device__ __forceinline__ QuadPlace quad_place(int64_t gl, int64_t cols) {
  const int64_t ngr = (cols + kGroup - 1) / kGroup;
  int64_t row, gi;
  if (gl <= 0xFFFFFFFFll && ngr <= 0xFFFFFFFFll) {  // 32-bit division when it fits
    const uint32_t r = static_cast<uint32_t>(gl) / static_cast<uint32_t>(ngr);
    row = r;
    gi = gl - static_cast<int64_t>(r) * ngr;
  } else {
    row = gl / ngr;
    gi = gl - row * ngr;
  }
  const int64_t col0 = gi * kGroup, left = cols - col0;
  return QuadPlace{row * cols + col0, left < kGroup ? static_cast<int>(left) : kGroup};
}

// Elements 32q .. 32q+31 of a group (first element `first`, `valid` of them
// exist) as float32, the missing ones 0.  WIDE: 16-byte loads; the caller
// guarantees a 16-byte aligned base and cols a multiple of 16 / element
// bytes, so every 16-byte piece lies in one row and exists whole or not at
// all.  Otherwise one load per element.  Addresses of missing pieces are
// clamped to the group's first element, so all loads issue unconditionally;
// the zero fill follows them.
template <bool BF16, bool WIDE>
__device__ __forceinline__ void quad_load(const uint8_t* __restrict__ w, int64_t first, int valid, int q,
                                          float (&x)[kQuadElems]) {
  constexpr int EB = BF16 ? 2 : 4;
  const int vq = valid - kQuadElems * q;
  const int64_t mine = first + kQuadElems * q;
  if constexpr (WIDE) {
    constexpr int VW = 16 / EB;  // elements per load
    constexpr int NL = kQuadElems / VW;
    uint4 raw[NL];
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      const int64_t e = VW * c < vq ? mine + VW * c : first;
      raw[c] = *reinterpret_cast<const uint4*>(w + e * EB);
    }
#pragma unroll
    for (int c = 0; c < NL; ++c) {
      const uint32_t u[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
      const bool in = VW * c < vq;
#pragma unroll
      for (int k = 0; k < VW; ++k) {
        uint32_t bits;
        if constexpr (BF16)
          bits = k & 1 ? u[k / 2] & 0xFFFF0000u : u[k / 2] << 16;
        else
          bits = u[k];
        x[VW * c + k] = in ? __builtin_bit_cast(float, bits) : 0.0f;
      }
    }
  } else {
    uint32_t raw[kQuadElems];
#pragma unroll
    for (int m = 0; m < kQuadElems; ++m) {
      const int64_t e = m < vq ? mine + m : first;
      if constexpr (BF16)
        raw[m] = static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(w)[e]) << 16;
      else
        raw[m] = reinterpret_cast<const uint32_t*>(w)[e];
    }
#pragma unroll
    for (int m = 0; m < kQuadElems; ++m) x[m] = m < vq ? __builtin_bit_cast(float, raw[m]) : 0.0f;
  }
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Writes the existing ones of elements 32q .. 32q+31 of a group (see
// quad_load for WIDE), float32 or bf16 (round to nearest even).
template <bool BF16, bool WIDE>
__device__ __forceinline__ void quad_store(uint8_t* __restrict__ out, int64_t first, int valid, int q,
                                           const float (&y)[kQuadElems]) {
  constexpr int EB = BF16 ? 2 : 4;
  const int vq = valid - kQuadElems * q;
  const int64_t mine = first + kQuadElems * q;
  if constexpr (WIDE) {
    constexpr int VW = 16 / EB;
#pragma unroll
    for (int c = 0; c < kQuadElems / VW; ++c) {
      uint32_t u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (BF16)
          u[k] = bf16_bits_rne(y[VW * c + 2 * k]) | (bf16_bits_rne(y[VW * c + 2 * k + 1]) << 16);
        else
          u[k] = __builtin_bit_cast(uint32_t, y[VW * c + k]);
      }
      if (VW * c < vq) *reinterpret_cast<uint4*>(out + (mine + VW * c) * EB) = make_uint4(u[0], u[1], u[2], u[3]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < kQuadElems; ++m) {
      if (m < vq) {
        if constexpr (BF16)
          reinterpret_cast<uint16_t*>(out)[mine + m] = static_cast<uint16_t>(bf16_bits_rne(y[m]));
        else
          reinterpret_cast<float*>(out)[mine + m] = y[m];
      }
    }
  }
}

// Elements per 16-byte piece of the WIDE forms: 8 (bf16) or 4 (float32).
constexpr int64_t wide_elems(bool bf16) { return bf16 ? 8 : 4; }

// Blocks (one wave each) of a ragged kernel over n_groups groups: one 16-group
// step per wave up to eight waves per CU, then a grid-stride loop.
inline int quad_blocks(int64_t n_groups) {
  const int64_t steps = (n_groups + kQuadGroups - 1) / kQuadGroups;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * 8;
  return static_cast<int>(steps < cap ? (steps > 0 ? steps : 1) : cap);
}

// Blocks of `waves` waves for a grid-stride kernel over n_batches batches in
// which each wave takes about `per_wave` batches, but never fewer than one
// batch per wave gives up to per_cu resident blocks per CU, so a mid-size
// tensor still reaches every CU.
inline int spread_blocks(int64_t n_batches, int waves, int per_wave, int per_cu) {
  const int64_t w = waves;
  const int64_t spread = (n_batches + w * per_wave - 1) / (w * per_wave);
  const int64_t one = (n_batches + w - 1) / w;
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
  const int64_t fill = one < cap ? one : cap;
  const int64_t b = spread > fill ? spread : fill;
  return static_cast<int>(b > 0 ? b : 1);
}

// Grid of a contiguous kernel: blocks and waves per block (the kernel reads
// its waves per block from blockDim).  With at least W batches per CU the
// blocks have W waves (spread_blocks); a smaller call gets blocks of
// ceil(batches / CUs) waves, one batch per wave, so that it spreads over as
// many CUs as it has batches.
struct ContigGrid {
  int blocks;
  int waves;
};
inline ContigGrid contig_grid(int64_t n_batches, int W, int per_wave, int per_cu) {
  const int64_t cus = device_cu_count();
  if (n_batches >= W * cus) return ContigGrid{spread_blocks(n_batches, W, per_wave, per_cu), W};
  const int w = n_batches > cus ? static_cast<int>((n_batches + cus - 1) / cus) : 1;  // 1 .. W
  return ContigGrid{static_cast<int>(n_batches > 0 ? (n_batches + w - 1) / w : 1), w};
}

// Launchers (return hipError_t of the launch).  All sizes already validated.
// trits: store the three-level code five indices per byte (26 B per group).
hipError_t launch_quantize(const void* w, bool bf16, bool trits, int64_t rows, int64_t cols,
                           const QuantParams& p, uint8_t* packed, uint16_t* norms,
                           hipStream_t stream);

hipError_t launch_fake_quant(const void* w, bool bf16_in, int64_t rows, int64_t cols,
                             const QuantParams& p, const LevelTable& lv, void* out, bool bf16_out,
                             hipStream_t stream);

hipError_t launch_dequantize(const uint8_t* packed, const uint16_t* norms,
                             int64_t rows, int64_t cols, int sbits,
                             const LevelTable& lv, void* out, bool bf16_out,
                             hipStream_t stream);

// Group sizes 32, 64 and 256 (single-tensor codec calls; one or four lanes
// per group).
hipError_t launch_quantize_g(int group_size, const void* w, bool bf16, int64_t rows, int64_t cols,
                             const QuantParams& p, uint8_t* packed, uint16_t* norms, hipStream_t stream);
hipError_t launch_dequantize_g(int group_size, const uint8_t* packed, const uint16_t* norms, int64_t rows,
                               int64_t cols, int sbits, const LevelTable& lv, void* out, bool bf16_out,
                               hipStream_t stream);
hipError_t launch_fake_quant_g(int group_size, const void* w, bool bf16, int64_t rows, int64_t cols,
                               const QuantParams& p, const LevelTable& lv, void* out, bool bf16_out,
                               hipStream_t stream);

// ---- Multi-tensor codec calls ----------------------------------------------

// One tensor of a multi-tensor quantize / dequantize call (device-side
// descriptors, 40 bytes each).
struct QuantDesc {
  const uint8_t* w;  // rows x cols input (f32 or bf16)
  uint8_t* packed;
  uint16_t* norms;
  int64_t rows, cols;
};
struct DequantDesc {
  const uint8_t* packed;
  const uint16_t* norms;
  uint8_t* out;  // rows x cols output (f32 or bf16)
  int64_t rows, cols;
};

// A device table of n descriptors plus the prefix start[0..n] of their work
// units (64-group batches on the fast path, groups on the ragged path):
// descriptor d owns units [start[d], start[d+1]).
template <class D>
struct TensorTable {
  const D* desc;
  const int64_t* start;
  int n;
};

// Read-only table entry read through the constant address space: with a
// wave-uniform address this is a scalar load (tracked apart from the vector
// memory counter, so it never waits for the wave's loads and stores in
// flight); with a per-lane address the compiler falls back to a vector load.
template <class T>
__device__ __forceinline__ T load_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Last d in [lo, n) with start[d] <= v (start ascending, start[lo] <= v <
// start[n]).
__device__ __forceinline__ int find_unit(const int64_t* __restrict__ start, int lo, int n, int64_t v) {
  int hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (load_const(start + mid) <= v)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// Copies `bytes` (a multiple of 4) host bytes to device memory at dst with
// kernel launches that carry them as arguments: asynchronous, and the host
// buffer may be reused as soon as the call returns.
hipError_t upload(const void* src, size_t bytes, void* dst, hipStream_t stream);

// ragged_cols_gcd: gcd of the ragged tensors' column counts (picks the
// 16-byte load / store form where every width allows it).
hipError_t launch_quantize_many(bool bf16, bool trits, const QuantParams& p, TensorTable<QuantDesc> contig,
                                int64_t contig_batches, TensorTable<QuantDesc> ragged,
                                int64_t ragged_groups, int64_t ragged_cols_gcd, hipStream_t stream);

hipError_t launch_dequantize_many(int sbits, const LevelTable& lv, bool bf16_out,
                                  TensorTable<DequantDesc> contig, int64_t contig_batches,
                                  TensorTable<DequantDesc> ragged, int64_t ragged_groups,
                                  int64_t ragged_cols_gcd, hipStream_t stream);

// One matrix of a dequant-matvec call (device-side descriptor).
struct MatvecDesc {
  const uint8_t* packed;  // [n_out][k / 128][128 * sbits / 8]
  const uint16_t* norms;  // [n_out][k / 128]
  const float* x;         // [batch][k]
  float* y;               // [batch][n_out]
  int64_t n_out;
  int64_t k;
  int64_t xr_offset;      // float offset of this matrix's rotated x in the workspace
};

// Descriptors are written to device memory by a small kernel that receives
// them as kernel arguments, kDescPerInit at a time (no host-to-device copy,
// so the call stays asynchronous).  A chunk is 80 kDescPerInit + 40 bytes:
// 48 keeps it under 4 KiB of kernel arguments (5 launches for 225 matrices).
constexpr int kDescPerInit = 48;
struct DescChunk {
  MatvecDesc d[kDescPerInit];
  int64_t gstart[kDescPerInit + 1];   // rotate-kernel group prefix
  int64_t bstart0[kDescPerInit + 1];  // product-kernel block prefix, full batch chunks
  int64_t bstart1[kDescPerInit + 1];  // same, for the last (partial) batch chunk
  int count;                          // descriptors in this chunk
  int first;                          // index of d[0] in the table
  int last_chunk;                     // 1: also write the sentinel entries [count]
};
static_assert(sizeof(DescChunk) <= 4096, "kernel arguments stay within 4 KiB");

hipError_t launch_table_init(const DescChunk& c, MatvecDesc* table, int64_t* gstart,
                             int64_t* bstart0, int64_t* bstart1, hipStream_t stream);

// Product kernel for a batch chunk of nb rows of sbits-bit codes over the n
// matrices of descs (host array): its rows per block (the block prefix is
// built from it) and, for the pair-table kernel, its rows per wave (0: the
// byte-table kernel).  launch_matvec runs the kernel the plan names.
struct MatvecPlan {
  int rows_per_block;
  int pair_rows_per_wave;
  int mfma;  // 1: the matrix-core kernel (2 to 8 batch rows per launch)
  int mfma_pass;  // its pass width: 4096 columns (one block per CU) or 2048 (two)
};
MatvecPlan matvec_plan(int sbits, int nb, const MatvecDesc* descs, int n);
// Batch rows per product-kernel launch for a call of `batch` rows over the n
// matrices of descs: 1 where the pair-table kernel takes each row, else 8.
int matvec_chunk(int sbits, int64_t batch, const MatvecDesc* descs, int n);

// Activation rotations run one wave per 128-group when a call has fewer
// than this many groups (a thread per group would leave most CUs idle), else
// one thread per group (cheaper per group: no cross-lane traffic).
constexpr int64_t kFewUnits = 32768;

hipError_t launch_rotate(const MatvecDesc* table, const int64_t* gstart, int n, int64_t total_groups,
                         int group_size, float* xr, hipStream_t stream);

hipError_t launch_matvec(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks,
                         int sbits, const LevelTable& lv, const float* xr, int64_t b0, int nb,
                         const MatvecPlan& plan, int group_size, hipStream_t stream);

hipError_t launch_zero(float* y, int64_t count, hipStream_t stream);

// The matrix-core product over many matrices (matvec_rot.hip): activations
// rotated beforehand into xr, batch rows b0 .. b0 + nb - 1 (nb 1 .. 8), at
// most mfma_rows_cap(sbits, nb) rows per block, passes of pass_cols (4096 or
// 2048) columns.  A matrix qualifies when mfma_fits(k): k % 64 == 0 and
// k <= 2^26.
int mfma_rows_cap(int sbits, int nb);
bool mfma_fits(int64_t k);
hipError_t launch_mfma_many(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks, int sbits,
                            const LevelTable& lv, const float* xr, int64_t b0, int nb, int log2g,
                            int rows_per_block, int pass_cols, hipStream_t stream);

// The multi-matrix product (cq_dequant_matvec_many) with a stream-ordered
// workspace (fixed_ws == nullptr) or a fixed one of fixed_cap bytes whose
// device address fixed_ws returns, called only after validation and the
// size check; defined in libcq_host.cpp.
int matvec_many_impl(int n, const cq_matvec_desc* descs, int bits, int group_size, const float* levels,
                     int n_levels, int64_t batch, void* stream, int (*fixed_ws)(uint8_t**), size_t fixed_cap);
// Records a failure (status and message) for cq_last_error; returns status.
int report(int status, const char* msg);

// ---- Single-matrix dequant-matvec: one launch, no workspace ---------------------

// The matrix and activations of one product, passed by value as a kernel
// argument.
struct MatvecArgs {
  const uint8_t* packed;  // [n_out][k / G][G * sbits / 8]
  const uint16_t* norms;  // [n_out][k / G]
  const float* x;         // [batch][k]
  float* y;               // [batch][n_out]
  int64_t n_out;
  int64_t k;
  int64_t batch;
};

// Which kernel runs a single-matrix product: the pair-table kernel with
// pair_rows_per_block rows per block (1 .. 64; 2-bit fields only, one batch
// row per grid row), the matrix-core kernel with mfma_rows_per_block rows
// per block (1 .. 48; chunks of 4 or 8 batch rows), or (both 0) the
// per-lane-table kernel aiming at blocks_per_cu blocks per compute unit.
struct MatvecOnePlan {
  int pair_rows_per_block;
  int blocks_per_cu;
  int mfma_rows_per_block;
};

MatvecOnePlan matvec_one_plan(int sbits, int64_t n_out, int64_t k, int64_t batch);
hipError_t launch_matvec_one(const MatvecArgs& a, int sbits, const LevelTable& lv, int group_size,
                             const MatvecOnePlan& plan, hipStream_t stream);

// ---- Dequantize-GEMM on the matrix cores --------------------------------------

// One matrix of a GEMM call (device-side descriptor).
struct GemmDesc {
  const uint8_t* packed;  // [n_out][k / 128][128 * sbits / 8]
  const uint16_t* norms;  // [n_out][k / 128]
  const float* x;         // [batch][k]
  float* y;               // [batch][n_out]
  int64_t n_out;
  int64_t k;
  int64_t mpad;           // batch rounded up to the block's row count
  int64_t xs_off;         // bf16 offset of this matrix's split rotated x in the workspace
  float* part;            // [ksplit][batch][n_out] partial sums in the workspace, or null: write y
  int64_t ksplit;         // ranges of 128-groups along k, one block each per output tile
  int64_t gps;            // groups per range (the last may be shorter)
};

// Levels split into bf16 halves (bits in the low 16 bits): level = hi + lo
// up to 2^-16 relative.
struct SplitLevels {
  uint32_t hi[kMaxLevels];
  uint32_t lo[kMaxLevels];
};

int gemm_block_rows(int64_t batch, int group_size);  // batch rows per GEMM block (32 or 64)
int gemm_block_cols();  // outputs per GEMM block

// Workspace units: matrix d has (k / 128) * mpad rotate units, each writing
// 256 bf16 values.
hipError_t launch_split_rotate(const GemmDesc* table, const int64_t* ustart, int n, int64_t units,
                               int64_t batch, int group_size, uint16_t* ws, hipStream_t stream);

// y = sum over the k ranges of each matrix's partial sums, in range order;
// ostart: prefix of batch * n_out over the table's matrices.
hipError_t launch_gemm_reduce(const GemmDesc* table, const int64_t* ostart, int n, int64_t outputs,
                              int64_t batch, hipStream_t stream);

hipError_t launch_gemm(const GemmDesc* table, const int64_t* bstart, int n, int64_t blocks, int sbits,
                       const SplitLevels& sl, const uint16_t* ws, int64_t batch, int group_size,
                       hipStream_t stream);

}  // namespace cq
