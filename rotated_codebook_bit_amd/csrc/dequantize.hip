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
// Mapping: one lane owns one group (lookup, 7 butterfly stages and scaling in
// registers).  The 512-byte (fp32) or 256-byte (bf16) output of a lane is
// passed through a wave-private LDS buffer in four phases of 32 elements so
// that the HBM stores are issued as full 128-byte lines by consecutive lanes.
// Within a phase, 16-byte chunk c of group g sits in physical chunk slot
// c ^ s(g) with s chosen so that 16 consecutive lanes never share a bank.

#include "cq_internal.h"

namespace cq {
namespace kd {

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;
// Floor of the covering grid for mid-size tensors: one block per CU.
constexpr int kBlocksPerCu = 1;
// Waves per block of dequantize_contig: eight.  On the 7B-shaped model that
// was 1.6% faster than four for float32 output (at about 200 VGPRs a CU holds
// eight waves either way) and, with the covering grid, 6.6% faster than the
// resident grid of 4-wave blocks that bf16 output used before.
constexpr int contig_waves(bool) { return 2 * kWaves; }

__device__ __forceinline__ void butterfly(float (&y)[kGroup]) {
#pragma unroll
  for (int h = 1; h < kGroup; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kGroup; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
    }
  }
}

template <int SB>
__device__ __forceinline__ void load_indices(const uint8_t* __restrict__ packed, int64_t g,
                                             uint32_t (&words)[4 * SB]) {
  const uint4* src = reinterpret_cast<const uint4*>(packed + g * (16 * SB));
#pragma unroll
  for (int i = 0; i < SB; ++i) {
    const uint4 v = src[i];
    words[4 * i] = v.x;
    words[4 * i + 1] = v.y;
    words[4 * i + 2] = v.z;
    words[4 * i + 3] = v.w;
  }
}

template <int SB>
__device__ __forceinline__ uint32_t index_at(const uint32_t (&words)[4 * SB], int j) {
  const int pos = SB * j, wd = pos >> 5, off = pos & 31;
  uint32_t v = words[wd] >> off;
  if (off + SB > 32) v |= words[wd + 1] << (32 - off);
  return v & ((1u << SB) - 1u);
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Reconstruct one group into y (float32, already scaled), generic form:
// per-element level lookup, then the 7 butterfly stages.
template <int SB>
__device__ __forceinline__ void reconstruct(const uint32_t (&words)[4 * SB], uint16_t n16,
                                            const float* lut, float (&y)[kGroup]) {
#pragma unroll
  for (int j = 0; j < kGroup; ++j) y[j] = lut[index_at<SB>(words, j)];
  butterfly(y);
  const float s = half_to_float(n16) * (1.0f / kGroup);
#pragma unroll
  for (int j = 0; j < kGroup; ++j) y[j] *= s;
}

// Butterfly stages with pair distance >= h0 (the earlier ones are done).
template <int H0>
__device__ __forceinline__ void butterfly_from(float (&y)[kGroup]) {
#pragma unroll
  for (int h = H0; h < kGroup; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kGroup; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
    }
  }
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
  // Byte k (0..G*SB/8-1) of the group's packed bits.
  static __device__ __forceinline__ uint32_t byte_at(const uint32_t (&words)[4 * SB], int k) {
    return (words[k >> 2] >> (8 * (k & 3))) & 0xFFu;
  }
  static __device__ __forceinline__ void decode(const uint32_t (&words)[4 * SB], const float* tab,
                                                float (&y)[kGroup]) {
#pragma unroll
    for (int k = 0; k < kGroup / E; ++k) {
      const uint32_t b = byte_at(words, k);
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

template <int SB>
__device__ __forceinline__ void reconstruct_fast(const uint32_t (&words)[4 * SB], uint16_t n16,
                                                 const float* tab, float (&y)[kGroup]) {
  if constexpr (SB == 3) {
    reconstruct<SB>(words, n16, tab, y);
  } else {
    ByteTable<SB>::decode(words, tab, y);
    butterfly_from<ByteTable<SB>::E>(y);
    const float s = half_to_float(n16) * (1.0f / kGroup);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) y[j] *= s;
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Packed words and norm of every lane's group of batch bt (zeros past the
// end: buffer loads outside the resource return 0).
template <int SB>
__device__ __forceinline__ void fetch_batch(const uint8_t* __restrict__ packed,
                                            const uint16_t* __restrict__ norms, int64_t bt,
                                            int nv, int lane, uint32_t (&words)[4 * SB],
                                            uint16_t& n16) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer builtins exist only for the GPU target
  constexpr int PB = 16 * SB;  // packed bytes per group
  const auto src = make_rsrc(packed + bt * kWave * PB, nv * PB);
#pragma unroll
  for (int i = 0; i < SB; ++i) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(src, lane * PB + 16 * i, 0, 0);
    words[4 * i] = v.x;
    words[4 * i + 1] = v.y;
    words[4 * i + 2] = v.z;
    words[4 * i + 3] = v.w;
  }
  const auto nsrc = make_rsrc(norms + bt * kWave, nv * 2);
  n16 = __builtin_amdgcn_raw_buffer_load_b16(nsrc, lane * 2, 0, 0);
#endif
}

// Trit storage (three-level code, 26 bytes per group at 2-byte alignment):
// 13 16-bit loads per lane, one trit byte pair in each dword's low half.
__device__ __forceinline__ void fetch_batch_trits(const uint8_t* __restrict__ packed,
                                                  const uint16_t* __restrict__ norms, int64_t bt,
                                                  int nv, int lane, uint32_t (&t)[13], uint16_t& n16) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer builtins exist only for the GPU target
  const auto src = make_rsrc(packed + bt * kWave * kTritBytes, nv * kTritBytes);
#pragma unroll
  for (int k = 0; k < 13; ++k) t[k] = __builtin_amdgcn_raw_buffer_load_b16(src, lane * kTritBytes + 2 * k, 0, 0);
  const auto nsrc = make_rsrc(norms + bt * kWave, nv * 2);
  n16 = __builtin_amdgcn_raw_buffer_load_b16(nsrc, lane * 2, 0, 0);
#endif
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
// 2 = nt, 16 = sc1).  Float32 output is stored "nt sc1", streaming: on the
// 7B-shaped model that took dequantize from 5.18 to 4.92 ms (nt or sc1 alone:
// 5.05, sc0 sc1: 5.05).  Every policy bit made bf16 output slower (3.21 ms ->
// 4.07-4.55 ms), so it keeps the default.
constexpr int kStoreF32 = 2 | 16;

template <int AUX>
__device__ __forceinline__ void store16(const uint4& v, __amdgpu_buffer_rsrc_t dst, uint32_t voff,
                                        uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, dst, voff, soff, AUX);
#endif
}

// Fast path: cols % 128 == 0, so group g's output is 128 contiguous values.
// The next batch's packed words and norm are loaded into registers while the
// current batch is computed.  Stores go through a per-batch buffer resource
// so the lanes past the end of the last batch are dropped by the hardware.
//
// One launch covers one tensor (MANY = false) or a table of tensors whose
// column counts are multiples of 128 (MANY = true, batches of each tensor
// numbered consecutively).
struct DequantJob {
  const uint8_t* packed;
  const uint16_t* norms;
  uint8_t* out;
  int64_t n_groups;
  TensorTable<DequantDesc> t;
  int64_t n_batches;
};

// Inputs and output of one 64-group batch: local batch bt of a tensor with
// n_groups groups.
struct DBatch {
  const uint8_t* packed;
  const uint16_t* norms;
  uint8_t* out;
  int64_t bt;
  int64_t n_groups;
  __device__ int nvalid() const {
    const int64_t left = n_groups - bt * kWave;
    return static_cast<int>(left < kWave ? left : kWave);
  }
};

template <bool MANY>
__device__ __forceinline__ DBatch resolve(const DequantJob& j, int64_t b, int& d) {
  if constexpr (!MANY) {
    return DBatch{j.packed, j.norms, j.out, b, j.n_groups};
  } else {
    d = find_unit(j.t.start, d, j.t.n, b);
    const DequantDesc* q = j.t.desc + d;  // field by field: scalar loads
    return DBatch{load_const(&q->packed), load_const(&q->norms), load_const(&q->out),
                  b - load_const(j.t.start + d), load_const(&q->rows) * (load_const(&q->cols) / kGroup)};
  }
}

// TRITS (with SB = 2): the packed input is trit storage, converted to 2-bit
// fields in registers.
template <int SB, bool BF16OUT, bool MANY, bool TRITS = false>
__global__ void __launch_bounds__(contig_waves(BF16OUT) * kWave, 2)
dequantize_contig(DequantJob job, LevelTable lv) {
  constexpr int W = contig_waves(BF16OUT);
  constexpr int OB = BF16OUT ? 2 : 4;        // output bytes per element
  constexpr int GOB = kGroup * OB;           // output bytes per group
  constexpr int PB = 32 * OB;                // bytes per group per phase
  constexpr int CPP = PB / 16;               // 16-byte chunks per group per phase
  constexpr int GPB = 256 / PB;              // groups per 256-byte LDS row
  constexpr int GPI = kWave / CPP;           // groups per store instruction
  constexpr int WAVE_BYTES = kWave * PB;
  constexpr int NI = WAVE_BYTES / 1024;      // store instructions per phase
  __shared__ __attribute__((aligned(16))) float tab[TableSize<SB>::floats];
  __shared__ __attribute__((aligned(16))) uint8_t lds[W * WAVE_BYTES];
  __shared__ uint16_t ttab[TRITS ? 256 : 1];
  // Blocks have 1 to W waves (dequant_grid); the tables need 256 entries.
  for (int t = threadIdx.x; t < 256; t += blockDim.x) {
    if constexpr (TRITS) fill_trit_table(ttab, t);
    fill_table<SB>(tab, lv, t);
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int waves = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
  uint8_t* const buf = lds + wave * WAVE_BYTES;
  const int64_t n_batches = job.n_batches;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * waves;
  int64_t batch = static_cast<int64_t>(blockIdx.x) * waves + wave;
  if (batch >= n_batches) return;
  int d = 0;

  // LDS write: this lane's chunk c of a phase goes to slot c ^ swz_w.
  const int swz_w = (lane / GPB) & (CPP - 1);
  // Store instruction i moves groups GPI*i + lane/CPP, chunk lane % CPP.
  const int gq = lane / CPP, cc = lane % CPP;
  const uint32_t st_lane = static_cast<uint32_t>(gq * GOB + 16 * cc);

  constexpr int FW = TRITS ? 13 : 4 * SB;  // fetched dwords per lane
  uint32_t nwords[FW];
  uint16_t nn16 = 0;
  auto fetch = [&](const DBatch& b_) __attribute__((always_inline)) {
    if constexpr (TRITS)
      fetch_batch_trits(b_.packed, b_.norms, b_.bt, b_.nvalid(), lane, nwords, nn16);
    else
      fetch_batch<SB>(b_.packed, b_.norms, b_.bt, b_.nvalid(), lane, nwords, nn16);
  };
  DBatch cur = resolve<MANY>(job, batch, d);
  fetch(cur);
  for (;;) {
    uint32_t words[4 * SB];
    if constexpr (TRITS) {
      static_assert(SB == 2, "trit storage decodes to 2-bit fields");
      trits_to_fields(nwords, ttab, words);
    } else {
#pragma unroll
      for (int i = 0; i < 4 * SB; ++i) words[i] = nwords[i];
    }
    const uint16_t n16 = nn16;
    const int64_t next = batch + stride;
    const int nv = cur.nvalid();
    DBatch nxt = cur;
    if (next < n_batches) {
      nxt = resolve<MANY>(job, next, d);
      fetch(nxt);
    }

    float y[kGroup];
    reconstruct_fast<SB>(words, n16, tab, y);

    const auto dst = make_rsrc(cur.out + cur.bt * kWave * GOB, nv * GOB);
    // bf16 output: all 128 values are rounded and packed before the first
    // phase, so the phases only move finished registers.
    uint32_t pk[BF16OUT ? kGroup / 2 : 1];
    if constexpr (BF16OUT) {
#pragma unroll
      for (int i = 0; i < kGroup / 2; ++i) pk[i] = f32_to_bf16_rne(y[2 * i]) | (f32_to_bf16_rne(y[2 * i + 1]) << 16);
    }
#pragma unroll
    for (int ph = 0; ph < 4; ++ph) {
      // Scatter this lane's 32 values of the phase into the swizzled buffer.
      uint4 ch[CPP];
#pragma unroll
      for (int c = 0; c < CPP; ++c) {
        if constexpr (BF16OUT) {
          const int q = 16 * ph + 4 * c;
          ch[c] = make_uint4(pk[q], pk[q + 1], pk[q + 2], pk[q + 3]);
        } else {
          const int e = 32 * ph + 4 * c;
          ch[c] = make_uint4(__builtin_bit_cast(uint32_t, y[e]), __builtin_bit_cast(uint32_t, y[e + 1]),
                             __builtin_bit_cast(uint32_t, y[e + 2]), __builtin_bit_cast(uint32_t, y[e + 3]));
        }
      }
#pragma unroll
      for (int c = 0; c < CPP; ++c) *reinterpret_cast<uint4*>(buf + lane * PB + 16 * (c ^ swz_w)) = ch[c];
      // Gather 16-byte chunks so consecutive lanes write consecutive bytes.
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int gs = GPI * i + gq;
        const int sw = (gs / GPB) & (CPP - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(buf + gs * PB + 16 * (cc ^ sw));
        store16<BF16OUT ? 0 : kStoreF32>(v, dst, st_lane + ph * PB, static_cast<uint32_t>(GPI * i * GOB));
      }
      // After the gather reads (which complete after the writes), so the wait
      // adds nothing to the phase.
      hold_until_lds_written(ch);
    }
    cur = nxt;
    batch = next;
    if (batch >= n_batches) break;
  }
}

// General path: rows of any length; each lane writes its own group's valid
// columns.
// With MANY, thread g of the launch takes group g of the concatenation of the
// table's tensors (t.start holds group prefixes); the plain arguments are
// ignored.
template <int SB, bool BF16OUT, bool MANY, bool TRITS = false>
__global__ void __launch_bounds__(kBlock)
dequantize_ragged(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                  int64_t rows, int64_t cols, LevelTable lv, uint8_t* __restrict__ out,
                  TensorTable<DequantDesc> t, int64_t total) {
  __shared__ __attribute__((aligned(16))) float tab[TableSize<SB>::floats];
  __shared__ uint16_t ttab[TRITS ? 256 : 1];
  if constexpr (TRITS) fill_trit_table(ttab, threadIdx.x);
  fill_table<SB>(tab, lv, threadIdx.x);
  __syncthreads();
  int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if constexpr (MANY) {
    if (g >= total) return;
    const int d = find_unit(t.start, 0, t.n, g);
    const DequantDesc q = t.desc[d];
    packed = q.packed;
    norms = q.norms;
    out = q.out;
    rows = q.rows;
    cols = q.cols;
    g -= t.start[d];
  }
  const int64_t ngr = (cols + kGroup - 1) / kGroup;
  if (g >= rows * ngr) return;
  const int64_t row = g / ngr, col0 = (g - row * ngr) * kGroup;
  const int64_t valid = cols - col0 < kGroup ? cols - col0 : kGroup;
  uint32_t words[4 * SB];
  if constexpr (TRITS) {
    uint32_t tr[13];
    const uint16_t* src = reinterpret_cast<const uint16_t*>(packed + g * kTritBytes);
#pragma unroll
    for (int k = 0; k < 13; ++k) tr[k] = src[k];
    trits_to_fields(tr, ttab, words);
  } else {
    load_indices<SB>(packed, g, words);
  }
  float y[kGroup];
  reconstruct_fast<SB>(words, norms[g], tab, y);
  const int64_t base = row * cols + col0;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    if (j < valid) {
      if constexpr (BF16OUT)
        reinterpret_cast<uint16_t*>(out)[base + j] = static_cast<uint16_t>(f32_to_bf16_rne(y[j]));
      else
        reinterpret_cast<float*>(out)[base + j] = y[j];
    }
  }
}

// Grid: one batch per wave, a grid that covers the tensor (5-6% faster on
// the 7B-shaped model than a resident grid for float32 output; 2 and 4
// batches per wave were 4% and 8% slower), in blocks of W waves.  A call
// with fewer than W batches per CU takes smaller blocks, so its batches
// spread over more CUs (256x512, 16 batches: 16 one-wave blocks instead of
// two of eight).
template <bool BF16OUT>
ContigGrid dequant_grid(int64_t n_batches) {
  return contig_grid(n_batches, contig_waves(BF16OUT), 1, kBlocksPerCu);
}

template <int SB, bool BF16OUT, bool TRITS>
hipError_t launch_sb(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols,
                     const LevelTable& lv, void* out, hipStream_t s) {
  uint8_t* ob = static_cast<uint8_t*>(out);
  if (cols % kGroup == 0) {
    const int64_t n_groups = rows * (cols / kGroup);
    const int64_t n_batches = (n_groups + kWave - 1) / kWave;
    const ContigGrid g = dequant_grid<BF16OUT>(n_batches);
    const DequantJob job{packed, norms, ob, n_groups, TensorTable<DequantDesc>{nullptr, nullptr, 0},
                         n_batches};
    hipLaunchKernelGGL((dequantize_contig<SB, BF16OUT, false, TRITS>), dim3(g.blocks), dim3(g.waves * kWave), 0, s,
                       job, lv);
  } else {
    const int64_t n_groups = rows * ((cols + kGroup - 1) / kGroup);
    const int blocks = static_cast<int>((n_groups + kBlock - 1) / kBlock);
    hipLaunchKernelGGL((dequantize_ragged<SB, BF16OUT, false, TRITS>), dim3(blocks), dim3(kBlock), 0, s,
                       packed, norms, rows, cols, lv, ob, TensorTable<DequantDesc>{nullptr, nullptr, 0},
                       int64_t{0});
  }
  return hipGetLastError();
}

template <int SB, bool BF16OUT, bool TRITS>
hipError_t launch_many_sb(const LevelTable& lv, TensorTable<DequantDesc> contig, int64_t contig_batches,
                          TensorTable<DequantDesc> ragged, int64_t ragged_groups, hipStream_t s) {
  if (contig_batches > 0) {
    const ContigGrid g = dequant_grid<BF16OUT>(contig_batches);
    const DequantJob job{nullptr, nullptr, nullptr, 0, contig, contig_batches};
    hipLaunchKernelGGL((dequantize_contig<SB, BF16OUT, true, TRITS>), dim3(g.blocks), dim3(g.waves * kWave), 0, s,
                       job, lv);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ragged_groups > 0) {
    const int blocks = static_cast<int>((ragged_groups + kBlock - 1) / kBlock);
    hipLaunchKernelGGL((dequantize_ragged<SB, BF16OUT, true, TRITS>), dim3(blocks), dim3(kBlock), 0, s,
                       nullptr, nullptr, int64_t{0}, int64_t{0}, lv, nullptr, ragged, ragged_groups);
  }
  return hipGetLastError();
}

template <int SB, bool TRITS = false>
hipError_t launch_many_out(const LevelTable& lv, bool bf16_out, TensorTable<DequantDesc> contig,
                           int64_t contig_batches, TensorTable<DequantDesc> ragged, int64_t ragged_groups,
                           hipStream_t s) {
  return bf16_out ? launch_many_sb<SB, true, TRITS>(lv, contig, contig_batches, ragged, ragged_groups, s)
                  : launch_many_sb<SB, false, TRITS>(lv, contig, contig_batches, ragged, ragged_groups, s);
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
                                  hipStream_t stream) {
  switch (sbits) {
    case 2: return kd::launch_many_out<2>(lv, bf16_out, contig, contig_batches, ragged, ragged_groups, stream);
    case 3: return kd::launch_many_out<3>(lv, bf16_out, contig, contig_batches, ragged, ragged_groups, stream);
    case 4: return kd::launch_many_out<4>(lv, bf16_out, contig, contig_batches, ragged, ragged_groups, stream);
    case kTritStorage:
      return kd::launch_many_out<2, true>(lv, bf16_out, contig, contig_batches, ragged, ragged_groups, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cq
