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

// Reconstruct one group into y (float32, already scaled).
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

// Fast path: cols % 128 == 0, so group g's output is 128 contiguous values.
template <int SB, bool BF16OUT>
__global__ void __launch_bounds__(kBlock)
dequantize_contig(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                  int64_t n_groups, LevelTable lv, uint8_t* __restrict__ out) {
  constexpr int OB = BF16OUT ? 2 : 4;        // output bytes per element
  constexpr int PB = 32 * OB;                // bytes per group per phase
  constexpr int CPP = PB / 16;               // 16-byte chunks per group per phase
  constexpr int GPB = 256 / PB;              // groups per 256-byte LDS row
  constexpr int WAVE_BYTES = kWave * PB;
  constexpr int NI = WAVE_BYTES / 1024;      // store instructions per phase
  __shared__ float lut[kMaxLevels];
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * WAVE_BYTES];
  if (threadIdx.x < kMaxLevels) lut[threadIdx.x] = threadIdx.x < lv.n_levels ? lv.c[threadIdx.x] : 0.0f;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  uint8_t* const buf = lds + wave * WAVE_BYTES;
  const int64_t n_batches = (n_groups + kWave - 1) / kWave;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kWaves;
  const int swz_w = (lane / GPB) & (CPP - 1);

  for (int64_t batch = static_cast<int64_t>(blockIdx.x) * kWaves + wave; batch < n_batches;
       batch += stride) {
    const int64_t g0 = batch * kWave;
    const int64_t g = g0 + lane;
    const bool valid = g < n_groups;
    uint32_t words[4 * SB];
    uint16_t n16 = 0;
    if (valid) {
      load_indices<SB>(packed, g, words);
      n16 = norms[g];
    } else {
#pragma unroll
      for (int i = 0; i < 4 * SB; ++i) words[i] = 0;
    }
    float y[kGroup];
    reconstruct<SB>(words, n16, lut, y);

#pragma unroll
    for (int ph = 0; ph < 4; ++ph) {
      // Scatter this lane's 32 values of the phase into the swizzled buffer.
#pragma unroll
      for (int c = 0; c < CPP; ++c) {
        uint4 v;
        if constexpr (BF16OUT) {
          const int e = 32 * ph + 8 * c;
          v.x = f32_to_bf16_rne(y[e]) | (f32_to_bf16_rne(y[e + 1]) << 16);
          v.y = f32_to_bf16_rne(y[e + 2]) | (f32_to_bf16_rne(y[e + 3]) << 16);
          v.z = f32_to_bf16_rne(y[e + 4]) | (f32_to_bf16_rne(y[e + 5]) << 16);
          v.w = f32_to_bf16_rne(y[e + 6]) | (f32_to_bf16_rne(y[e + 7]) << 16);
        } else {
          const int e = 32 * ph + 4 * c;
          v = make_uint4(__builtin_bit_cast(uint32_t, y[e]), __builtin_bit_cast(uint32_t, y[e + 1]),
                         __builtin_bit_cast(uint32_t, y[e + 2]), __builtin_bit_cast(uint32_t, y[e + 3]));
        }
        *reinterpret_cast<uint4*>(buf + lane * PB + 16 * (c ^ swz_w)) = v;
      }
      // Gather 16-byte chunks so consecutive lanes write consecutive bytes.
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int slot = i * kWave + lane;
        const int gs = slot / CPP, c = slot % CPP;
        const int sw = (gs / GPB) & (CPP - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(buf + gs * PB + 16 * (c ^ sw));
        if (g0 + gs < n_groups)
          *reinterpret_cast<uint4*>(out + (g0 + gs) * (kGroup * OB) + ph * PB + 16 * c) = v;
      }
    }
  }
}

// General path: rows of any length; each lane writes its own group's valid
// columns.
template <int SB, bool BF16OUT>
__global__ void __launch_bounds__(kBlock)
dequantize_ragged(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms,
                  int64_t rows, int64_t cols, LevelTable lv, uint8_t* __restrict__ out) {
  __shared__ float lut[kMaxLevels];
  if (threadIdx.x < kMaxLevels) lut[threadIdx.x] = threadIdx.x < lv.n_levels ? lv.c[threadIdx.x] : 0.0f;
  __syncthreads();
  const int64_t ngr = (cols + kGroup - 1) / kGroup;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (g >= rows * ngr) return;
  const int64_t row = g / ngr, col0 = (g - row * ngr) * kGroup;
  const int64_t valid = cols - col0 < kGroup ? cols - col0 : kGroup;
  uint32_t words[4 * SB];
  load_indices<SB>(packed, g, words);
  float y[kGroup];
  reconstruct<SB>(words, norms[g], lut, y);
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

template <int SB, bool BF16OUT>
hipError_t launch_sb(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols,
                     const LevelTable& lv, void* out, hipStream_t s) {
  uint8_t* ob = static_cast<uint8_t*>(out);
  if (cols % kGroup == 0) {
    const int64_t n_groups = rows * (cols / kGroup);
    const int64_t n_batches = (n_groups + kWave - 1) / kWave;
    const int64_t want = (n_batches + kWaves - 1) / kWaves;
    const int blocks = static_cast<int>(want < 4096 ? want : 4096);
    hipLaunchKernelGGL((dequantize_contig<SB, BF16OUT>), dim3(blocks), dim3(kBlock), 0, s, packed,
                       norms, n_groups, lv, ob);
  } else {
    const int64_t n_groups = rows * ((cols + kGroup - 1) / kGroup);
    const int blocks = static_cast<int>((n_groups + kBlock - 1) / kBlock);
    hipLaunchKernelGGL((dequantize_ragged<SB, BF16OUT>), dim3(blocks), dim3(kBlock), 0, s, packed,
                       norms, rows, cols, lv, ob);
  }
  return hipGetLastError();
}

template <int SB>
hipError_t launch_out(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols,
                      const LevelTable& lv, void* out, bool bf16_out, hipStream_t s) {
  return bf16_out ? launch_sb<SB, true>(packed, norms, rows, cols, lv, out, s)
                  : launch_sb<SB, false>(packed, norms, rows, cols, lv, out, s);
}

}  // namespace kd

hipError_t launch_dequantize(const uint8_t* packed, const uint16_t* norms, int64_t rows,
                             int64_t cols, int sbits, const LevelTable& lv, void* out,
                             bool bf16_out, hipStream_t stream) {
  switch (sbits) {
    case 2: return kd::launch_out<2>(packed, norms, rows, cols, lv, out, bf16_out, stream);
    case 3: return kd::launch_out<3>(packed, norms, rows, cols, lv, out, bf16_out, stream);
    case 4: return kd::launch_out<4>(packed, norms, rows, cols, lv, out, bf16_out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cq
