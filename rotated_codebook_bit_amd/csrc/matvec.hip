// CQ dequantize-matvec kernels for gfx950: y = x . W_hat^T.
//
// The pages use the quantized weights in an ordinary forward product
// ("Performance Differences Between 2-Bit and 4-Bit Quantization in Needle",
// section Practical Code Comparison) and describe a runtime that decodes the
// packed tensors on the fly ("How Needle 2 Model Compresses to a Single
// Binary", section Stage 3).  Here the decode is fused into the product.
//
// Because the orthonormal Hadamard matrix is symmetric and its own inverse,
// for every group g of a row
//     x_g . W_hat_g = (norm_g / G) * < H x_g , levels[idx_g] >
// with H the +-1 Sylvester matrix.  So the activations are rotated once per
// (batch row, group) by rotate_rows, and the main kernel never applies a
// per-weight inverse rotation: it looks the level up and accumulates.
//
// Main kernel mapping: a lane owns 16 consecutive columns of a 1024-column
// tile and keeps the rotated activations of those columns (16 per batch row)
// in registers; a wave handles RW rows, walking the tiles, and keeps RW x NB
// per-lane partial sums.  The cross-lane reduction happens once per row at
// the end.  Packed bits of 16 consecutive columns are 4 (2-bit), 6 (3-bit)
// or 8 (4-bit) bytes, so one wave instruction reads 256-512 contiguous bytes
// of a row.

#include "cq_internal.h"

namespace cq {
namespace km {

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;
constexpr int kRowsPerWave = 4;
constexpr int kTile = 16 * kWave;  // columns per tile

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// xr[g][:] = H x[g][:] for n_groups consecutive 128-value groups.
__global__ void __launch_bounds__(kBlock)
rotate_rows_kernel(const float* __restrict__ x, int64_t n_groups, float* __restrict__ xr) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (g >= n_groups) return;
  float y[kGroup];
  const float4* src = reinterpret_cast<const float4*>(x + g * kGroup);
#pragma unroll
  for (int i = 0; i < kGroup / 4; ++i) {
    const float4 v = src[i];
    y[4 * i] = v.x;
    y[4 * i + 1] = v.y;
    y[4 * i + 2] = v.z;
    y[4 * i + 3] = v.w;
  }
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
  float4* dst = reinterpret_cast<float4*>(xr + g * kGroup);
#pragma unroll
  for (int i = 0; i < kGroup / 4; ++i) dst[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Packed bits of the 16 columns starting at column c0 (c0 % 16 == 0) of a
// row, as a 64-bit value with column c0+e at bits [SB*e, SB*e + SB).
template <int SB>
__device__ __forceinline__ uint64_t load_bits16(const uint8_t* __restrict__ row_ptr, int64_t c0) {
  if constexpr (SB == 2) {
    return *reinterpret_cast<const uint32_t*>(row_ptr + c0 / 4);
  } else if constexpr (SB == 4) {
    return *reinterpret_cast<const uint64_t*>(row_ptr + c0 / 2);
  } else {
    // 6 bytes at the 2-byte aligned offset 6*(c0/16); read exactly those
    // bytes so the last chunk of the last row stays inside the buffer.
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row_ptr + 6 * (c0 / 16));
    return static_cast<uint64_t>(p[0]) | (static_cast<uint64_t>(p[1]) << 16) |
           (static_cast<uint64_t>(p[2]) << 32);
  }
}

template <int SB, int NB>
__global__ void __launch_bounds__(kBlock)
matvec_kernel(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms, int64_t n_out,
              int64_t k, LevelTable lv, const float* __restrict__ xr, int64_t batch, int64_t b0,
              float* __restrict__ y) {
  __shared__ float lut[kMaxLevels];
  if (threadIdx.x < kMaxLevels) lut[threadIdx.x] = threadIdx.x < lv.n_levels ? lv.c[threadIdx.x] : 0.0f;
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / kWave;
  const int64_t r0 = wave * kRowsPerWave;
  if (r0 >= n_out) return;
  const int64_t row_bytes = k * SB / 8;
  const int64_t ngr = k / kGroup;

  float acc[kRowsPerWave][NB];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;

  for (int64_t t0 = 0; t0 < k; t0 += kTile) {
    const int64_t c0 = t0 + 16 * lane;
    if (c0 < k) {
      float xv[NB][16];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float4* src = reinterpret_cast<const float4*>(xr + (b0 + b) * k + c0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 v = src[i];
          xv[b][4 * i] = v.x;
          xv[b][4 * i + 1] = v.y;
          xv[b][4 * i + 2] = v.z;
          xv[b][4 * i + 3] = v.w;
        }
      }
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        const int64_t row = r0 + r;
        if (row < n_out) {
          const uint64_t bits = load_bits16<SB>(packed + row * row_bytes, c0);
          const float s = half_to_float(norms[row * ngr + c0 / kGroup]) * (1.0f / kGroup);
          float part[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) part[b] = 0.0f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float v = lut[(bits >> (SB * e)) & ((1u << SB) - 1u)];
#pragma unroll
            for (int b = 0; b < NB; ++b) part[b] = __builtin_fmaf(v, xv[b][e], part[b]);
          }
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[r][b] = __builtin_fmaf(s, part[b], acc[r][b]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float v = wave_sum(acc[r][b]);
      const int64_t row = r0 + r;
      if (lane == 0 && row < n_out) y[(b0 + b) * n_out + row] = v;
    }
  }
}

template <int SB, int NB>
hipError_t launch_nb(const uint8_t* packed, const uint16_t* norms, int64_t n_out, int64_t k,
                     const LevelTable& lv, const float* xr, int64_t batch, int64_t b0, float* y,
                     hipStream_t s) {
  const int64_t waves = (n_out + kRowsPerWave - 1) / kRowsPerWave;
  const int blocks = static_cast<int>((waves + kWaves - 1) / kWaves);
  hipLaunchKernelGGL((matvec_kernel<SB, NB>), dim3(blocks), dim3(kBlock), 0, s, packed, norms, n_out,
                     k, lv, xr, batch, b0, y);
  return hipGetLastError();
}

template <int SB>
hipError_t launch_sb(const uint8_t* packed, const uint16_t* norms, int64_t n_out, int64_t k,
                     const LevelTable& lv, const float* xr, int64_t batch, float* y, hipStream_t s) {
  for (int64_t b0 = 0; b0 < batch; b0 += 8) {
    const int64_t nb = batch - b0 < 8 ? batch - b0 : 8;
    hipError_t e;
    switch (nb) {
      case 1: e = launch_nb<SB, 1>(packed, norms, n_out, k, lv, xr, batch, b0, y, s); break;
      case 2: e = launch_nb<SB, 2>(packed, norms, n_out, k, lv, xr, batch, b0, y, s); break;
      case 3: e = launch_nb<SB, 3>(packed, norms, n_out, k, lv, xr, batch, b0, y, s); break;
      case 4: e = launch_nb<SB, 4>(packed, norms, n_out, k, lv, xr, batch, b0, y, s); break;
      case 5: e = launch_nb<SB, 5>(packed, norms, n_out, k, lv, xr, batch, b0, y, s); break;
      case 6: e = launch_nb<SB, 6>(packed, norms, n_out, k, lv, xr, batch, b0, y, s); break;
      case 7: e = launch_nb<SB, 7>(packed, norms, n_out, k, lv, xr, batch, b0, y, s); break;
      default: e = launch_nb<SB, 8>(packed, norms, n_out, k, lv, xr, batch, b0, y, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace km

hipError_t launch_rotate_rows(const float* x, int64_t n_groups, float* xr, hipStream_t stream) {
  if (n_groups <= 0) return hipSuccess;
  const int blocks = static_cast<int>((n_groups + km::kBlock - 1) / km::kBlock);
  hipLaunchKernelGGL(km::rotate_rows_kernel, dim3(blocks), dim3(km::kBlock), 0, stream, x, n_groups, xr);
  return hipGetLastError();
}

hipError_t launch_matvec(const uint8_t* packed, const uint16_t* norms, int64_t n_out, int64_t k,
                         int sbits, const LevelTable& lv, const float* xr, int64_t batch, float* y,
                         hipStream_t stream) {
  switch (sbits) {
    case 2: return km::launch_sb<2>(packed, norms, n_out, k, lv, xr, batch, y, stream);
    case 3: return km::launch_sb<3>(packed, norms, n_out, k, lv, xr, batch, y, stream);
    case 4: return km::launch_sb<4>(packed, norms, n_out, k, lv, xr, batch, y, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cq
