// CQ quantize / dequantize / fake quantization for group sizes other than
// 128 (32, 64, 256).  The pages make the group size a parameter of the
// quantizer, default 128, and describe the trade-off: smaller groups get
// finer norms for more storage, larger groups the reverse ("Cactus Quants
// CQ2-bit Quantization: Extreme Compression for Edge LLMs", FAQ on group
// size; "How Quantization Codebooks Are Trained in Cactus Quants", FAQ on
// group size and the codebook).
//
// Mapping: a group is handled by R adjacent lanes (R = G / 64 for G = 256,
// else 1), lane r holding the C = G / R consecutive values [r C, r C + C).
// The Sylvester matrix factors as H_G = H_R (x) H_C, so each lane applies the
// C-point butterfly to its own values and then log2(R) butterfly stages run
// across the group's lanes (lane r combines with lane r ^ d).  The norm is
// the sum of squares over the group's lanes.  A lane's indices are a
// contiguous run of the group's bit stream (bits [sbits r C, sbits (r+1) C)),
// so each lane stores its own packed bytes; lane 0 stores the norm.
//
// Decisions are the same as for G = 128: z = Y / n with Y the unnormalised
// butterfly output, index = number of thresholds t with t * n < Y (for a
// zero group, n is taken as 1 and Y = 0).  These kernels load and store
// with plain vector memory operations (16-byte when a lane's span is whole
// and aligned, else per element); the G = 128 path has the tuned kernels.

#include "cq_internal.h"

namespace cq {
namespace kgs {

constexpr int kBlock = 256;

template <int G>
struct GS {
  static constexpr int R = G > 64 ? G / 64 : 1;  // lanes per group
  static constexpr int C = G / R;                // values per lane
};

// Where this lane's values sit: group, lane-in-group, first column, number
// of valid columns (0..C; columns past the row end are zero padding).
struct Span {
  int64_t group, row, col0, valid;
  int r;
  bool live;
};

template <int G>
__device__ __forceinline__ Span locate(int64_t rows, int64_t cols) {
  constexpr int R = GS<G>::R, C = GS<G>::C;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  Span s;
  s.group = t / R;
  s.r = static_cast<int>(t % R);
  const int64_t ngr = (cols + G - 1) / G;
  s.live = s.group < rows * ngr;
  s.row = s.live ? s.group / ngr : 0;
  s.col0 = s.live ? (s.group - s.row * ngr) * G + s.r * C : 0;
  const int64_t left = cols - s.col0;
  s.valid = !s.live ? 0 : (left < 0 ? 0 : (left < C ? left : C));
  return s;
}

template <int C, bool BF16>
__device__ __forceinline__ void load_values(const uint8_t* __restrict__ w, int64_t cols, const Span& s,
                                            float (&x)[C]) {
  const int64_t base = s.row * cols + s.col0;
  constexpr int EB = BF16 ? 2 : 4;
  const bool vec = s.valid == C && ((base * EB) % 16 == 0);
  if (vec) {
    const uint4* src = reinterpret_cast<const uint4*>(w + base * EB);
#pragma unroll
    for (int i = 0; i < C * EB / 16; ++i) {
      const uint4 v = src[i];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if constexpr (BF16) {
          x[8 * i + 2 * q] = __builtin_bit_cast(float, u[q] << 16);
          x[8 * i + 2 * q + 1] = __builtin_bit_cast(float, u[q] & 0xFFFF0000u);
        } else {
          x[4 * i + q] = __builtin_bit_cast(float, u[q]);
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < C; ++j) {
      float v = 0.0f;
      if (j < s.valid) {
        if constexpr (BF16)
          v = __builtin_bit_cast(float, static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(w)[base + j]) << 16);
        else
          v = reinterpret_cast<const float*>(w)[base + j];
      }
      x[j] = v;
    }
  }
}

// In-lane C-point butterfly (unnormalised), then the cross-lane stages.
template <int C, int R>
__device__ __forceinline__ void hadamard(float (&y)[C], int r) {
#pragma unroll
  for (int h = 1; h < C; h <<= 1) {
#pragma unroll
    for (int i = 0; i < C; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int d = 1; d < R; d <<= 1) {
    const bool upper = (r & d) != 0;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const float o = __shfl_xor(y[j], d, kWave);
      y[j] = upper ? o - y[j] : y[j] + o;
    }
  }
}

template <int R>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int d = 1; d < R; d <<= 1) v += __shfl_xor(v, d, kWave);
  return v;
}

__device__ __forceinline__ uint32_t decide(float y, float ns, const QuantParams& p) {
  uint32_t idx = 0;
#pragma unroll
  for (int i = 0; i < kMaxLevels - 1; ++i)
    if (i < p.n_levels - 1) idx += (p.thr[i] * ns < y) ? 1u : 0u;
  return idx;
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int C, bool BF16OUT>
__device__ __forceinline__ void store_values(uint8_t* __restrict__ out, int64_t cols, const Span& s,
                                             const float (&y)[C]) {
  const int64_t base = s.row * cols + s.col0;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    if (j < s.valid) {
      if constexpr (BF16OUT)
        reinterpret_cast<uint16_t*>(out)[base + j] = static_cast<uint16_t>(bf16_rne(y[j]));
      else
        reinterpret_cast<float*>(out)[base + j] = y[j];
    }
  }
}

template <int G, int SB, bool BF16>
__global__ void __launch_bounds__(kBlock)
quantize_g(const uint8_t* __restrict__ w, int64_t rows, int64_t cols, QuantParams p,
           uint8_t* __restrict__ packed, uint16_t* __restrict__ norms) {
  constexpr int R = GS<G>::R, C = GS<G>::C;
  constexpr int LW = C * SB / 32;  // packed dwords per lane
  const Span s = locate<G>(rows, cols);
  float y[C];
  load_values<C, BF16>(w, cols, s, y);  // valid == 0 on dead lanes: zeros
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < C; ++j) ss = __builtin_fmaf(y[j], y[j], ss);
  ss = group_sum<R>(ss);
  hadamard<C, R>(y, s.r);
  if (!s.live) return;  // after the cross-lane stages: every lane took part
  const float n = __builtin_sqrtf(ss);
  const float ns = ss > 0.0f ? n : 1.0f;
  uint32_t words[LW];
#pragma unroll
  for (int i = 0; i < LW; ++i) words[i] = 0u;
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const uint32_t idx = decide(y[j], ns, p);
    const int bit = SB * j;
    words[bit / 32] |= idx << (bit % 32);
    if (bit % 32 + SB > 32) words[bit / 32 + 1] |= idx >> (32 - bit % 32);
  }
  uint32_t* dst = reinterpret_cast<uint32_t*>(packed + s.group * (G * SB / 8) + s.r * (C * SB / 8));
#pragma unroll
  for (int i = 0; i < LW; ++i) dst[i] = words[i];
  if (s.r == 0) norms[s.group] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(n));
}

template <int G, int SB, bool BF16OUT>
__global__ void __launch_bounds__(kBlock)
dequantize_g(const uint8_t* __restrict__ packed, const uint16_t* __restrict__ norms, int64_t rows,
             int64_t cols, LevelTable lv, uint8_t* __restrict__ out) {
  constexpr int R = GS<G>::R, C = GS<G>::C;
  constexpr int LW = C * SB / 32;
  const Span s = locate<G>(rows, cols);
  float y[C];
  uint32_t words[LW];
  float scale = 0.0f;
  if (s.live) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(packed + s.group * (G * SB / 8) + s.r * (C * SB / 8));
#pragma unroll
    for (int i = 0; i < LW; ++i) words[i] = src[i];
    scale = static_cast<float>(__builtin_bit_cast(_Float16, norms[s.group])) * (1.0f / G);
  } else {
#pragma unroll
    for (int i = 0; i < LW; ++i) words[i] = 0u;
  }
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int bit = SB * j;
    uint32_t idx = words[bit / 32] >> (bit % 32);
    if (bit % 32 + SB > 32) idx |= words[bit / 32 + 1] << (32 - bit % 32);
    y[j] = level_at(lv, static_cast<int>(idx & ((1u << SB) - 1u)));
  }
  hadamard<C, R>(y, s.r);
  if (!s.live) return;
#pragma unroll
  for (int j = 0; j < C; ++j) y[j] *= scale;
  store_values<C, BF16OUT>(out, cols, s, y);
}

template <int G, bool BF16, bool BF16OUT>
__global__ void __launch_bounds__(kBlock)
fake_quant_g(const uint8_t* __restrict__ w, int64_t rows, int64_t cols, QuantParams p, LevelTable lv,
             uint8_t* __restrict__ out) {
  constexpr int R = GS<G>::R, C = GS<G>::C;
  const Span s = locate<G>(rows, cols);
  float y[C];
  load_values<C, BF16>(w, cols, s, y);
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < C; ++j) ss = __builtin_fmaf(y[j], y[j], ss);
  ss = group_sum<R>(ss);
  hadamard<C, R>(y, s.r);
  const float n = __builtin_sqrtf(ss);
  const float ns = ss > 0.0f ? n : 1.0f;
#pragma unroll
  for (int j = 0; j < C; ++j) y[j] = level_at(lv, static_cast<int>(decide(y[j], ns, p)));
  hadamard<C, R>(y, s.r);
  if (!s.live) return;
  const float sc = n * (1.0f / G);
#pragma unroll
  for (int j = 0; j < C; ++j) y[j] *= sc;
  store_values<C, BF16OUT>(out, cols, s, y);
}

template <int G>
int64_t grid(int64_t rows, int64_t cols) {
  const int64_t threads = rows * ((cols + G - 1) / G) * GS<G>::R;
  return (threads + kBlock - 1) / kBlock;
}

template <int G, int SB>
hipError_t quantize_sb(const void* w, bool bf16, int64_t rows, int64_t cols, const QuantParams& p,
                       uint8_t* packed, uint16_t* norms, hipStream_t s) {
  const auto* wb = static_cast<const uint8_t*>(w);
  const dim3 b(static_cast<unsigned>(grid<G>(rows, cols)));
  if (bf16)
    hipLaunchKernelGGL((quantize_g<G, SB, true>), b, dim3(kBlock), 0, s, wb, rows, cols, p, packed, norms);
  else
    hipLaunchKernelGGL((quantize_g<G, SB, false>), b, dim3(kBlock), 0, s, wb, rows, cols, p, packed, norms);
  return hipGetLastError();
}

template <int G>
hipError_t quantize_gs(const void* w, bool bf16, int64_t rows, int64_t cols, const QuantParams& p,
                       uint8_t* packed, uint16_t* norms, hipStream_t s) {
  switch (p.n_levels) {
    case 3:
    case 4: return quantize_sb<G, 2>(w, bf16, rows, cols, p, packed, norms, s);
    case 8: return quantize_sb<G, 3>(w, bf16, rows, cols, p, packed, norms, s);
    case 16: return quantize_sb<G, 4>(w, bf16, rows, cols, p, packed, norms, s);
    default: return hipErrorInvalidValue;
  }
}

template <int G, int SB>
hipError_t dequantize_sb(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols,
                         const LevelTable& lv, void* out, bool bf16_out, hipStream_t s) {
  auto* ob = static_cast<uint8_t*>(out);
  const dim3 b(static_cast<unsigned>(grid<G>(rows, cols)));
  if (bf16_out)
    hipLaunchKernelGGL((dequantize_g<G, SB, true>), b, dim3(kBlock), 0, s, packed, norms, rows, cols, lv, ob);
  else
    hipLaunchKernelGGL((dequantize_g<G, SB, false>), b, dim3(kBlock), 0, s, packed, norms, rows, cols, lv, ob);
  return hipGetLastError();
}

template <int G>
hipError_t dequantize_gs(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols, int sbits,
                         const LevelTable& lv, void* out, bool bf16_out, hipStream_t s) {
  switch (sbits) {
    case 2: return dequantize_sb<G, 2>(packed, norms, rows, cols, lv, out, bf16_out, s);
    case 3: return dequantize_sb<G, 3>(packed, norms, rows, cols, lv, out, bf16_out, s);
    case 4: return dequantize_sb<G, 4>(packed, norms, rows, cols, lv, out, bf16_out, s);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
hipError_t fake_quant_gs(const void* w, bool bf16, int64_t rows, int64_t cols, const QuantParams& p,
                         const LevelTable& lv, void* out, bool bf16_out, hipStream_t s) {
  const auto* wb = static_cast<const uint8_t*>(w);
  auto* ob = static_cast<uint8_t*>(out);
  const dim3 b(static_cast<unsigned>(grid<G>(rows, cols)));
  if (bf16) {
    if (bf16_out)
      hipLaunchKernelGGL((fake_quant_g<G, true, true>), b, dim3(kBlock), 0, s, wb, rows, cols, p, lv, ob);
    else
      hipLaunchKernelGGL((fake_quant_g<G, true, false>), b, dim3(kBlock), 0, s, wb, rows, cols, p, lv, ob);
  } else {
    if (bf16_out)
      hipLaunchKernelGGL((fake_quant_g<G, false, true>), b, dim3(kBlock), 0, s, wb, rows, cols, p, lv, ob);
    else
      hipLaunchKernelGGL((fake_quant_g<G, false, false>), b, dim3(kBlock), 0, s, wb, rows, cols, p, lv, ob);
  }
  return hipGetLastError();
}

}  // namespace kgs

hipError_t launch_quantize_g(int group_size, const void* w, bool bf16, int64_t rows, int64_t cols,
                             const QuantParams& p, uint8_t* packed, uint16_t* norms, hipStream_t stream) {
  switch (group_size) {
    case 32: return kgs::quantize_gs<32>(w, bf16, rows, cols, p, packed, norms, stream);
    case 64: return kgs::quantize_gs<64>(w, bf16, rows, cols, p, packed, norms, stream);
    case 256: return kgs::quantize_gs<256>(w, bf16, rows, cols, p, packed, norms, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequantize_g(int group_size, const uint8_t* packed, const uint16_t* norms, int64_t rows,
                               int64_t cols, int sbits, const LevelTable& lv, void* out, bool bf16_out,
                               hipStream_t stream) {
  switch (group_size) {
    case 32: return kgs::dequantize_gs<32>(packed, norms, rows, cols, sbits, lv, out, bf16_out, stream);
    case 64: return kgs::dequantize_gs<64>(packed, norms, rows, cols, sbits, lv, out, bf16_out, stream);
    case 256: return kgs::dequantize_gs<256>(packed, norms, rows, cols, sbits, lv, out, bf16_out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fake_quant_g(int group_size, const void* w, bool bf16, int64_t rows, int64_t cols,
                               const QuantParams& p, const LevelTable& lv, void* out, bool bf16_out,
                               hipStream_t stream) {
  switch (group_size) {
    case 32: return kgs::fake_quant_gs<32>(w, bf16, rows, cols, p, lv, out, bf16_out, stream);
    case 64: return kgs::fake_quant_gs<64>(w, bf16, rows, cols, p, lv, out, bf16_out, stream);
    case 256: return kgs::fake_quant_gs<256>(w, bf16, rows, cols, p, lv, out, bf16_out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cq
