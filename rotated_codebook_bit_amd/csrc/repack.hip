// Conversion between the two storage forms of the three-level ("1.58-bit")
// code ("How Quantization Codebooks Are Trained in Cactus Quants", section
// Ternary Special Case Handling): 2-bit fields (32 bytes per 128-group, the
// layout the product kernels decode) and trits (five indices per byte, 26
// bytes per 128-group, ceil(G / 5) at group size G).  One thread per group.

#include "cq_internal.h"

namespace cq {
namespace {

constexpr int kBlock = 256;

__global__ void __launch_bounds__(kBlock)
fields_to_trits_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n_groups) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (g >= n_groups) return;
  const uint4* s = reinterpret_cast<const uint4*>(src + g * 32);
  const uint4 a = s[0], b = s[1];
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t t[13];
  fields_to_trits(w, t);
  uint16_t* d = reinterpret_cast<uint16_t*>(dst + g * kTritBytes);
#pragma unroll
  for (int k = 0; k < 13; ++k) d[k] = static_cast<uint16_t>(t[k]);
}

__global__ void __launch_bounds__(kBlock)
trits_to_fields_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n_groups) {
  __shared__ uint16_t tab[256];
  {
    const uint32_t v = trit_table_entry(threadIdx.x);
    tab[threadIdx.x] = static_cast<uint16_t>(v);
    wait_lds_writes();  // the value keeps its register until stored
    hold_values(v);
  }
  __syncthreads();
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (g >= n_groups) return;
  const uint16_t* s = reinterpret_cast<const uint16_t*>(src + g * kTritBytes);
  uint32_t t[13];
#pragma unroll
  for (int k = 0; k < 13; ++k) t[k] = s[k];
  uint32_t w[8];
  trits_to_fields(t, tab, w);
  uint4* d = reinterpret_cast<uint4*>(dst + g * 32);
  d[0] = make_uint4(w[0], w[1], w[2], w[3]);
  d[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// Other group sizes G (32, 64, 256): G / 4 bytes of fields (read and
// written as G / 16 dwords) and ceil(G / 5) trit bytes (byte accesses: a
// group's trit bytes need not be aligned), the same digit order.
template <int G>
__global__ void __launch_bounds__(kBlock)
fields_to_trits_g(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n_groups) {
  constexpr int TB = (G + 4) / 5;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (g >= n_groups) return;
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src + g * (G / 4));
  uint32_t w[G / 16];
#pragma unroll
  for (int i = 0; i < G / 16; ++i) w[i] = s[i];
  uint8_t* d = dst + g * TB;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 4; i >= 0; --i) {
      const int j = 5 * b + i;
      if (j < G) v = v * 3u + ((w[j / 16] >> (2 * (j % 16))) & 3u);
    }
    d[b] = static_cast<uint8_t>(v);
  }
}

template <int G>
__global__ void __launch_bounds__(kBlock)
trits_to_fields_g(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int64_t n_groups) {
  constexpr int TB = (G + 4) / 5;
  __shared__ uint16_t tab[256];
  {
    const uint32_t v = trit_table_entry(threadIdx.x);
    tab[threadIdx.x] = static_cast<uint16_t>(v);
    wait_lds_writes();  // the value keeps its register until stored
    hold_values(v);
  }
  __syncthreads();
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (g >= n_groups) return;
  const uint8_t* s = src + g * TB;
  uint32_t w[G / 16];
#pragma unroll
  for (int i = 0; i < G / 16; ++i) w[i] = 0u;
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    const uint32_t f = tab[s[b]];  // five 2-bit fields, digit i at bits 2i
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int j = 5 * b + i;
      if (j < G) w[j / 16] |= ((f >> (2 * i)) & 3u) << (2 * (j % 16));
    }
  }
  uint32_t* d = reinterpret_cast<uint32_t*>(dst + g * (G / 4));
#pragma unroll
  for (int i = 0; i < G / 16; ++i) d[i] = w[i];
}

template <int G>
void launch_g(const uint8_t* src, bool to_trits, uint8_t* dst, int64_t n_groups, hipStream_t stream) {
  const unsigned blocks = static_cast<unsigned>((n_groups + kBlock - 1) / kBlock);
  if (to_trits)
    hipLaunchKernelGGL(fields_to_trits_g<G>, dim3(blocks), dim3(kBlock), 0, stream, src, dst, n_groups);
  else
    hipLaunchKernelGGL(trits_to_fields_g<G>, dim3(blocks), dim3(kBlock), 0, stream, src, dst, n_groups);
}

}  // namespace

hipError_t launch_repack(const uint8_t* src, bool to_trits, uint8_t* dst, int64_t n_groups, int group_size,
                         hipStream_t stream) {
  if (n_groups <= 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((n_groups + kBlock - 1) / kBlock);
  switch (group_size) {
    case kGroup:
      if (to_trits)
        hipLaunchKernelGGL(fields_to_trits_kernel, dim3(blocks), dim3(kBlock), 0, stream, src, dst, n_groups);
      else
        hipLaunchKernelGGL(trits_to_fields_kernel, dim3(blocks), dim3(kBlock), 0, stream, src, dst, n_groups);
      break;
    case 32: launch_g<32>(src, to_trits, dst, n_groups, stream); break;
    case 64: launch_g<64>(src, to_trits, dst, n_groups, stream); break;
    case 256: launch_g<256>(src, to_trits, dst, n_groups, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace cq
