// CQ dequantize-matvec kernels for gfx950: y = x . W_hat^T for one or many
// quantized matrices.
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
// (batch row, group) by rotate_kernel, and the product kernel never applies
// a per-weight inverse rotation: it looks the levels up and accumulates.
//
// Both kernels read a table of matrix descriptors in device memory, so any
// number of matrices (a whole model's decode step) runs as two launches.
//
// Product kernel mapping: a block (4 waves) owns RB consecutive rows of one
// matrix.  Thread t owns 16-column chunks t, t + 256, ... of the row (one
// 4096-column pass per 256 chunks) and keeps the rotated activations of its
// chunk in registers for the whole pass; for every row it loads the 4 (2-bit)
// / 6 (3-bit) / 8 (4-bit) bytes of codes of its chunk (a wave instruction
// reads 256-512 contiguous bytes of the row), decodes four (2-bit) or two
// (4-bit) levels per LDS read from a byte table, and accumulates NB partial
// sums per row.  The block reduces its RB x NB partials through LDS in a
// fixed order, so results are deterministic.

#include "cq_internal.h"

namespace cq {
namespace km {

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;
constexpr int kChunk = 16;              // columns per thread per pass
constexpr int kPass = kChunk * kBlock;  // columns per pass (4096)

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Index of the descriptor whose [start[d], start[d+1]) range holds v
// (start ascending, start[0] = 0, start[n] = total, v < total).
__device__ __forceinline__ int find_desc(const int64_t* __restrict__ start, int n, int64_t v) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] <= v)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// xr[m][b][g][:] = H x[m][b][g][:] for every 128-value group of every
// matrix's activations; one thread per group.
__global__ void __launch_bounds__(kBlock)
rotate_kernel(const MatvecDesc* __restrict__ table, const int64_t* __restrict__ gstart, int n,
              float* __restrict__ xr) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (g >= gstart[n]) return;
  const int d = find_desc(gstart, n, g);
  const MatvecDesc& m = table[d];
  const int64_t local = g - gstart[d];  // group within the matrix's batch*k/128
  const float* src = m.x + local * kGroup;
  float* dst = xr + m.xr_offset + local * kGroup;
  float y[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup / 4; ++i) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
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
#pragma unroll
  for (int i = 0; i < kGroup / 4; ++i)
    reinterpret_cast<float4*>(dst)[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
}

// Packed codes of the 16 columns starting at column c0 (c0 % 16 == 0) of a
// row, as a 64-bit value with column c0+e at bits [SB*e, SB*e + SB).
template <int SB>
__device__ __forceinline__ uint64_t load_codes16(const uint8_t* __restrict__ row_ptr, int64_t c0) {
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

// Level table in LDS.  2 bits: entry b (a code byte) holds the 4 levels its
// four 2-bit codes select; 4 bits: entry b holds the 2 levels of its two
// nibbles; 3 bits: plain 8-entry table.
//
// The lookups are data-dependent, so lanes reading the LDS in the same cycle
// collide on banks.  With K > 1 the table is stored in K interleaved copies
// (entry e of copy c at slot e * K + c) and lane l reads copy l % K, so the
// bank a lane touches depends on its copy rather than on its code.  Filling
// K copies costs every block K times the table writes and K times the LDS:
// measured on the 225-matrix pass, 8 copies pay from batch chunks of 4 rows
// (batch 8: 7.0 -> 6.15 ms) and cost at 1 to 3 rows.
template <int SB, int K>
struct Levels {
  static constexpr int entry = SB == 2 ? 4 : (SB == 4 ? 2 : 1);  // floats per entry
  static constexpr int entries = SB == 3 ? kMaxLevels : 256;
  static constexpr int floats = entries * entry * K;
  static __device__ __forceinline__ float lev(const LevelTable& lv, int i) { return level_at(lv, i); }
  static __device__ __forceinline__ void fill(float* tab, const LevelTable& lv, int t) {
    if (t >= entries) return;
    float e[entry];
    if constexpr (SB == 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) e[q] = lev(lv, (t >> (2 * q)) & 3);
    } else if constexpr (SB == 4) {
      e[0] = lev(lv, t & 15);
      e[1] = lev(lv, t >> 4);
    } else {
      e[0] = lev(lv, t);
    }
#pragma unroll
    for (int c = 0; c < K; ++c)
#pragma unroll
      for (int q = 0; q < entry; ++q) tab[(t * K + c) * entry + q] = e[q];
  }
  // Levels of the 16 codes into v[16]; copy = lane % K.
  static __device__ __forceinline__ void decode(uint64_t codes, const float* tab, int copy, float (&v)[16]) {
    const float* t = tab + copy * entry;
    if constexpr (SB == 2) {
      const uint32_t c = static_cast<uint32_t>(codes);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 f = *reinterpret_cast<const float4*>(t + 4 * K * ((c >> (8 * q)) & 0xFFu));
        v[4 * q] = f.x;
        v[4 * q + 1] = f.y;
        v[4 * q + 2] = f.z;
        v[4 * q + 3] = f.w;
      }
    } else if constexpr (SB == 4) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float2 f = *reinterpret_cast<const float2*>(t + 2 * K * ((codes >> (8 * q)) & 0xFFu));
        v[2 * q] = f.x;
        v[2 * q + 1] = f.y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = t[K * ((codes >> (3 * e)) & 7u)];
    }
  }
};

// Table copies for a batch chunk of NB rows.
constexpr int table_copies(int nb) { return nb >= 4 ? 8 : 1; }

// RB rows x NB batch rows per block; RB * NB <= 32 keeps the accumulators
// and the activations of a chunk (16 * NB) in registers.
template <int SB, int NB, int RB>
__global__ void __launch_bounds__(kBlock)
matvec_kernel(const MatvecDesc* __restrict__ table, const int64_t* __restrict__ bstart, int n,
              LevelTable lv, const float* __restrict__ xr, int64_t b0) {
  using Lv = Levels<SB, table_copies(NB)>;
  __shared__ __attribute__((aligned(16))) float tab[Lv::floats];
  __shared__ float red[RB * NB][kBlock + 1];
  Lv::fill(tab, lv, threadIdx.x);
  __syncthreads();
  const int t = threadIdx.x;
  const int64_t total = bstart[n];

  // Each block walks row blocks blk, blk + gridDim.x, ... (one when the grid
  // covers them all, as launched).
  for (int64_t blk = blockIdx.x; blk < total; blk += gridDim.x) {
    const int d = find_desc(bstart, n, blk);
    const MatvecDesc& m = table[d];
    const int64_t n_out = m.n_out, k = m.k;
    const int64_t row0 = (blk - bstart[d]) * RB;
    const int64_t row_bytes = k * SB / 8;
    const int64_t ngr = k / kGroup;
    const float* x_rot = xr + m.xr_offset;

    float acc[RB][NB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;

    for (int64_t p0 = 0; p0 < k; p0 += kPass) {
      const int64_t c0 = p0 + kChunk * t;
      if (c0 < k) {
        float xv[NB][16];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const float4* src = reinterpret_cast<const float4*>(x_rot + (b0 + b) * k + c0);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float4 v = src[i];
            xv[b][4 * i] = v.x;
            xv[b][4 * i + 1] = v.y;
            xv[b][4 * i + 2] = v.z;
            xv[b][4 * i + 3] = v.w;
          }
        }
        // All rows' codes and norms are loaded before any is used, so a
        // thread keeps RB loads in flight.  Rows past the end re-read the
        // last row; their sums are never stored.
        uint64_t codes[RB];
        float scale[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int64_t row = row0 + r < n_out ? row0 + r : n_out - 1;
          codes[r] = load_codes16<SB>(m.packed + row * row_bytes, c0);
          scale[r] = half_to_float(m.norms[row * ngr + c0 / kGroup]) * (1.0f / kGroup);
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          float v[16];
          Lv::decode(codes[r], tab, t % table_copies(NB), v);
          float part[NB];
#pragma unroll
          for (int b = 0; b < NB; ++b) part[b] = 0.0f;
#pragma unroll
          for (int e = 0; e < 16; ++e)
#pragma unroll
            for (int b = 0; b < NB; ++b) part[b] = __builtin_fmaf(v[e], xv[b][e], part[b]);
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[r][b] = __builtin_fmaf(scale[r], part[b], acc[r][b]);
        }
      }
    }

    // Block reduction in a fixed order: thread t's partials go to column t
    // of `red`; thread t then sums value t / 8 over columns 32*(t%8) ..
    // 32*(t%8)+31 and the 8 threads of a value combine by shuffles.
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) red[r * NB + b][t] = acc[r][b];
    __syncthreads();
    constexpr int V = RB * NB;  // values to reduce (<= 32)
    const int vi = t / 8, part = t % 8;
    float s = 0.0f;
    if (vi < V) {
#pragma unroll 8
      for (int i = 0; i < 32; ++i) s += red[vi][32 * part + i];
    }
    s += __shfl_xor(s, 1, kWave);
    s += __shfl_xor(s, 2, kWave);
    s += __shfl_xor(s, 4, kWave);
    if (vi < V && part == 0) {
      const int r = vi / NB, b = vi % NB;
      const int64_t row = row0 + r;
      if (row < n_out) m.y[(b0 + b) * n_out + row] = s;
    }
    __syncthreads();  // `red` is rewritten by the next row block
  }
}

// Writes a chunk of descriptors (received as kernel arguments) to the table.
__global__ void table_init_kernel(DescChunk c, MatvecDesc* __restrict__ table,
                                  int64_t* __restrict__ gstart, int64_t* __restrict__ bstart0,
                                  int64_t* __restrict__ bstart1) {
  const int i = threadIdx.x;
  if (i < c.count) table[c.first + i] = c.d[i];
  if (i < c.count + c.last_chunk) {
    gstart[c.first + i] = c.gstart[i];
    bstart0[c.first + i] = c.bstart0[i];
    bstart1[c.first + i] = c.bstart1[i];
  }
}

// y[i] = 0 for i < count (matrices whose k is 0: an empty sum).
__global__ void __launch_bounds__(kBlock) zero_kernel(float* __restrict__ y, int64_t count) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (i < count) y[i] = 0.0f;
}

// Rows per block for NB batch rows: RB * NB <= 32 keeps the accumulators in
// registers; batch 1 uses 16 (a smaller reduction buffer and more resident
// blocks measured faster than 32).
constexpr int rows_per_block(int nb) {
  return nb <= 1 ? 16 : 32 / (nb <= 2 ? 2 : nb <= 4 ? 4 : 8);
}

template <int SB, int NB>
hipError_t launch_nb(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks,
                     const LevelTable& lv, const float* xr, int64_t b0, hipStream_t s) {
  constexpr int RB = rows_per_block(NB);
  // One block per row block: the blocks are short, and letting the hardware
  // refill free slots measured faster than a resident grid that loops.
  hipLaunchKernelGGL((matvec_kernel<SB, NB, RB>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     s, table, bstart, n, lv, xr, b0);
  return hipGetLastError();
}

template <int SB>
hipError_t launch_sb(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks,
                     const LevelTable& lv, const float* xr, int64_t b0, int nb, hipStream_t s) {
  switch (nb) {
    case 1: return launch_nb<SB, 1>(table, bstart, n, blocks, lv, xr, b0, s);
    case 2: return launch_nb<SB, 2>(table, bstart, n, blocks, lv, xr, b0, s);
    case 3: return launch_nb<SB, 3>(table, bstart, n, blocks, lv, xr, b0, s);
    case 4: return launch_nb<SB, 4>(table, bstart, n, blocks, lv, xr, b0, s);
    case 5: return launch_nb<SB, 5>(table, bstart, n, blocks, lv, xr, b0, s);
    case 6: return launch_nb<SB, 6>(table, bstart, n, blocks, lv, xr, b0, s);
    case 7: return launch_nb<SB, 7>(table, bstart, n, blocks, lv, xr, b0, s);
    default: return launch_nb<SB, 8>(table, bstart, n, blocks, lv, xr, b0, s);
  }
}

}  // namespace km

int matvec_rows_per_block(int nb) { return km::rows_per_block(nb); }

hipError_t launch_rotate(const MatvecDesc* table, const int64_t* gstart, int n, int64_t total_groups,
                         float* xr, hipStream_t stream) {
  if (total_groups <= 0) return hipSuccess;
  const int64_t blocks = (total_groups + km::kBlock - 1) / km::kBlock;
  hipLaunchKernelGGL(km::rotate_kernel, dim3(static_cast<unsigned>(blocks)), dim3(km::kBlock), 0,
                     stream, table, gstart, n, xr);
  return hipGetLastError();
}

hipError_t launch_matvec(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks,
                         int sbits, const LevelTable& lv, const float* xr, int64_t b0, int nb,
                         hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  switch (sbits) {
    case 2: return km::launch_sb<2>(table, bstart, n, blocks, lv, xr, b0, nb, stream);
    case 3: return km::launch_sb<3>(table, bstart, n, blocks, lv, xr, b0, nb, stream);
    case 4: return km::launch_sb<4>(table, bstart, n, blocks, lv, xr, b0, nb, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_table_init(const DescChunk& c, MatvecDesc* table, int64_t* gstart,
                             int64_t* bstart0, int64_t* bstart1, hipStream_t stream) {
  hipLaunchKernelGGL(km::table_init_kernel, dim3(1), dim3(kDescPerInit + 1), 0, stream, c, table, gstart,
                     bstart0, bstart1);
  return hipGetLastError();
}

hipError_t launch_zero(float* y, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t blocks = (count + km::kBlock - 1) / km::kBlock;
  hipLaunchKernelGGL(km::zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(km::kBlock), 0, stream,
                     y, count);
  return hipGetLastError();
}

}  // namespace cq
