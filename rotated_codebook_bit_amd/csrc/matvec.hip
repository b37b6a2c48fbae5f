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
// Product kernel mapping: a block (4 waves) owns up to 8 groups of RB
// consecutive rows of one matrix.  Thread t owns 16-column chunks t, t + 256,
// ... of a row (one 4096-column pass per 256 chunks) and keeps the rotated
// activations of its chunk in registers for the pass; for every row it loads
// the 4 (2-bit) / 6 (3-bit) / 8 (4-bit) bytes of codes of its chunk (a wave
// instruction reads 256-512 contiguous bytes of the row), decodes four
// (2-bit) or two (4-bit) levels per LDS read from a byte table, and
// accumulates NB partial sums per row.  The block reduces each group's RB x
// NB partials through LDS in a fixed order, so results are deterministic.
//
// One batch row with 2-bit codes (a decode step), and large calls of up to 8
// rows, take matvec_pair_kernel instead, one launch per batch row: per column pair it tabulates the 16 partial products
// a 4-bit code pair can select, so the inner loop is one conflict-free LDS
// read and one add per two weights (see the comment above that kernel).

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

// xr[m][b][g][:] = H x[m][b][g][:] for every G-value group of every
// matrix's activations; one thread per group.
template <int G>
__global__ void __launch_bounds__(kBlock)
rotate_kernel(const MatvecDesc* __restrict__ table, const int64_t* __restrict__ gstart, int n,
              float* __restrict__ xr) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (g >= gstart[n]) return;
  const int d = find_desc(gstart, n, g);
  const MatvecDesc& m = table[d];
  const int64_t local = g - gstart[d];  // group within the matrix's batch*k/G
  const float* src = m.x + local * G;
  float* dst = xr + m.xr_offset + local * G;
  float y[G];
#pragma unroll
  for (int i = 0; i < G / 4; ++i) {
    const float4 v = reinterpret_cast<const float4*>(src)[i];
    y[4 * i] = v.x;
    y[4 * i + 1] = v.y;
    y[4 * i + 2] = v.z;
    y[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int h = 1; h < G; h <<= 1) {
#pragma unroll
    for (int i = 0; i < G; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = y[j], b = y[j + h];
        y[j] = a + b;
        y[j + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < G / 4; ++i)
    reinterpret_cast<float4*>(dst)[i] = make_float4(y[4 * i], y[4 * i + 1], y[4 * i + 2], y[4 * i + 3]);
}

// The same for G = 128, one wave per group, for calls with few groups (the
// thread version then leaves most of the chip idle).  Lane l holds values 2l and
// 2l + 1: butterfly stage 1 runs inside the lane, stages 2..7 between lane l
// and lane l ^ h (the lane with the bit clear keeps the sum), the same
// operations in the same order as the sequential butterfly.
__global__ void __launch_bounds__(kBlock)
rotate_wave_kernel(const MatvecDesc* __restrict__ table, const int64_t* __restrict__ gstart, int n,
              float* __restrict__ xr) {
  const int lane = threadIdx.x % kWave;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / kWave;
  if (g >= gstart[n]) return;
  const int d = find_desc(gstart, n, g);
  const MatvecDesc& m = table[d];
  const int64_t local = g - gstart[d];  // group within the matrix's batch*k/128
  const float2 v = reinterpret_cast<const float2*>(m.x + local * kGroup)[lane];
  float y0 = v.x + v.y, y1 = v.x - v.y;
#pragma unroll
  for (int h = 1; h < kWave; h <<= 1) {
    const float o0 = __shfl_xor(y0, h, kWave), o1 = __shfl_xor(y1, h, kWave);
    const bool hi = lane & h;
    y0 = hi ? o0 - y0 : y0 + o0;
    y1 = hi ? o1 - y1 : y1 + o1;
  }
  reinterpret_cast<float2*>(xr + m.xr_offset + local * kGroup)[lane] = make_float2(y0, y1);
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
    wait_lds_writes();  // the values keep their registers until stored
#pragma unroll
    for (int q = 0; q < entry; ++q) hold_values(e[q]);
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

// rg groups of RB rows x NB batch rows per block; RB * NB <= 32 keeps the
// accumulators and the activations of a chunk (16 * NB) in registers.  The
// groups of a block run one after the other, each with its own block
// reduction.  When the matrix fits one pass (k <= kPass) the thread's
// activations are loaded once for all rg groups: at batch 8 they are 8 bytes
// of L2 traffic per weight, which a 4-row block re-read for every 4 rows.
template <int SB, int NB, int RB>
__global__ void __launch_bounds__(kBlock)
matvec_kernel(const MatvecDesc* __restrict__ table, const int64_t* __restrict__ bstart, int n,
              LevelTable lv, const float* __restrict__ xr, int64_t b0, int log2g, int rg) {
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
    const int64_t row_base = (blk - bstart[d]) * RB * rg;
    const int64_t row_bytes = k * SB / 8;
    const int64_t ngr = k >> log2g;
    const float inv_g = 1.0f / static_cast<float>(1 << log2g);  // exact: a power of two
    const float* x_rot = xr + m.xr_offset;
    const bool one_pass = k <= kPass;

    float xv[NB][16];
    auto load_x = [&](int64_t c0) __attribute__((always_inline)) {
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
    };
    if (one_pass && kChunk * t < k) load_x(kChunk * t);

    for (int g = 0; g < rg; ++g) {
      const int64_t row0 = row_base + static_cast<int64_t>(g) * RB;
      if (row0 >= n_out) break;  // the same for every thread of the block

      float acc[RB][NB];
#pragma unroll
      for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;

      for (int64_t p0 = 0; p0 < k; p0 += kPass) {
        const int64_t c0 = p0 + kChunk * t;
        if (c0 < k) {
          if (!one_pass) load_x(c0);
          // All rows' codes and norms are loaded before any is used, so a
          // thread keeps RB loads in flight.  Rows past the end re-read the
          // last row; their sums are never stored.
          uint64_t codes[RB];
          float scale[RB];
#pragma unroll
          for (int r = 0; r < RB; ++r) {
            const int64_t row = row0 + r < n_out ? row0 + r : n_out - 1;
            codes[r] = load_codes16<SB>(m.packed + row * row_bytes, c0);
            scale[r] = half_to_float(m.norms[row * ngr + (c0 >> log2g)]) * inv_g;
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
      __syncthreads();  // `red` is rewritten by the next row group
    }
  }
}

// ---- One batch row, 2-bit codes: pair tables -----------------------------
//
// With one activation row, the partial product of two adjacent columns
// depends only on their 4-bit code pair:
//     P_j[v] = c[v & 3] * xr[2j] + c[v >> 2] * xr[2j + 1],   v = 0 .. 15.
// A block builds the 16 sums of every column pair of a 1024-column tile once
// and all its rows read them: one LDS read and one add per two weights,
// instead of a level read and a multiply-add per weight.
//
// Lane l of every wave owns columns 16l .. 16l + 15 of the tile (pairs
// q = 0 .. 7).  Entry (q, v, l) sits at float (16q + v) * 64 + l, so in any
// read instruction lane l touches bank l (mod the bank count) whatever its
// codes: the lookups are free of bank conflicts.  The byte address is
// 4096 q + 256 v + 4 l; q is a compile-time offset, and 256 v + 4 l is one
// byte permute of the code word (its nibbles first spread one per byte) and
// the lane's byte.
//
// A block is kPairWaves waves over consecutive rows of one matrix (16 per
// wave, or kPairRowsPerWaveFew for calls with few rows); each wave keeps its
// rows' sums in registers across the tiles and reduces them over its lanes
// at the end.  Summation order is fixed, so results are deterministic.
constexpr int kPairWaves = 8;
constexpr int kPairRowsPerWave = 16;
// Rows per wave for calls whose 128-row blocks would not give every CU two:
// more, shorter blocks.
constexpr int kPairRowsPerWaveFew = 4;
constexpr int log2i(int v) { return v <= 1 ? 0 : 1 + log2i(v / 2); }
constexpr int kPairTile = kWave * kChunk;  // 1024 columns per tile

__device__ __forceinline__ __amdgpu_buffer_rsrc_t pair_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// Eight waves per SIMD: at most 64 VGPRs (the 16-row kernel needs 65
// unconstrained; capped, it spills two SGPRs into VGPR lanes), so four
// 32 KiB blocks fit a CU instead of three.  The latency of the small code
// loads is hidden by resident waves: 2.6% faster on the 225-matrix pass,
// while loading the next tile ahead (115 VGPRs, two blocks) was 11% slower.
template <int W, int RPW>
__global__ void __launch_bounds__(W * kWave, 8)
matvec_pair_kernel(const MatvecDesc* __restrict__ table, const int64_t* __restrict__ bstart, int n,
                   LevelTable lv, const float* __restrict__ xr, int64_t b0, int log2g) {
  __shared__ __attribute__((aligned(16))) float tab[8 * 16 * kWave];
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t blk = blockIdx.x;  // one block per row block
  const int d = find_unit(bstart, 0, n, blk);
  const MatvecDesc* md = table + d;
  const int64_t n_out = load_const(&md->n_out), k = load_const(&md->k);
  const int64_t row0 = (blk - load_const(bstart + d)) * (W * RPW) + w * RPW;
  const int64_t row_bytes = k / 4, ngr = k >> log2g;
  const float* x_rot = xr + load_const(&md->xr_offset) + b0 * k;
  // The wave's rows as buffer resources: rows past the end of the matrix lie
  // outside them and read as zero (their sums are never stored).  The host
  // sends a matrix here only when k <= 2^28, so 16 rows of codes (4 k bytes)
  // and every offset below stay under 2^31.
  const int64_t rows_in = n_out - row0 < RPW ? (n_out - row0 > 0 ? n_out - row0 : 0) : RPW;
  const auto codes_src = pair_rsrc(load_const(&md->packed) + (rows_in ? row0 * row_bytes : 0), rows_in * row_bytes);
  const auto norms_src = pair_rsrc(load_const(&md->norms) + (rows_in ? row0 * ngr : 0), rows_in * ngr * 2);
  const float c0l = lv.c[0], c1l = lv.c[1], c2l = lv.c[2], c3l = lv.c[3];
  const uint32_t lane_bytes = 4u * static_cast<uint32_t>(lane);

  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;

  // Tile inputs: the activations of the PPT pairs this thread tabulates
  // (pairs PPT w .. PPT w + PPT - 1 of lane `lane`'s chunk), and for each of
  // the wave's rows the codes of this lane's 16 columns and the norm of
  // their group.  The whole buffer offset goes in the range-checked vector
  // operand; a lane without columns in the tile offsets by 2^30, past every
  // resource (at most 4 k <= 2^30 bytes), and reads zero.
  constexpr int PPT = W >= 8 ? 1 : 8 / W;
  const bool builds = PPT * w < 8;  // with more than 8 waves, waves 8.. only read
  struct Tile {
    float2 x[PPT];
    uint32_t codes[RPW];
    _Float16 norm[RPW];
  };
  // Row r of the wave reads at scalar offset r * row_bytes; rows past the
  // end of the matrix re-read its last row (their sums are never stored), so
  // every in-range access lies inside the matrix.
  int soff_c[RPW], soff_n[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int rr = r < rows_in ? r : (rows_in > 0 ? static_cast<int>(rows_in) - 1 : 0);
    soff_c[r] = __builtin_amdgcn_readfirstlane(static_cast<int>(rr * row_bytes));
    soff_n[r] = __builtin_amdgcn_readfirstlane(static_cast<int>(2 * rr * ngr));
  }
  auto load_x = [&](int64_t p0, Tile& t) {
    const int64_t c0 = p0 + kChunk * lane;
    const bool active = c0 < k;  // k % 128 == 0: whole chunks only
#pragma unroll
    for (int h = 0; h < PPT; ++h)
      t.x[h] = active && builds ? *reinterpret_cast<const float2*>(x_rot + c0 + 2 * (PPT * w + h))
                                : make_float2(0.0f, 0.0f);
  };
  auto load_codes = [&](int64_t p0, Tile& t) {
    const int64_t c0 = p0 + kChunk * lane;
    const bool active = c0 < k;
    const int coff = active ? static_cast<int>(c0 / 4) : (1 << 30);
    const int noff = active ? static_cast<int>(2 * (c0 >> log2g)) : (1 << 30);
    // The codes are read once: loaded non-temporal (aux bit nt), they leave
    // the L2 to the activations every row block re-reads (4.6% faster on the
    // 225-matrix pass; nt on the norms as well was 3% slower).
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      t.codes[r] = __builtin_amdgcn_raw_buffer_load_b32(codes_src, coff, soff_c[r], 2);
      t.norm[r] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(norms_src, noff, soff_n[r], 0));
    }
  };
  auto step = [&](int64_t p0, Tile& t) {
    const bool active = p0 + kChunk * lane < k;
    __syncthreads();  // the previous tile's reads are done
    if (active && builds) {
#pragma unroll
      for (int h = 0; h < PPT; ++h) {
        const float x0 = t.x[h].x, x1 = t.x[h].y;
        const float pa[4] = {c0l * x0, c1l * x0, c2l * x0, c3l * x0};
        const float cb[4] = {c0l, c1l, c2l, c3l};
        float* dst = tab + (16 * (PPT * w + h)) * kWave + lane;
        // The 16 entries keep their registers until the LDS has them.  The
        // tile's codes and norms are loaded only after this, so the held
        // entries fit the 64-VGPR budget without spilling (held four at a
        // time with the codes already in flight, one register spilled and
        // the 225-matrix pass took 0.415 ms; this way 0.392, unguarded 0.374).
        float e[16];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
          for (int a = 0; a < 4; ++a) e[a + 4 * bb] = __builtin_fmaf(cb[bb], x1, pa[a]);
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[v * kWave] = e[v];
        wait_lds_writes();
#pragma unroll
        for (int v = 0; v < 16; ++v) hold_values(e[v]);
      }
    }
    load_codes(p0, t);  // in flight across the barrier
    __syncthreads();
    if (active) {
      const char* tb = reinterpret_cast<const char*>(tab);
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        // Pair q's nibble is byte q/2 of `ev` (q even) or of `od` (q odd).
        const uint32_t ev = t.codes[r] & 0x0F0F0F0Fu, od = (t.codes[r] >> 4) & 0x0F0F0F0Fu;
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          // Byte 0 of the address is the lane's (4 l), byte 1 is byte q/2
          // of the spread nibbles (v), bytes 2 and 3 are zero (selector 12).
          const uint32_t e = (q & 1) ? od : ev;
          const uint32_t addr = __builtin_amdgcn_perm(e, lane_bytes, 0x0C0C0000u | ((4u + (q >> 1)) << 8));
          const float v = *reinterpret_cast<const float*>(tb + addr + 4096 * q);
          s = q ? s + v : v;
        }
        // norm * s here, and the exact power-of-two 1/128 once at the end.
        acc[r] = __builtin_fmaf(static_cast<float>(t.norm[r]), s, acc[r]);
      }
    }
  };

  for (int64_t p0 = 0; p0 < k; p0 += kPairTile) {
    Tile cur;
    load_x(p0, cur);
    step(p0, cur);
  }

  // Reduce the RPW row sums over the 64 lanes: each exchange halves the
  // values a lane holds (the lane with the offset's bit set keeps the upper
  // half), then the remaining offsets sum within groups of 64 / RPW lanes.
  // With RPW = 16, lane l ends with row 8*b5 + 4*b4 + 2*b3 + b2 of its wave
  // (b_i = bit i of l).  Both halves are summed and one is kept, so every
  // select has constant operands (the two partners add the same two values,
  // in either order).
  constexpr int kSteps = log2i(RPW);
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int o = 32 >> i, V = RPW >> i;
    const bool hi = lane & o;
#pragma unroll
    for (int j = 0; j < V / 2; ++j) {
      const float lo_sum = acc[j] + __shfl_xor(acc[j], o, kWave);
      const float hi_sum = acc[j + V / 2] + __shfl_xor(acc[j + V / 2], o, kWave);
      acc[j] = hi ? hi_sum : lo_sum;
    }
  }
  float s = acc[0];
#pragma unroll
  for (int o = 32 >> kSteps; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
  s *= 1.0f / static_cast<float>(1 << log2g);  // exact: a power of two
  int r = 0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) r += ((lane >> (5 - i)) & 1) * (RPW >> (i + 1));
  if ((lane & (64 / RPW - 1)) == 0 && row0 + r < n_out) load_const(&md->y)[b0 * n_out + row0 + r] = s;
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

// Most row groups per block of the byte-table kernel.
constexpr int kMaxRowGroups = 8;

// 2-bit codes with one batch row take the pair-table kernel when a wave's 16
// rows of codes (4 k bytes) fit its 32-bit buffer range.
constexpr int64_t kPairMaxK = int64_t(1) << 28;
constexpr bool use_pairs(int sb, int nb, int64_t max_k) { return sb == 2 && nb == 1 && max_k <= kPairMaxK; }
// Large calls of 2 to kPairMaxBatch batch rows with 2-bit codes run the
// pair-table kernel once per row, reading the codes once per row; other
// calls take the byte-table kernel eight rows at a time.  Call times on
// subsets of the 7B-shaped model's matrices, per-row pairs / byte table (us):
// 11 MB of codes: batch 2 43-46 / 42, batch 8 78-83 / 50; 51 MB: batch 2
// 55-56 / 72, batch 4 99-105 / 102, batch 8 185-235 / 142; 202 MB: batch 2
// 158-160 / 196, batch 4 306-308 / 267, batch 8 594-603 / 499; 1.65 GB:
// batch 2 823-907 / 1090, batch 4 1577-1594 / 1922, batch 8 3069-3084 / 3686.
// A pair launch costs about bytes / 4.3 TB/s + 28 us there, the byte table
// about 1.16 (batch 4) to 2.23 (batch 8) us per MB, which puts the switch
// for batches 3-8 at 480-610 MB; batch 2 switches between 11 and 51 MB.
constexpr int64_t kPairMaxBatch = 8;
constexpr int64_t kPairMinBytesBatch2 = int64_t(32) << 20;
constexpr int64_t kPairMinBytes = int64_t(512) << 20;

template <int SB, int NB>
hipError_t launch_nb(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks,
                     const LevelTable& lv, const float* xr, int64_t b0, int log2g, int rg, hipStream_t s) {
  constexpr int RB = rows_per_block(NB);
  // One block per row block: the blocks are short, and letting the hardware
  // refill free slots measured faster than a resident grid that loops.
  hipLaunchKernelGGL((matvec_kernel<SB, NB, RB>), dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0,
                     s, table, bstart, n, lv, xr, b0, log2g, rg);
  return hipGetLastError();
}

template <int SB>
hipError_t launch_sb(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks,
                     const LevelTable& lv, const float* xr, int64_t b0, int nb, int log2g, int rg,
                     hipStream_t s) {
  switch (nb) {
    case 1: return launch_nb<SB, 1>(table, bstart, n, blocks, lv, xr, b0, log2g, rg, s);
    case 2: return launch_nb<SB, 2>(table, bstart, n, blocks, lv, xr, b0, log2g, rg, s);
    case 3: return launch_nb<SB, 3>(table, bstart, n, blocks, lv, xr, b0, log2g, rg, s);
    case 4: return launch_nb<SB, 4>(table, bstart, n, blocks, lv, xr, b0, log2g, rg, s);
    case 5: return launch_nb<SB, 5>(table, bstart, n, blocks, lv, xr, b0, log2g, rg, s);
    case 6: return launch_nb<SB, 6>(table, bstart, n, blocks, lv, xr, b0, log2g, rg, s);
    case 7: return launch_nb<SB, 7>(table, bstart, n, blocks, lv, xr, b0, log2g, rg, s);
    default: return launch_nb<SB, 8>(table, bstart, n, blocks, lv, xr, b0, log2g, rg, s);
  }
}

template <int G>
void launch_rotate_threads(const MatvecDesc* table, const int64_t* gstart, int n, int64_t total_groups,
                           float* xr, hipStream_t stream) {
  const int64_t blocks = (total_groups + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(rotate_kernel<G>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream, table,
                     gstart, n, xr);
}

constexpr int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 256 ? 8 : 7; }

}  // namespace km

namespace {
// Whether a launch of nb batch rows takes the matrix-core kernel: 3 to 8
// rows when every matrix qualifies.  Whole-call times on the 7B-shaped
// model's matrices (us), matrix cores / the kernels before them: batch 8, all
// 225 matrices 2316 / 3179 (per-row pairs), one layer 108 / 152 (byte
// table); batch 4, all 1493 / 1670 (pairs), one layer 87 / 110 (byte table);
// batch 2, all 1469 / 861 (pairs), one layer 87 / 61 (pairs).  With one or
// two live batch rows of a 4-row chunk the matrix cores do 2-4 times the
// useful work, so batch 2 keeps the pair and byte-table kernels.
bool use_mfma(int nb, const MatvecDesc* descs, int n) {
  if (nb < 3) return false;
  for (int i = 0; i < n; ++i)
    if (!mfma_fits(descs[i].k)) return false;
  return true;
}
}  // namespace

int matvec_chunk(int sbits, int64_t batch, const MatvecDesc* descs, int n) {
  if (use_mfma(batch < 8 ? static_cast<int>(batch) : 8, descs, n)) return 8;
  int64_t max_k = 0;
  for (int i = 0; i < n; ++i) max_k = descs[i].k > max_k ? descs[i].k : max_k;
  if (sbits != 2 || max_k > km::kPairMaxK || batch > km::kPairMaxBatch) return 8;
  int64_t bytes = 0;  // 2-bit codes: k / 4 bytes per row
  for (int i = 0; i < n; ++i) bytes += descs[i].n_out * (descs[i].k / 4);
  if (batch == 1 || bytes >= km::kPairMinBytes) return 1;
  return batch == 2 && bytes >= km::kPairMinBytesBatch2 ? 1 : 8;
}

MatvecPlan matvec_plan(int sbits, int nb, const MatvecDesc* descs, int n) {
  if (use_mfma(nb, descs, n)) {
    // Matrix-core kernel: one block of up to 48 rows per compute unit at a
    // time; fewer rows per block when the call has too few rows to give
    // every CU one.
    int64_t rows = 0;
    for (int i = 0; i < n; ++i) rows += descs[i].n_out;
    const int64_t cus = device_cu_count();
    const int64_t cap = mfma_rows_cap(sbits, nb);
    int64_t rpb = (rows + cus - 1) / cus;
    rpb = rpb < 1 ? 1 : rpb > cap ? cap : rpb;
    // Calls of at least 16 row blocks per CU take 2048-column passes: half
    // the LDS, so two blocks share a CU and one's activation load and
    // reduction overlap the other's products (all 225 matrices of the
    // 7B-shaped model at batch 8: 2315 against 2659 us).  Smaller calls keep
    // 4096-column passes (one layer: 109 against 122 us; one 11008x4096
    // matrix: 41 against 45 us), whose single pass lets 4096-column rows
    // scale each accumulator once.
    int64_t blocks = 0;
    for (int i = 0; i < n; ++i) blocks += (descs[i].n_out + rpb - 1) / rpb;
    const int pass = blocks >= 16 * cus ? 2048 : 4096;
    return MatvecPlan{static_cast<int>(rpb), 0, 1, pass};
  }
  int64_t max_k = 0;
  for (int i = 0; i < n; ++i) max_k = descs[i].k > max_k ? descs[i].k : max_k;
  if (!km::use_pairs(sbits, nb, max_k)) {
    // Byte-table kernel: the most row groups per block (8, 4, 2) that still
    // give every CU two blocks.
    const int rb = km::rows_per_block(nb);
    for (int rg = km::kMaxRowGroups; rg > 1; rg /= 2) {
      int64_t blocks = 0;
      for (int i = 0; i < n; ++i) blocks += (descs[i].n_out + rb * rg - 1) / (rb * rg);
      if (blocks >= 2 * static_cast<int64_t>(device_cu_count())) return MatvecPlan{rb * rg, 0};
    }
    return MatvecPlan{rb, 0};
  }
  constexpr int many = km::kPairWaves * km::kPairRowsPerWave;
  int64_t blocks = 0;
  for (int i = 0; i < n; ++i) blocks += (descs[i].n_out + many - 1) / many;
  const int rpw = blocks >= 2 * static_cast<int64_t>(device_cu_count()) ? km::kPairRowsPerWave
                                                                         : km::kPairRowsPerWaveFew;
  return MatvecPlan{km::kPairWaves * rpw, rpw};
}

hipError_t launch_rotate(const MatvecDesc* table, const int64_t* gstart, int n, int64_t total_groups,
                         int group_size, float* xr, hipStream_t stream) {
  if (total_groups <= 0) return hipSuccess;
  if (group_size == kGroup && total_groups < kFewUnits) {  // a wave per group
    const int64_t blocks = (total_groups + km::kWaves - 1) / km::kWaves;
    hipLaunchKernelGGL(km::rotate_wave_kernel, dim3(static_cast<unsigned>(blocks)), dim3(km::kBlock), 0,
                       stream, table, gstart, n, xr);
    return hipGetLastError();
  }
  switch (group_size) {  // a thread per group
    case 32: km::launch_rotate_threads<32>(table, gstart, n, total_groups, xr, stream); break;
    case 64: km::launch_rotate_threads<64>(table, gstart, n, total_groups, xr, stream); break;
    case 128: km::launch_rotate_threads<128>(table, gstart, n, total_groups, xr, stream); break;
    case 256: km::launch_rotate_threads<256>(table, gstart, n, total_groups, xr, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_matvec(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks,
                         int sbits, const LevelTable& lv, const float* xr, int64_t b0, int nb,
                         const MatvecPlan& plan, int group_size, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  const int log2g = km::log2_group(group_size);
  if ((1 << log2g) != group_size) return hipErrorInvalidValue;
  if (plan.mfma)
    return launch_mfma_many(table, bstart, n, blocks, sbits, lv, xr, b0, nb, log2g, plan.rows_per_block,
                            plan.mfma_pass, stream);
  if (plan.pair_rows_per_wave == km::kPairRowsPerWave) {
    hipLaunchKernelGGL((km::matvec_pair_kernel<km::kPairWaves, km::kPairRowsPerWave>),
                       dim3(static_cast<unsigned>(blocks)), dim3(km::kPairWaves * kWave), 0, stream, table, bstart,
                       n, lv, xr, b0, log2g);
    return hipGetLastError();
  }
  if (plan.pair_rows_per_wave == km::kPairRowsPerWaveFew) {
    hipLaunchKernelGGL((km::matvec_pair_kernel<km::kPairWaves, km::kPairRowsPerWaveFew>),
                       dim3(static_cast<unsigned>(blocks)), dim3(km::kPairWaves * kWave), 0, stream, table, bstart,
                       n, lv, xr, b0, log2g);
    return hipGetLastError();
  }
  const int rb = km::rows_per_block(nb);
  const int rg = plan.rows_per_block / rb;
  if (plan.pair_rows_per_wave != 0 || plan.rows_per_block % rb || rg < 1 || rg > km::kMaxRowGroups)
    return hipErrorInvalidValue;
  switch (sbits) {
    case 2: return km::launch_sb<2>(table, bstart, n, blocks, lv, xr, b0, nb, log2g, rg, stream);
    case 3: return km::launch_sb<3>(table, bstart, n, blocks, lv, xr, b0, nb, log2g, rg, stream);
    case 4: return km::launch_sb<4>(table, bstart, n, blocks, lv, xr, b0, nb, log2g, rg, stream);
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
