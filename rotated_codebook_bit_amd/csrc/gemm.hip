// CQ dequantize-GEMM on the matrix cores (gfx950 MFMA), for batched
// products y = x . W_hat^T such as a prefill pass over every weight matrix.
//
// The pages run quantized weights in an ordinary forward product ("Performance
// Differences Between 2-Bit and 4-Bit Quantization in Needle", section
// Practical Code Comparison) and decode packed tensors at run time ("How Needle
// 2 Model Compresses to a Single Binary", section Stage 3).  As in the matvec,
// the activations are rotated instead of the weights: the orthonormal Hadamard
// matrix is symmetric and self-inverse, so for group g of row n
//     x_g . W_hat_g = (norm_ng / G) * < H x_g , levels[idx_ng] >
// with H the +-1 Sylvester matrix.  What remains is a dense contraction of the
// rotated activations with the looked-up levels, scaled per (row, group).
//
// Arithmetic.  Operands are split into two bf16 halves, v = hi + lo with
// hi = bf16(v) and lo = bf16(v - hi) (both round to nearest even), and each
// product is taken as hi*hi + hi*lo + lo*hi with float32 accumulation: three
// bf16 MFMAs per product.  Each split operand is within 2^-16 (relative) of
// its float32 value, so each product carries at most about 3 * 2^-16 relative
// error, and a whole output at most about 5e-5 * ||x_b|| * ||W_hat_n||.
//
// Kernels.
//   split_rotate_kernel: one thread per (matrix, group, padded batch row)
//     (split_rotate_wave_kernel: one wave, for calls with few of them at
//     G = 128): writes H x_g as hi and lo bf16 values to the workspace, laid
//     out [group][row][hi 128 | lo 128] so that the 64-row tile of a group is
//     32 KiB of contiguous memory; rows past the batch are zeros.
//   gemm_kernel: a block computes a 64 (batch) x 256 (outputs) tile of one
//     matrix; wave w owns outputs [64w, 64w + 64) as 2 x 2 tiles of 32 x 32
//     (batches of at most 32: 32 x 256 tiles, 1 x 2 per wave).
//     Per 128-value group:
//       - the group's activation tile moves HBM -> LDS by direct-to-LDS DMA
//         (double-buffered: the next group's DMA runs under this group's
//         MFMAs); chunk c of row r sits in slot c ^ (r & 15) so the fragment
//         reads are conflict-free;
//       - every lane holds the packed codes of its output column, prefetched
//         one group ahead; one LDS read from a byte table yields the bf16 hi
//         and lo level values of four (2-bit) codes;
//       - 8 steps of 16 values, 3 MFMAs (32x32x16 bf16) per step and tile,
//         into a per-group accumulator that is then scaled by norm/G and added
//         to the output accumulator.
//     Blocks are numbered so that consecutive blocks of a matrix share their
//     weight tile, and the numbering is laid out so that such runs of blocks
//     execute on the same XCD and share its L2.
//   When a call has too few output tiles to give every CU two blocks (one
//   matrix at a small batch, say), each tile's 128-groups are split into
//   ranges, one block each, that write partial sums to the workspace, and
//   gemm_reduce_kernel adds them in range order (deterministic results).

#include "cq_internal.h"

namespace cq {
namespace kg {

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;
constexpr int BN = 256;           // outputs per block
constexpr int TN = 2;             // 32 x 32 tiles per wave along the outputs
constexpr int kRowBytes = 512;    // one workspace row of a group: 128 hi + 128 lo bf16
// Rows per block: TM x 32 with TM = 2 (64 rows), or TM = 1 (32 rows) for
// batches of at most 32, which halves the work spent on padding rows, and
// at group size 32, whose 64-row kernel would not fit its registers.
constexpr int block_rows(int64_t batch, int group_size) { return batch <= 32 || group_size < 64 ? 32 : 64; }
constexpr int kXcds = 8;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima; on gfx9 the
// vector-memory count is split over bits 3:0 and 15:14).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_value(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

// Work-unit prefix search, as find_unit but over a per-lane value (vector
// loads).
__device__ __forceinline__ int find_lane(const int64_t* __restrict__ start, int n, int64_t v) {
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

// Rotated, split activations in 128-column tiles:
//   ws[xs_off + (t * mpad + m) * 256 + (0..127 | 128..255)] = hi | lo of
//   columns 128 t .. 128 t + 127 of (H x_g for each G-group g) in row m.
// One thread per (G-group, padded row); a 256-group fills two tiles, a
// smaller one part of a tile.
template <int G>
__global__ void __launch_bounds__(kBlock)
split_rotate_kernel(const GemmDesc* __restrict__ table, const int64_t* __restrict__ ustart, int n,
                    int64_t batch, uint16_t* __restrict__ ws) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (u >= ustart[n]) return;
  const int d = find_lane(ustart, n, u);
  const GemmDesc& m = table[d];
  const int64_t local = u - ustart[d];
  const int64_t g = local / m.mpad, row = local - g * m.mpad;
  float y[G];
  if (row < batch) {
    const float4* src = reinterpret_cast<const float4*>(m.x + row * m.k + g * G);
#pragma unroll
    for (int i = 0; i < G / 4; ++i) {
      const float4 v = src[i];
      y[4 * i] = v.x;
      y[4 * i + 1] = v.y;
      y[4 * i + 2] = v.z;
      y[4 * i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < G; ++i) y[i] = 0.0f;
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
  uint32_t hi[G / 2], lo[G / 2];
#pragma unroll
  for (int i = 0; i < G; i += 2) {
    const uint32_t h0 = bf16_rne_bits(y[i]), h1 = bf16_rne_bits(y[i + 1]);
    const uint32_t l0 = bf16_rne_bits(y[i] - bf16_value(h0)), l1 = bf16_rne_bits(y[i + 1] - bf16_value(h1));
    hi[i / 2] = h0 | (h1 << 16);
    lo[i / 2] = l0 | (l1 << 16);
  }
  constexpr int W = G < kGroup ? G : kGroup;  // values per tile piece
  const int64_t c0 = g * G;                   // first column of the group
#pragma unroll
  for (int piece = 0; piece < G / W; ++piece) {
    const int64_t c = c0 + piece * W;
    uint16_t* dst = ws + m.xs_off + ((c / kGroup) * m.mpad + row) * 256 + c % kGroup;
    uint4* dh = reinterpret_cast<uint4*>(dst);
    uint4* dl = reinterpret_cast<uint4*>(dst + kGroup);
    const int o = piece * (W / 2);  // first packed word of the piece
#pragma unroll
    for (int i = 0; i < W / 8; ++i) {
      dh[i] = make_uint4(hi[o + 4 * i], hi[o + 4 * i + 1], hi[o + 4 * i + 2], hi[o + 4 * i + 3]);
      dl[i] = make_uint4(lo[o + 4 * i], lo[o + 4 * i + 1], lo[o + 4 * i + 2], lo[o + 4 * i + 3]);
    }
  }
}

// The same, one wave per (group, padded row), for calls with few units.  Lane l holds values 2l and 2l + 1:
// butterfly stage 1 inside the lane, stages 2..7 between lane l and lane
// l ^ h (the lane with the bit clear keeps the sum), the same operations in
// the same order as the sequential butterfly.  Rows past the batch are zero.
__global__ void __launch_bounds__(kBlock)
split_rotate_wave_kernel(const GemmDesc* __restrict__ table, const int64_t* __restrict__ ustart, int n,
                    int64_t batch, uint16_t* __restrict__ ws) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kWaves + threadIdx.x / kWave;
  if (u >= ustart[n]) return;  // whole waves
  const int d = find_lane(ustart, n, u);
  const GemmDesc& m = table[d];
  const int64_t local = u - ustart[d];
  const int64_t g = local / m.mpad, row = local - g * m.mpad;
  float2 v = make_float2(0.0f, 0.0f);
  if (row < batch) v = reinterpret_cast<const float2*>(m.x + row * m.k + g * kGroup)[lane];
  float y0 = v.x + v.y, y1 = v.x - v.y;
#pragma unroll
  for (int h = 1; h < kWave; h <<= 1) {
    const float o0 = __shfl_xor(y0, h, kWave), o1 = __shfl_xor(y1, h, kWave);
    const bool up = lane & h;
    y0 = up ? o0 - y0 : y0 + o0;
    y1 = up ? o1 - y1 : y1 + o1;
  }
  const uint32_t h0 = bf16_rne_bits(y0), h1 = bf16_rne_bits(y1);
  const uint32_t l0 = bf16_rne_bits(y0 - bf16_value(h0)), l1 = bf16_rne_bits(y1 - bf16_value(h1));
  uint32_t* dst = reinterpret_cast<uint32_t*>(ws + m.xs_off + local * 256);
  dst[lane] = h0 | (h1 << 16);
  dst[64 + lane] = l0 | (l1 << 16);
}

// Byte tables in LDS.  SB = 2: entry b (a code byte, four codes) holds the
// bf16 hi values of the four levels in .x/.y and the lo values in .z/.w;
// SB = 4: entry b (two codes) holds the hi pair in .x and the lo pair in .y;
// SB = 3: entry p (a 6-bit pair of codes) likewise.
template <int SB>
struct Table {
  static constexpr int entries = SB == 3 ? 64 : 256;
  static constexpr int words = SB == 2 ? 4 : 2;
};

__device__ __forceinline__ uint32_t split_at(const SplitLevels& s, int i, bool lo) {
  uint32_t v = 0;
#pragma unroll
  for (int j = 0; j < kMaxLevels; ++j) v = (i == j) ? (lo ? s.lo[j] : s.hi[j]) : v;
  return v;
}

template <int SB>
__device__ __forceinline__ void fill_table(uint32_t* tab, const SplitLevels& s, int t) {
  if (t >= Table<SB>::entries) return;
  if constexpr (SB == 2) {
    const int c0 = t & 3, c1 = (t >> 2) & 3, c2 = (t >> 4) & 3, c3 = t >> 6;
    // hi pairs in the first 512 words, lo pairs in the next 512
    const uint32_t h0 = split_at(s, c0, false) | (split_at(s, c1, false) << 16);
    const uint32_t h1 = split_at(s, c2, false) | (split_at(s, c3, false) << 16);
    const uint32_t l0 = split_at(s, c0, true) | (split_at(s, c1, true) << 16);
    const uint32_t l1 = split_at(s, c2, true) | (split_at(s, c3, true) << 16);
    tab[2 * t] = h0;
    tab[2 * t + 1] = h1;
    tab[512 + 2 * t] = l0;
    tab[512 + 2 * t + 1] = l1;
    wait_lds_writes();  // the values keep their registers until stored
    hold_values(h0, h1, l0, l1);
  } else {
    const int c0 = SB == 4 ? (t & 15) : (t & 7), c1 = SB == 4 ? (t >> 4) : (t >> 3);
    const uint32_t h = split_at(s, c0, false) | (split_at(s, c1, false) << 16);
    const uint32_t l = split_at(s, c0, true) | (split_at(s, c1, true) << 16);
    tab[2 * t] = h;
    tab[2 * t + 1] = l;
    wait_lds_writes();
    hold_values(h, l);
  }
}

// Packed codes of one group of one row: 16 * SB bytes = 4 * SB dwords.
template <int SB>
struct Codes {
  uint32_t w[4 * SB];
};

template <int SB>
__device__ __forceinline__ void load_codes(const uint8_t* __restrict__ p, Codes<SB>& c) {
#pragma unroll
  for (int i = 0; i < SB; ++i) {
    const uint4 v = reinterpret_cast<const uint4*>(p)[i];
    c.w[4 * i] = v.x;
    c.w[4 * i + 1] = v.y;
    c.w[4 * i + 2] = v.z;
    c.w[4 * i + 3] = v.w;
  }
}

// B-operand fragments (bf16 hi and lo levels) of step s for this lane: the
// 8 codes of values 16 s + 8 h .. 16 s + 8 h + 7 of the group (h = lane / 32).
template <int SB>
__device__ __forceinline__ void decode(const Codes<SB>& c, int s, int h, const uint32_t* tab,
                                       bf16x8& bh, bf16x8& bl) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 H, L;
  if constexpr (SB == 2) {
    // Two 8-byte reads per operand, straight into its register quadruple.
    const uint32_t pair = (c.w[s] >> (16 * h)) & 0xFFFFu;
    const uint2 h0 = reinterpret_cast<const uint2*>(tab)[pair & 0xFFu];
    const uint2 h1 = reinterpret_cast<const uint2*>(tab)[pair >> 8];
    const uint2 l0 = reinterpret_cast<const uint2*>(tab + 512)[pair & 0xFFu];
    const uint2 l1 = reinterpret_cast<const uint2*>(tab + 512)[pair >> 8];
    H = u32x4{h0.x, h0.y, h1.x, h1.y};
    L = u32x4{l0.x, l0.y, l1.x, l1.y};
  } else if constexpr (SB == 4) {
    const uint32_t q = h ? c.w[2 * s + 1] : c.w[2 * s];
    const uint2 e0 = reinterpret_cast<const uint2*>(tab)[q & 0xFFu];
    const uint2 e1 = reinterpret_cast<const uint2*>(tab)[(q >> 8) & 0xFFu];
    const uint2 e2 = reinterpret_cast<const uint2*>(tab)[(q >> 16) & 0xFFu];
    const uint2 e3 = reinterpret_cast<const uint2*>(tab)[q >> 24];
    H = u32x4{e0.x, e1.x, e2.x, e3.x};
    L = u32x4{e0.y, e1.y, e2.y, e3.y};
  } else {
    // 24 bits at bit 48 s + 24 h of the group's stream.
    const int o0 = 48 * s, o1 = 48 * s + 24;
    const uint32_t lo0 = c.w[o0 / 32], hi0 = (o0 / 32 + 1 < 12) ? c.w[o0 / 32 + 1] : 0u;
    const uint32_t lo1 = c.w[o1 / 32], hi1 = (o1 / 32 + 1 < 12) ? c.w[o1 / 32 + 1] : 0u;
    const uint32_t v0 = __builtin_amdgcn_alignbit(hi0, lo0, o0 % 32);
    const uint32_t v1 = __builtin_amdgcn_alignbit(hi1, lo1, o1 % 32);
    const uint32_t v = h ? v1 : v0;
    const uint2 e0 = reinterpret_cast<const uint2*>(tab)[v & 63u];
    const uint2 e1 = reinterpret_cast<const uint2*>(tab)[(v >> 6) & 63u];
    const uint2 e2 = reinterpret_cast<const uint2*>(tab)[(v >> 12) & 63u];
    const uint2 e3 = reinterpret_cast<const uint2*>(tab)[(v >> 18) & 63u];
    H = u32x4{e0.x, e1.x, e2.x, e3.x};
    L = u32x4{e0.y, e1.y, e2.y, e3.y};
  }
  bh = __builtin_bit_cast(bf16x8, H);
  bl = __builtin_bit_cast(bf16x8, L);
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// G: the quantization group size.  The K loop runs over 128-column tiles
// either way; a tile holds 128 / G groups (G <= 128), each scaled by its own
// norm after its G / 16 MFMA steps, or half of a 256-group (scaled by that
// group's norm, the scale distributing over the two halves).
template <int SB, int TM, int G>
__global__ void __launch_bounds__(kBlock, G < kGroup ? 1 : 2)  // G < 128: more live norms and sums
gemm_kernel(const GemmDesc* __restrict__ table, const int64_t* __restrict__ bstart, int n,
            SplitLevels sl, const uint8_t* __restrict__ ws, int64_t batch) {
  constexpr int BM = 32 * TM;                 // batch rows per block
  constexpr int kTileBytes = BM * kRowBytes;  // 16 or 32 KiB per group
  constexpr int kDmaPerWave = BM / 8;         // 1 KiB DMA instructions per wave per tile
  // Two tile buffers as separate objects, each access naming one of them, so
  // the compiler can tell the next tile's DMA from this tile's reads and does
  // not wait for the former before the latter.
  __shared__ __attribute__((aligned(16))) uint8_t xt0[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t xt1[kTileBytes];
  __shared__ __attribute__((aligned(16))) uint32_t tab[Table<SB>::entries * Table<SB>::words];
  fill_table<SB>(tab, sl, threadIdx.x);

  // Logical block: runs of consecutive logical blocks execute on one XCD
  // (the hardware deals blocks to the XCDs round-robin).
  const int64_t total = load_const(bstart + n);
  const int64_t per_xcd = (total + kXcds - 1) / kXcds;
  const int64_t lb = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (lb >= total) return;
  const int d = find_unit(bstart, 0, n, lb);
  const GemmDesc* md = table + d;
  const uint8_t* const packed = load_const(&md->packed);
  const uint16_t* const norms = load_const(&md->norms);
  float* const y = load_const(&md->y);
  const int64_t n_out = load_const(&md->n_out), k = load_const(&md->k);
  const int64_t mpad = load_const(&md->mpad), xs_off = load_const(&md->xs_off);
  const int64_t mtiles = mpad / BM;
  const int64_t ksplit = load_const(&md->ksplit), gps = load_const(&md->gps);
  float* const part = load_const(&md->part);
  const int64_t local = lb - load_const(bstart + d);
  const int64_t ks = local % ksplit, tile = local / ksplit;
  const int64_t nt = tile / mtiles, mt = tile - nt * mtiles;  // consecutive blocks share nt
  const int64_t ngr = k / kGroup;  // 128-column tiles
  constexpr int NPT = G <= kGroup ? kGroup / G : 1;  // norms per tile
  constexpr int SPG = G <= kGroup ? G / 16 : 8;      // MFMA steps per scaled piece
  const int64_t nrow_len = k / G;                    // norms per output row
  // This block's range of tiles (never empty: the host sizes the ranges).
  const int64_t g_begin = ks * gps;
  const int64_t g_end = g_begin + gps < ngr ? g_begin + gps : ngr;
  const int64_t row_bytes = k * SB / 8;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int h = lane >> 5, c32 = lane & 31;

  // This lane's output columns (one per 32-wide tile), clamped for loads.
  int64_t col[TN];
  const uint8_t* crow[TN];
  const uint16_t* nrow[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    col[t] = nt * BN + 64 * wave + 32 * t + c32;
    const int64_t cl = col[t] < n_out ? col[t] : n_out - 1;
    crow[t] = packed + cl * row_bytes;
    nrow[t] = norms + cl * nrow_len;
  }

  // DMA of group g's activation tile into buffer b.  Instruction i of wave w
  // fills LDS slots 64 (4 i + w) .. + 63 (16 bytes each): row r = slot / 32,
  // physical chunk p = slot % 32, holding logical chunk p ^ (r & 15).
  const uint8_t* xs = ws + 2 * xs_off + mt * kTileBytes;  // xs_off counts bf16 values
  auto issue_tile = [&](int64_t g, uint8_t* dst) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
    const auto src = make_rsrc(xs + g * mpad * kRowBytes, kTileBytes);
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int slot0 = 64 * (4 * i + wave);
      const int slot = slot0 + lane;
      const int r = slot >> 5, p = slot & 31;
      const uint32_t off = static_cast<uint32_t>(r * kRowBytes + 16 * (p ^ (r & 15)));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_ptr_t)(dst + 16 * slot0), 16, off, 0, 0, 0);
    }
#endif
  };

  Codes<SB> cur[TN], nxt[TN];
  // Norm bits held in 32-bit registers: packing two 16-bit loads into one
  // register would make the compiler wait for them (and, in order, for the
  // DMA issued before them) right away.
  uint32_t ncur[TN][NPT], nnxt[TN][NPT];
  // Norm j of tile g for output column t.
  auto norm_at = [&](int t, int64_t g, int j) __attribute__((always_inline)) -> uint32_t {
    return G <= kGroup ? nrow[t][g * NPT + j] : nrow[t][g / 2];
  };
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    load_codes<SB>(crow[t] + g_begin * 16 * SB, cur[t]);
#pragma unroll
    for (int j = 0; j < NPT; ++j) ncur[t][j] = norm_at(t, g_begin, j);
  }
  issue_tile(g_begin, xt0);
  wait_vm0();       // own DMA and loads
  __syncthreads();                              // every wave's DMA; the table

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x16{};

  // One group: DMA of the next group's tile into `next`, MFMAs on `tile`.
  auto group = [&](int64_t g, const uint8_t* tile, uint8_t* next) __attribute__((always_inline)) {
    if (g + 1 < g_end) {
      issue_tile(g + 1, next);
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        load_codes<SB>(crow[t] + (g + 1) * 16 * SB, nxt[t]);
#pragma unroll
        for (int j = 0; j < NPT; ++j) nnxt[t][j] = norm_at(t, g + 1, j);
      }
    }
    f32x16 tmp[TM][TN];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 ah[TM], al[TM], bh[TN], bl[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = 32 * i + c32;
        const int chi = 2 * s + h, clo = 16 + 2 * s + h;
        ah[i] = *reinterpret_cast<const bf16x8*>(tile + r * kRowBytes + 16 * (chi ^ (r & 15)));
        al[i] = *reinterpret_cast<const bf16x8*>(tile + r * kRowBytes + 16 * (clo ^ (r & 15)));
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) decode<SB>(cur[t], s, h, tab, bh[t], bl[t]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          f32x16 c = s % SPG == 0 ? f32x16{} : tmp[i][t];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[t], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[t], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[t], c, 0, 0, 0);
          tmp[i][t] = c;
        }
      if (s % SPG == SPG - 1) {  // a piece of one group is complete: scale and add
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          const float sc = half_to_float(static_cast<uint16_t>(ncur[t][s / SPG])) * (1.0f / G);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[i][t][j] = __builtin_fmaf(sc, tmp[i][t][j], acc[i][t][j]);
        }
      }
    }
    if (g + 1 < g_end) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        cur[t] = nxt[t];
#pragma unroll
        for (int j = 0; j < NPT; ++j) ncur[t][j] = nnxt[t][j];
      }
    }
    wait_vm0();       // next tile and codes
    __syncthreads();  // next tile complete in every wave; this tile no longer read
  };
  for (int64_t g = g_begin; g < g_end; g += 2) {
    group(g, xt0, xt1);
    if (g + 1 < g_end) group(g + 1, xt1, xt0);
  }

  // D layout of a 32x32 tile: lane holds column c32, rows 8 (j / 4) + 4 h + j % 4.
  // A split matrix writes its range's partial sums; the reduction adds them.
  float* const out = part ? part + ks * batch * n_out : y;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      if (col[t] >= n_out) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int64_t m = mt * BM + 32 * i + 8 * (j / 4) + 4 * h + (j % 4);
        if (m < batch) out[m * n_out + col[t]] = acc[i][t][j];
      }
    }
}

// y[m][c] = sum over ranges r = 0 .. ksplit - 1 of part[r][m][c], in order;
// one thread per output of the matrices that were split.
__global__ void __launch_bounds__(kBlock)
gemm_reduce_kernel(const GemmDesc* __restrict__ table, const int64_t* __restrict__ ostart, int n,
                   int64_t batch) {
  const int64_t o = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (o >= ostart[n]) return;
  const int d = find_lane(ostart, n, o);
  const GemmDesc& m = table[d];
  if (!m.part) return;
  const int64_t local = o - ostart[d];  // m * n_out + c
  const int64_t step = batch * m.n_out;
  float s = m.part[local];
  for (int64_t r = 1; r < m.ksplit; ++r) s += m.part[r * step + local];
  m.y[local] = s;
}

template <int SB, int G>
hipError_t launch_sbg(const GemmDesc* table, const int64_t* bstart, int n, int64_t blocks,
                      const SplitLevels& sl, const uint8_t* ws, int64_t batch, hipStream_t s) {
  const int64_t grid = ((blocks + kXcds - 1) / kXcds) * kXcds;
  if constexpr (G >= 64) {
    if (block_rows(batch, G) == 64) {
      hipLaunchKernelGGL((gemm_kernel<SB, 2, G>), dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, s, table,
                         bstart, n, sl, ws, batch);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<SB, 1, G>), dim3(static_cast<unsigned>(grid)), dim3(kBlock), 0, s, table,
                     bstart, n, sl, ws, batch);
  return hipGetLastError();
}

template <int SB>
hipError_t launch_sb(const GemmDesc* table, const int64_t* bstart, int n, int64_t blocks,
                     const SplitLevels& sl, const uint8_t* ws, int64_t batch, int group_size, hipStream_t s) {
  switch (group_size) {
    case 32: return launch_sbg<SB, 32>(table, bstart, n, blocks, sl, ws, batch, s);
    case 64: return launch_sbg<SB, 64>(table, bstart, n, blocks, sl, ws, batch, s);
    case 128: return launch_sbg<SB, 128>(table, bstart, n, blocks, sl, ws, batch, s);
    case 256: return launch_sbg<SB, 256>(table, bstart, n, blocks, sl, ws, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int G>
void launch_split_rotate_threads(const GemmDesc* table, const int64_t* ustart, int n, int64_t units,
                                 int64_t batch, uint16_t* ws, hipStream_t stream) {
  const int64_t blocks = (units + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(split_rotate_kernel<G>, dim3(static_cast<unsigned>(blocks)), dim3(kBlock), 0, stream, table,
                     ustart, n, batch, ws);
}

}  // namespace kg

int gemm_block_rows(int64_t batch, int group_size) { return kg::block_rows(batch, group_size); }
int gemm_block_cols() { return kg::BN; }

hipError_t launch_split_rotate(const GemmDesc* table, const int64_t* ustart, int n, int64_t units,
                               int64_t batch, int group_size, uint16_t* ws, hipStream_t stream) {
  if (units <= 0) return hipSuccess;
  if (group_size == kGroup && units < kFewUnits) {  // a wave per unit
    const int64_t blocks = (units + kg::kWaves - 1) / kg::kWaves;
    hipLaunchKernelGGL(kg::split_rotate_wave_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kg::kBlock), 0,
                       stream, table, ustart, n, batch, ws);
    return hipGetLastError();
  }
  switch (group_size) {  // a thread per unit
    case 32: kg::launch_split_rotate_threads<32>(table, ustart, n, units, batch, ws, stream); break;
    case 64: kg::launch_split_rotate_threads<64>(table, ustart, n, units, batch, ws, stream); break;
    case 128: kg::launch_split_rotate_threads<128>(table, ustart, n, units, batch, ws, stream); break;
    case 256: kg::launch_split_rotate_threads<256>(table, ustart, n, units, batch, ws, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_reduce(const GemmDesc* table, const int64_t* ostart, int n, int64_t outputs,
                              int64_t batch, hipStream_t stream) {
  if (outputs <= 0) return hipSuccess;
  const int64_t blocks = (outputs + kg::kBlock - 1) / kg::kBlock;
  hipLaunchKernelGGL(kg::gemm_reduce_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kg::kBlock), 0, stream,
                     table, ostart, n, batch);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmDesc* table, const int64_t* bstart, int n, int64_t blocks, int sbits,
                       const SplitLevels& sl, const uint16_t* ws, int64_t batch, int group_size,
                       hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  const uint8_t* w8 = reinterpret_cast<const uint8_t*>(ws);
  switch (sbits) {
    case 2: return kg::launch_sb<2>(table, bstart, n, blocks, sl, w8, batch, group_size, stream);
    case 3: return kg::launch_sb<3>(table, bstart, n, blocks, sl, w8, batch, group_size, stream);
    case 4: return kg::launch_sb<4>(table, bstart, n, blocks, sl, w8, batch, group_size, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cq
