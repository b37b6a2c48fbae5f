// Single-matrix dequant-matvec in one launch, y = x . W_hat^T, with no
// memory beyond the call's own buffers.
//
// The product is the forward pass of "Performance Differences Between 2-Bit
// and 4-Bit Quantization in Needle" (section Practical Code Comparison) with
// the weights decoded on the fly, as the runtime of "How Needle 2 Model
// Compresses to a Single Binary" (section Stage 3) decodes them.  Because
// the orthonormal Hadamard matrix is symmetric and its own inverse, every
// group g of a row contributes
//     x_g . W_hat_g = (norm_g / G) * < H x_g , levels[idx_g] >
// with H the +-1 Sylvester matrix.  Here each block rotates the activations
// it consumes itself (no rotated copy in device memory, no second launch),
// and the matrix descriptor is a kernel argument.
//
// Three kernels:
//   - matvec_pair_rot_kernel: 2-bit fields, one batch row per grid row
//     (blockIdx.y).  Per 1024-column tile the block builds, for every column
//     pair, the 16 partial products a 4-bit code pair can select; every row
//     of the block then spends one conflict-free LDS read and one add per two
//     weights.  The tile's activations are rotated by the block's 512
//     threads (two values each: one butterfly stage inside the thread, the
//     rest across lanes) into LDS, from where the table build reads them.
//   - matvec_rot_kernel: any field width, NB batch rows.  Each thread owns
//     16 consecutive columns of a 4096-column pass and keeps their rotated
//     activations for all NB rows in registers (16-point butterfly inside the
//     thread, the remaining stages across lanes), decodes the codes through
//     a per-lane copy of a small level table (so the data-dependent lookups
//     never collide on LDS banks) and reduces each group of rows over the
//     block in a fixed order.  It serves rows whose length is not a multiple
//     of 64 columns.
//   - matvec_mfma_kernel: any field width, 2 or more batch rows in chunks of
//     4 or 8.  The block rotates its chunk of activations into LDS; the
//     products run on the matrix cores (v_mfma_f32_4x4x1_16b_f32: the batch
//     rows of a chunk against one decoded weight per lane), so a weight costs
//     one table read and a quarter of a byte permute however many batch rows
//     share it.
// All are deterministic: every sum runs in a fixed order.

#include <type_traits>

#include "cq_internal.h"

namespace cq {
namespace kr {

constexpr int kChunk = 16;  // columns per thread
constexpr int kTile = kWave * kChunk;  // 1024 columns: one pair-table tile

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// One butterfly stage across lanes: this lane's value v and lane (l ^ s)'s
// value o combine into v + o (lane bit s clear) or o - v (set); sgn is +1 or
// -1 accordingly, so the stage is one exact fma per value.
__device__ __forceinline__ float xstage(float v, int s, float sgn) {
  const float o = __shfl_xor(v, s, kWave);
  return __builtin_fmaf(sgn, v, o);
}

// The same stage for a lane stride s of 1, 2, 4 or 8, inside the 16-lane
// rows of DPP: the lane with bit s clear takes v + (lane l + s's value), the
// other (lane l - s's value) - v.  No LDS traffic, only VALU operations.
template <int S>
__device__ __forceinline__ float dpp_stage(float v, bool upper) {
  // row_shl:S (0x100 + S): lane l reads lane l + S of its row; row_shr:S
  // (0x110 + S): lane l reads lane l - S.  Lanes whose source falls outside
  // the row keep 0 and never use the value.
  const float from_above = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), 0x100 + S, 0xF, 0xF, false));
  const float from_below = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), 0x110 + S, 0xF, 0xF, false));
  return upper ? from_below - v : v + from_above;
}

// ---- pair tables, one batch row per grid row ------------------------------------

constexpr int kPairWaves = 8;
constexpr int kPairBlock = kPairWaves * kWave;
// A pass is 4096 columns: lane l of every wave owns columns 64 l .. 64 l + 63
// of it, so a row's codes for the lane are one 16-byte load and its norm
// (group size >= 64) one 2-byte load.
constexpr int kPassCols = kWave * 64;
// Rotated x of a pass in LDS: column c at float c + 4 (c / 64), so that the
// table build's 16-byte reads (lane l at column 64 l + 8 w) and the
// rotation's 16-byte writes (thread t at column 8 t) spread over the banks.
constexpr int kXsFloats = kPassCols + kPassCols / 16;
__device__ __forceinline__ int xpad(int c) { return c + 4 * (c >> 6); }
// Pair tables of a pass: entry (pair q of lane l's 64 columns, code pair v)
// at float (16 q + v) * 64 + l, 128 KiB.  In every lookup instruction lane l
// touches bank l whatever its code: no bank conflicts by construction.
constexpr int kTableFloats = 32 * 16 * kWave;

// A block owns rows_per_block consecutive rows of the matrix (about an equal
// share for every compute unit); wave w takes rows w, w + 8, w + 16, ... of
// them, at most MAXR.  Per 4096-column pass: the block loads the pass's
// activations and rotates them into LDS; the codes and norms of all the
// wave's rows are then requested at once, and the block builds the pass's
// pair tables while they arrive; then every wave runs through its rows
// without further barriers.
template <int MAXR, bool TWO_NORMS>
__global__ void __launch_bounds__(kPairBlock, 1)
matvec_pair_rot_kernel(MatvecArgs a, LevelTable lv, int log2g, int rows_per_block) {
  __shared__ __attribute__((aligned(16))) float tab[kTableFloats];
  __shared__ __attribute__((aligned(16))) float xs[kXsFloats];
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t k = a.k, n_out = a.n_out;
  const int64_t brow = blockIdx.y;  // batch row
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * rows_per_block;
  const int64_t block_rows = n_out - row_base < rows_per_block ? n_out - row_base : rows_per_block;
  // This wave's rows: row_base + w + 8 i for i < nrows.
  const int nrows = block_rows > w ? static_cast<int>((block_rows - w + kPairWaves - 1) / kPairWaves) : 0;
  const int64_t row_bytes = k / 4, ngr = k >> log2g;
  const int G = 1 << log2g;
  const float* __restrict__ xrow = a.x + brow * k;

  // The wave's rows as one buffer resource from its first row; row i at the
  // scalar offset 8 i rows.  Rows past the wave's last re-read its last one
  // (their sums are never stored); a lane without columns in a pass offsets
  // by 2^30, past the resource, and reads zeros.  The host sends a matrix
  // here only when k <= 2^26 and k % 64 == 0, so a block's 64 rows of codes
  // (16 k bytes) stay under 2^30 and every offset under 2^31.
  const int64_t first = row_base + w;
  const int64_t span = nrows ? (static_cast<int64_t>(nrows - 1) * kPairWaves + 1) : 0;
  const auto codes_src = rsrc(a.packed + (nrows ? first * row_bytes : 0), span * row_bytes);
  const auto norms_src = rsrc(a.norms + (nrows ? first * ngr : 0), span * ngr * 2);
  int soff_c[MAXR], soff_n[MAXR];
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int ii = i < nrows ? i : (nrows > 0 ? nrows - 1 : 0);
    soff_c[i] = __builtin_amdgcn_readfirstlane(static_cast<int>(ii * kPairWaves * row_bytes));
    soff_n[i] = __builtin_amdgcn_readfirstlane(static_cast<int>(2 * ii * kPairWaves * ngr));
  }
  const float c0l = lv.c[0], c1l = lv.c[1], c2l = lv.c[2], c3l = lv.c[3];
  // Table byte address of (pair q, code pair v) for this lane: one byte
  // permute of the spread nibbles and one of these (byte 0 the lane's 4 l;
  // byte 2 selects the upper 64 KiB for pairs 16 .. 31).
  const uint32_t lane_lo = 4u * static_cast<uint32_t>(lane);
  const uint32_t lane_hi = lane_lo | 0x10000u;
  // TWO_NORMS: group size 32, two groups (two norms) per lane.

  float acc[MAXR];
#pragma unroll
  for (int i = 0; i < MAXR; ++i) acc[i] = 0.0f;
  const float sgn16 = (lane >> 4) & 1 ? -1.0f : 1.0f;

  for (int64_t p0 = 0; p0 < k; p0 += kPassCols) {
    // 1. The pass's activations: thread t takes columns 8 t .. 8 t + 7, at
    //    addresses clamped into the row.
    const int64_t my_c = p0 + 8 * static_cast<int64_t>(threadIdx.x);
    const bool my_live = my_c < k;  // whole 8-value runs: k % 64 == 0
    float xv[8];
    {
      const int64_t c = my_live ? my_c : 0;
      const float4 p = *reinterpret_cast<const float4*>(xrow + c);
      const float4 q = *reinterpret_cast<const float4*>(xrow + c + 4);
      xv[0] = p.x; xv[1] = p.y; xv[2] = p.z; xv[3] = p.w;
      xv[4] = q.x; xv[5] = q.y; xv[6] = q.z; xv[7] = q.w;
    }
    const int64_t c0 = p0 + 64 * lane;
    const bool active = c0 < k;
    const int coff = active ? static_cast<int>(c0 / 4) : (1 << 30);
    const int noff = active ? static_cast<int>(2 * (c0 >> log2g)) : (1 << 30);
    uint32_t codes[MAXR][4];
    uint32_t nrm[MAXR];  // binary16 norm(s): low half, and the high half for group size 32
    __syncthreads();  // the previous pass's tables and activations are no longer read
    // 2. Rotate: butterfly stages 1, 2, 4 inside the thread, lane strides
    //    1, 2, 4, 8 (element strides 8 .. 64) inside DPP rows, lane stride
    //    16 (element stride 128, group size 256) across rows; store to LDS.
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = my_live ? xv[e] : 0.0f;
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int i = 0; i < 8; i += 2 * h)
#pragma unroll
        for (int j = i; j < i + h; ++j) {
          const float u = xv[j], v = xv[j + h];
          xv[j] = u + v;
          xv[j + h] = u - v;
        }
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = dpp_stage<1>(xv[e], lane & 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) xv[e] = dpp_stage<2>(xv[e], lane & 2);
    if (G > 32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = dpp_stage<4>(xv[e], lane & 4);
    }
    if (G > 64) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = dpp_stage<8>(xv[e], lane & 8);
    }
    if (G > 128) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = xstage(xv[e], 16, sgn16);
    }
    {
      float* dst = xs + xpad(8 * threadIdx.x);
      *reinterpret_cast<float4*>(dst) = make_float4(xv[0], xv[1], xv[2], xv[3]);
      *reinterpret_cast<float4*>(dst + 4) = make_float4(xv[4], xv[5], xv[6], xv[7]);
      wait_lds_writes();  // the stored values keep their registers until the LDS has them
#pragma unroll
      for (int e = 0; e < 8; ++e) hold_values(xv[e]);
    }
    __syncthreads();
    // The codes and norms of the wave's rows are requested only now: issued
    // together with the activations, the whole grid's code stream delayed
    // the activations that every block waits for first (11008x4096: 8.04 ->
    // 7.80 us; 4096x11008, three passes: 13.44 -> 12.20 us).
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(codes_src, coff, soff_c[r], 2);  // nt: read once
      codes[r][0] = v[0]; codes[r][1] = v[1]; codes[r][2] = v[2]; codes[r][3] = v[3];
      if constexpr (TWO_NORMS)
        nrm[r] = __builtin_amdgcn_raw_buffer_load_b32(norms_src, noff, soff_n[r], 0);
      else
        nrm[r] = __builtin_amdgcn_raw_buffer_load_b16(norms_src, noff, soff_n[r], 0);
    }
    // 3. Pair tables: thread (w, lane) builds pairs 4 w .. 4 w + 3 of the
    //    lane's 64 columns (columns 64 lane + 8 w .. 64 lane + 8 w + 7).
    if (active) {
      const float* src = xs + xpad(64 * lane + 8 * w);
      const float4 p = *reinterpret_cast<const float4*>(src);
      const float4 q = *reinterpret_cast<const float4*>(src + 4);
      const float xr[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
      const float cb[4] = {c0l, c1l, c2l, c3l};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float x0 = xr[2 * h], x1 = xr[2 * h + 1];
        const float pa[4] = {c0l * x0, c1l * x0, c2l * x0, c3l * x0};
        float e[16];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) e[qq + 4 * bb] = __builtin_fmaf(cb[bb], x1, pa[qq]);
        float* dst = tab + (16 * (4 * w + h)) * kWave + lane;
#pragma unroll
        for (int v = 0; v < 16; ++v) dst[v * kWave] = e[v];
        wait_lds_writes();
#pragma unroll
        for (int v = 0; v < 16; ++v) hold_values(e[v]);
      }
    }
    __syncthreads();
    // 4. Every row of the wave: 32 lookups and adds per lane, then the norm.
    const char* tb = reinterpret_cast<const char*>(tab);
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < nrows) {  // the same for the whole wave (a guard: an early exit stops the unrolling)
      float part[2] = {0.0f, 0.0f};  // columns 0-31 and 32-63 of the lane
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t cw = codes[r][d];
        const uint32_t ev = cw & 0x0F0F0F0Fu, od = (cw >> 4) & 0x0F0F0F0Fu;
        const uint32_t base = d < 2 ? lane_lo : lane_hi;
#pragma unroll
        for (int qq = 0; qq < 8; ++qq) {
          // Pair q = 8 d + qq: its nibble is byte qq / 2 of ev (qq even) or od.
          const uint32_t e = (qq & 1) ? od : ev;
          // Selector: byte 0 = base byte 0 (4 l), byte 1 = byte qq / 2 of e,
          // byte 2 = base byte 2 (the 64 KiB half), byte 3 = zero.
          const uint32_t addr = __builtin_amdgcn_perm(e, base, 0x0C020000u | ((4u + (qq >> 1)) << 8));
          const float v = *reinterpret_cast<const float*>(tb + addr + 4096 * ((8 * d + qq) & 15));
          part[d >> 1] = (d & 1) || qq ? part[d >> 1] + v : v;
        }
      }
      // Lanes without columns in the pass read codes 0 and norms 0: they add 0.
      const float n_lo = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(nrm[r])));
      if constexpr (TWO_NORMS) {
        const float n_hi = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(nrm[r] >> 16)));
        acc[r] = __builtin_fmaf(n_hi, part[1], __builtin_fmaf(n_lo, part[0], acc[r]));
      } else {
        acc[r] = __builtin_fmaf(n_lo, part[0] + part[1], acc[r]);
      }
      }
    }
  }

  // acc[r] holds lane partial sums of row first + 8 r: sum over the 64 lanes
  // (a fixed shuffle tree), then lane 0 stores.
#pragma unroll
  for (int r = 0; r < MAXR; ++r) {
    float v = acc[r];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    acc[r] = v;
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < MAXR; ++r)
      if (r < nrows) a.y[brow * n_out + first + static_cast<int64_t>(r) * kPairWaves] = acc[r] * (1.0f / static_cast<float>(G));
  }
}

// ---- any width, NB batch rows -------------------------------------------------

constexpr int kRotWaves = 4;
constexpr int kRotBlock = kRotWaves * kWave;
constexpr int kPass = kRotBlock * kChunk;  // 4096 columns per pass

// Per-lane copies of a small level table: entry (v, lane l) at byte
// 256 v + 4 l, so the lookup address of lane l is one byte permute of its
// code and its own lane byte, and in every read instruction lane l touches
// bank l whatever its code (no bank conflicts by construction).
//   2-bit fields: the codes of two adjacent columns form a nibble v; table 0
//     holds level[v & 3], table 1 (4 KiB + 64 bytes further, so that a lane's
//     two reads fall on different banks) level[v >> 2];
//   4-bit fields: one code per nibble, one table;
//   3-bit fields: one 8-entry table, the code extracted by a shift.
template <int SB>
struct LaneTab {
  static constexpr int entries = SB == 3 ? 8 : 16;
  static constexpr int tables = SB == 2 ? 2 : 1;
  static constexpr int kSecond = 16 * kWave + 16;  // float offset of table 1
  static constexpr int floats = tables == 2 ? kSecond + 16 * kWave : 16 * kWave;
  static __device__ __forceinline__ void fill(float* tab, const LevelTable& lv, int t) {
    for (int i = t; i < floats; i += kRotBlock) {
      const int tb = tables == 2 && i >= kSecond ? 1 : 0;
      const int v = ((tb ? i - kSecond : i) / kWave) % 16;
      float val = 0.0f;
      if (v < entries) {
        if constexpr (SB == 2)
          val = level_at(lv, tb == 0 ? (v & 3) : (v >> 2));
        else
          val = level_at(lv, v);
      }
      tab[i] = val;
      wait_lds_writes();
      hold_values(val);
    }
  }
  // Levels of the 16 codes of a chunk (column c0 + e at bits [SB e, SB e + SB)).
  static __device__ __forceinline__ void decode(uint64_t codes, const char* tb, uint32_t lane_bytes,
                                                float (&v)[16]) {
    if constexpr (SB == 2) {
      const uint32_t cw = static_cast<uint32_t>(codes);
      const uint32_t ev = cw & 0x0F0F0F0Fu, od = (cw >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const uint32_t e = (q & 1) ? od : ev;
        const uint32_t addr = __builtin_amdgcn_perm(e, lane_bytes, 0x0C0C0000u | ((4u + (q >> 1)) << 8));
        v[2 * q] = *reinterpret_cast<const float*>(tb + addr);
        v[2 * q + 1] = *reinterpret_cast<const float*>(tb + addr + 4 * kSecond);
      }
    } else if constexpr (SB == 4) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t cw = static_cast<uint32_t>(codes >> (32 * h));
        const uint32_t ev = cw & 0x0F0F0F0Fu, od = (cw >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t e = (q & 1) ? od : ev;
          const uint32_t addr = __builtin_amdgcn_perm(e, lane_bytes, 0x0C0C0000u | ((4u + (q >> 1)) << 8));
          v[8 * h + q] = *reinterpret_cast<const float*>(tb + addr);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t c = static_cast<uint32_t>(codes >> (3 * e)) & 7u;
        v[e] = *reinterpret_cast<const float*>(tb + ((c << 8) | lane_bytes));
      }
    }
  }
};

// Packed codes of the 16 columns starting at column c0 (c0 % 16 == 0) of a
// row, column c0 + e at bits [SB e, SB e + SB).
template <int SB>
__device__ __forceinline__ uint64_t codes16(const uint8_t* __restrict__ row_ptr, int64_t c0) {
  if constexpr (SB == 2) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(row_ptr + c0 / 4));
  } else if constexpr (SB == 4) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(row_ptr + c0 / 2));
  } else {
    // 6 bytes at the 2-byte aligned offset 6 (c0 / 16): exactly those bytes,
    // so the last chunk of the last row stays inside the buffer.
    const uint16_t* p = reinterpret_cast<const uint16_t*>(row_ptr + 6 * (c0 / 16));
    return static_cast<uint64_t>(p[0]) | (static_cast<uint64_t>(p[1]) << 16) | (static_cast<uint64_t>(p[2]) << 32);
  }
}

// A block owns rg groups of RB consecutive rows of the matrix and a chunk of
// NB batch rows (blockIdx.y; rows past the batch read zero activations and
// are not stored).  Work units are (row group, pass) in order; the codes and
// norms of PF units are in flight while one is computed.  When k fits one
// pass the thread's activations are loaded and rotated once for all of the
// block's rows; otherwise once per unit.
template <int SB, int NB, int RB, int PF>
__global__ void __launch_bounds__(kRotBlock, 2)
matvec_rot_kernel(MatvecArgs a, LevelTable lv, int log2g, int rg) {
  using LT = LaneTab<SB>;
  __shared__ __attribute__((aligned(16))) float tab[LT::floats];
  __shared__ float red[RB * NB][kRotBlock + 1];
  LT::fill(tab, lv, threadIdx.x);
  __syncthreads();
  const int t = threadIdx.x, lane = t % kWave;
  const int64_t k = a.k, n_out = a.n_out;
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * NB;
  const int64_t row_base = static_cast<int64_t>(blockIdx.x) * RB * rg;
  const int64_t row_bytes = k * SB / 8, ngr = k >> log2g;
  const int n_pass = static_cast<int>((k + kPass - 1) / kPass);
  const bool one_pass = n_pass == 1;
  const int G = 1 << log2g;
  const float inv_g = 1.0f / static_cast<float>(G);  // exact: a power of two
  const int64_t groups_here = (n_out - row_base + RB - 1) / RB;
  const int n_units = static_cast<int>((groups_here < rg ? groups_here : rg) * n_pass);
  const char* tb = reinterpret_cast<const char*>(tab);
  const uint32_t lane_bytes = 4u * static_cast<uint32_t>(lane);

  // Butterfly signs of the cross-lane stages (lane stride 1, 2, 4, 8).
  float sgn[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sgn[i] = (lane >> i) & 1 ? -1.0f : 1.0f;

  float xv[NB][kChunk];
  // Activations of this thread's 16 columns of pass p, loaded at addresses
  // clamped into x (past k: the row's last chunk; past the batch: its last
  // row), unconditionally, so that the wait before the rotation counts them
  // exactly; out-of-range values become zeros at use.
  auto load_x = [&](int p) __attribute__((always_inline)) {
    int64_t c0 = static_cast<int64_t>(p) * kPass + kChunk * t;
    c0 = c0 < k ? c0 : k - kChunk;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int64_t bb = b0 + b < a.batch ? b0 + b : a.batch - 1;
      const float4* src = reinterpret_cast<const float4*>(a.x + bb * k + c0);
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
  // Rotated activations of pass p: zeros where out of range, then the
  // 16-point butterfly inside the thread, then log2(G / 16) stages across
  // the lanes that share the group.
  auto rotate_x = [&](int p) __attribute__((always_inline)) {
    const bool cols = static_cast<int64_t>(p) * kPass + kChunk * t < k;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bool live = cols && b0 + b < a.batch;
#pragma unroll
      for (int e = 0; e < kChunk; ++e) xv[b][e] = live ? xv[b][e] : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int h = 1; h < kChunk; h <<= 1)
#pragma unroll
        for (int i = 0; i < kChunk; i += 2 * h)
#pragma unroll
          for (int j = i; j < i + h; ++j) {
            const float u = xv[b][j], v = xv[b][j + h];
            xv[b][j] = u + v;
            xv[b][j + h] = u - v;
          }
#pragma unroll
      for (int st = 0; st < 4; ++st)
        if ((kChunk << st) < G)
#pragma unroll
          for (int e = 0; e < kChunk; ++e) xv[b][e] = xstage(xv[b][e], 1 << st, sgn[st]);
    }
  };

  // Codes and binary16 norms of PF units in flight, loaded through buffer
  // resources of the unit's rows: each row's offset is a scalar, the lane's
  // column offset one register shared by all rows, and a thread without
  // columns in the pass offsets by 2^30, past the resource, and reads zeros
  // (norm 0, so its products vanish even where a stored norm is +Inf).  Rows
  // past the end of the matrix re-read its last row (never stored); units
  // past the block's last re-read that one (never used).  No loaded value is
  // selected or converted before its unit comes up, so no load is waited
  // for early.  The host sends a matrix here only when k <= 2^28, so a unit's
  // RB rows of codes and every offset stay under 2^31.
  using CodeT = typename std::conditional<SB == 2, uint32_t, uint64_t>::type;
  CodeT codes[PF][RB];
  _Float16 nbits[PF][RB];
  auto issue = [&](int u, CodeT (&c)[RB], _Float16 (&nb)[RB]) __attribute__((always_inline)) {
    const int uu = u < n_units ? u : n_units - 1;
    const int g = uu / n_pass, p = uu - g * n_pass;
    const int64_t grow0 = row_base + static_cast<int64_t>(g) * RB;
    const int64_t rows_in = n_out - grow0 < RB ? n_out - grow0 : RB;  // >= 1
    const auto csrc = rsrc(a.packed + grow0 * row_bytes, rows_in * row_bytes);
    const auto nsrc = rsrc(a.norms + grow0 * ngr, rows_in * ngr * 2);
    const int64_t c0 = static_cast<int64_t>(p) * kPass + kChunk * t;
    const bool in = c0 < k;
    const int coff = in ? static_cast<int>(c0 * SB / 8) : (1 << 30);
    const int noff = in ? static_cast<int>(2 * (c0 >> log2g)) : (1 << 30);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int rr = r < rows_in ? r : static_cast<int>(rows_in) - 1;
      const int sc = __builtin_amdgcn_readfirstlane(static_cast<int>(rr * row_bytes));
      const int sn = __builtin_amdgcn_readfirstlane(static_cast<int>(2 * rr * ngr));
      if constexpr (SB == 2) {
        c[r] = __builtin_amdgcn_raw_buffer_load_b32(csrc, coff, sc, 2);  // nt: read once
      } else if constexpr (SB == 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(csrc, coff, sc, 2);
        c[r] = static_cast<uint64_t>(v[0]) | (static_cast<uint64_t>(v[1]) << 32);
      } else {
        // 6 bytes at the 2-byte aligned offset 6 (c0 / 16).
        const uint64_t h0 = __builtin_amdgcn_raw_buffer_load_b16(csrc, coff, sc, 2);
        const uint64_t h1 = __builtin_amdgcn_raw_buffer_load_b16(csrc, coff + 2, sc, 2);
        const uint64_t h2 = __builtin_amdgcn_raw_buffer_load_b16(csrc, coff + 4, sc, 2);
        c[r] = h0 | (h1 << 16) | (h2 << 32);
      }
      nb[r] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(nsrc, noff, sn, 0));
    }
  };
  if (one_pass) load_x(0);  // before the codes, so the rotation waits for these loads only
#pragma unroll
  for (int j = 0; j < PF; ++j) issue(j, codes[j], nbits[j]);
  if (one_pass) rotate_x(0);

  float acc[RB][NB];
  for (int u0 = 0; u0 < n_units; u0 += PF) {
    // Unrolled by PF with a guard (not an early exit), so that every index
    // into the ring of codes is a compile-time constant.
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int u = u0 + j;
      if (u < n_units) {  // the same for the whole block
      const int g = u / n_pass, p = u - g * n_pass;
      if (p == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;
      }
      if (!one_pass) {
        load_x(p);
        rotate_x(p);
      }
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float v[kChunk];
        LT::decode(codes[j][r], tb, lane_bytes, v);
        float part[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) part[b] = 0.0f;
#pragma unroll
        for (int e = 0; e < kChunk; ++e)
#pragma unroll
          for (int b = 0; b < NB; ++b) part[b] = __builtin_fmaf(v[e], xv[b][e], part[b]);
        const float sc = static_cast<float>(nbits[j][r]) * inv_g;
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = __builtin_fmaf(sc, part[b], acc[r][b]);
        // One row at a time: without this the compiler hoists every row's
        // table reads to the top and needs a register per level read.
        __builtin_amdgcn_sched_barrier(0);
      }
      if (u + PF < n_units) issue(u + PF, codes[j], nbits[j]);
      if (p == n_pass - 1) {
        // Block reduction in a fixed order: thread t's partials go to column
        // t of `red`; thread t then sums value t / 8 over columns
        // 32 (t % 8) .. 32 (t % 8) + 31 and the 8 threads of a value combine
        // by shuffles.
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) red[r * NB + b][t] = acc[r][b];
        __syncthreads();
        constexpr int V = RB * NB;  // values to reduce (<= 32)
        const int vi = t / 8, part_i = t % 8;
        float s = 0.0f;
        if (vi < V) {
#pragma unroll 8
          for (int i = 0; i < 32; ++i) s += red[vi][32 * part_i + i];
        }
        s += __shfl_xor(s, 1, kWave);
        s += __shfl_xor(s, 2, kWave);
        s += __shfl_xor(s, 4, kWave);
        if (vi < V && part_i == 0) {
          const int r = vi / NB, b = vi % NB;
          const int64_t row = row_base + static_cast<int64_t>(g) * RB + r;
          if (row < n_out && b0 + b < a.batch) a.y[(b0 + b) * n_out + row] = s;
        }
        __syncthreads();  // `red` is rewritten by the next row group
      }
      }
    }
  }
}

// ---- matrix cores, up to 8 batch rows per block ---------------------------------

typedef float mf_v4 __attribute__((ext_vector_type(4)));

constexpr int kMfWaves = 8;
constexpr int kMfBlock = kMfWaves * kWave;     // 512 threads, one block per compute unit
constexpr int kMfPass = 4096;                  // columns of rotated activations in LDS
constexpr int kMfSlices = 4;                   // column slices of a pass
constexpr int kMfSlice = kMfPass / kMfSlices;  // 1024 columns: 64 for each group of 4 lanes
constexpr int kMfSubsets = kMfWaves / kMfSlices;  // row subsets: waves per slice
constexpr int kMfMaxQuads = 6;                 // row quads per wave
constexpr int kMfMaxRows = kMfSubsets * kMfMaxQuads * 4;  // 48 rows per block
// Row quads per wave of a kernel instance: 3- and 4-bit codes of 8 batch
// rows take 4 (32 rows per block), which keeps them within 256 registers.
__host__ __device__ constexpr int mf_quads(int sb, int nh) { return nh == 2 && sb != 2 ? 4 : kMfMaxQuads; }

// Activations of the pass in LDS: float4 f of batch row r at float4
// r * kMfRowF4 + f + f / 16 (one float4 of padding per 16, rows 1090 float4
// apart, 2 mod 8).  In every group of eight lanes the product's 16-byte
// reads (lanes 4 b + q: row q (+4), float4 16 b + c) and the coalesced
// writes (consecutive float4s) fall on eight different 16-byte bank slots,
// as do the rotation's own-run reads and writes with 16 float4 per thread
// (8 float4 per thread: two lanes per slot); and every address is a
// per-lane base plus a constant offset.
constexpr int kMfRowF4 = 1090;
__device__ __forceinline__ int mf_pad(int f) { return f + (f >> 4); }

// Sum of a value over the four lanes l, l +- 4, l +- 8 of a 16-lane DPP row
// that share l % 4: two row rotations (DPP row_ror 4 and 8), no LDS.
__device__ __forceinline__ float mf_row_sum4(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  return v;
}

// Codes of the lane's 64 columns of a slice (SB bits each, 8 SB bytes).
template <int SB>
struct MfCodes {
  uint32_t d[2 * SB];
  // Codes of columns 16 c .. 16 c + 15 of the 64, column 16 c + e at bits [SB e, SB e + SB).
  __device__ __forceinline__ uint64_t chunk(int c) const {
    if constexpr (SB == 2) {
      return d[c];
    } else if constexpr (SB == 4) {
      return static_cast<uint64_t>(d[2 * c]) | (static_cast<uint64_t>(d[2 * c + 1]) << 32);
    } else {
      const uint64_t w0 = static_cast<uint64_t>(d[0]) | (static_cast<uint64_t>(d[1]) << 32);
      const uint64_t w1 = static_cast<uint64_t>(d[2]) | (static_cast<uint64_t>(d[3]) << 32);
      const uint64_t w2 = static_cast<uint64_t>(d[4]) | (static_cast<uint64_t>(d[5]) << 32);
      return c == 0 ? w0 : c == 1 ? (w0 >> 48) | (w1 << 16) : c == 2 ? (w1 >> 32) | (w2 << 32) : w2 >> 16;
    }
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t src, int voff) {
    if constexpr (SB == 2) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(src, voff, 0, 2);  // nt: read once
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
    } else if constexpr (SB == 4) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(src, voff, 0, 2);
      const auto u = __builtin_amdgcn_raw_buffer_load_b128(src, voff + 16, 0, 2);
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
      d[4] = u[0]; d[5] = u[1]; d[6] = u[2]; d[7] = u[3];
    } else {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(src, voff + 8 * i, 0, 2);
        d[2 * i] = v[0]; d[2 * i + 1] = v[1];
      }
    }
  }
};

// The many-matrix form's arguments: the device descriptor table, its
// row-block prefix (block b belongs to descriptor d with bstart[d] <= b <
// bstart[d + 1]), the rotated activations and the batch rows b0 .. b0 + nb - 1
// of this launch.
struct MfMany {
  const MatvecDesc* table;
  const int64_t* bstart;
  int n;
  const float* xr;
  int64_t b0;
  int nb;
};

__device__ __forceinline__ int mf_find_desc(const int64_t* __restrict__ start, int n, int64_t v) {
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

// One block per compute unit owns rows_per_block consecutive rows of a
// matrix (at most 48; 32 for 3- and 4-bit codes at 8 batch rows) and a
// chunk of 4 NH batch rows (blockIdx.y; the many-matrix form: one chunk per
// launch, the block's matrix from the descriptor table).  Per 4096-column
// pass the block brings the pass's activations of its batch rows into LDS
// and, in the single-matrix form, rotates them there (the threads of a batch
// row own V consecutive columns: the butterfly inside the thread, the
// remaining stages across lanes by DPP).  Wave w takes column slice w % 4 of
// the pass and the row quads w / 4, w / 4 + 2, ... of the block.
//
// The products run on v_mfma_f32_4x4x1_16b_f32: 16 blocks of a 4x4 outer
// product per instruction.  Lane l = 4 b + q feeds block b the activation of
// batch row q (+4 h) and the level of weight row q of the quad, both at
// column 64 b + 16 c + j of the slice in step (c, j); the block's
// accumulator, held by lanes 4 b .. 4 b + 3, sums x[batch i] * w[row q]
// over block b's columns.  The 16 blocks' sums are added over the lanes at
// the end and the slices and lane rows in LDS, in a fixed order.  Lane l's
// 64 columns are one 8 SB-byte load of codes per row and lie in one or two
// groups, whose norms scale either each decoded level (one multiply per
// weight, shared by all batch rows) or, for rows of one pass with groups of
// 64 or more columns, the lane's accumulator once at the end.
template <int SB, int NH, bool MANY, int PC>
__global__ void __launch_bounds__(PC / 8, 4096 / PC)
matvec_mfma_kernel(MatvecArgs a, LevelTable lv, int log2g, int rows_per_block, MfMany many) {
  // Block shape of a pass width PC (4096 or 2048 columns): PC / 512 waves,
  // PC / 1024 slices of 1024 columns, two row subsets; one block per CU at
  // 4096 columns, two at 2048 (half the LDS).
  constexpr int WV = PC / 512;
  constexpr int BLOCK = WV * kWave;
  constexpr int SLICES = PC / 1024;
  constexpr int SLICE = 1024;
  constexpr int SUBSETS = WV / SLICES;
  static_assert(SUBSETS == kMfSubsets, "the row caps assume two row subsets");
  constexpr int RF4 = PC / 4 + PC / 64 + 2;  // float4 per LDS row: 2 mod 8
  constexpr int NP = SLICES * 4;             // partial sums per output: slices x lane rows
  constexpr int NB = 4 * NH;                 // batch rows per block
  constexpr int TPR = BLOCK / NB;            // rotation threads per batch row
  constexpr int V = PC / TPR;                // columns per rotation thread: 32 or 64
  constexpr int MQ = mf_quads(SB, NH);       // row quads per wave
  static_assert(MQ % 2 == 0, "quads run in pairs");
  using LT = LaneTab<SB>;
  // One LDS array: the level table first, at address 0, so that its reads
  // take their offsets as immediates; then the activations.
  constexpr int kTabF = (LT::floats + 3) / 4 * 4;
  __shared__ __attribute__((aligned(16))) float lds[kTabF + NB * RF4 * 4];
  float* const tab = lds;
  float* const xs = lds + kTabF;
  if (threadIdx.x < kRotBlock) LT::fill(tab, lv, threadIdx.x);

  const int t = threadIdx.x, lane = t % kWave;
  const int w = __builtin_amdgcn_readfirstlane(t / kWave);
  const int slice = w % SLICES, rsub = w / SLICES;
  const int bq = lane >> 2, q = lane & 3;
  int64_t b0, row_base;
  if constexpr (MANY) {
    // The block's matrix from the descriptor table (scalar loads); its
    // activations are the rotated copy, batch rows b0 .. b0 + nb - 1.
    const int d = mf_find_desc(many.bstart, many.n, blockIdx.x);
    const MatvecDesc* m = many.table + d;
    a.packed = m->packed;
    a.norms = m->norms;
    a.x = many.xr + m->xr_offset;
    a.y = m->y;
    a.n_out = m->n_out;
    a.k = m->k;
    a.batch = many.b0 + many.nb;
    b0 = many.b0;
    row_base = (static_cast<int64_t>(blockIdx.x) - many.bstart[d]) * rows_per_block;
  } else {
    b0 = static_cast<int64_t>(blockIdx.y) * NB;
    row_base = static_cast<int64_t>(blockIdx.x) * rows_per_block;
  }
  const int64_t k = a.k, n_out = a.n_out;
  const int block_rows = static_cast<int>(n_out - row_base < rows_per_block ? n_out - row_base : rows_per_block);
  const int n_quads = (block_rows + 3) / 4;
  const int nq = n_quads > rsub ? (n_quads - rsub + SUBSETS - 1) / SUBSETS : 0;  // this wave's quads
  const int64_t row_bytes = k * SB / 8, ngr = k >> log2g;
  const int G = 1 << log2g;
  const char* tb = reinterpret_cast<const char*>(tab);
  const uint32_t lane_bytes = 4u * static_cast<uint32_t>(lane);
  // The block's rows as one buffer resource; lanes past the block's last row
  // re-read it (never stored).  The host sends a matrix here only when
  // k <= 2^26, so 48 rows of codes stay under 2^31 bytes.
  const auto codes_src = rsrc(a.packed + row_base * row_bytes, block_rows * row_bytes);
  const auto norms_src = rsrc(a.norms + row_base * ngr, block_rows * ngr * 2);
  int roff_c[MQ], roff_n[MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    int r = 4 * (rsub + SUBSETS * i) + q;
    r = r < block_rows ? r : block_rows - 1;
    roff_c[i] = static_cast<int>(r * row_bytes);
    roff_n[i] = static_cast<int>(r * ngr * 2);
  }
  // Rotation thread: batch row rr, columns V cb .. V cb + V - 1 of the pass.
  const int rr = t / TPR, cb = t % TPR;
  const bool row_live = b0 + rr < a.batch;
  const float* __restrict__ xrow = a.x + (b0 + rr) * k;  // dereferenced only when row_live

  mf_v4 acc[MQ][NH];
#pragma unroll
  for (int i = 0; i < MQ; ++i)
#pragma unroll
    for (int h = 0; h < NH; ++h) acc[i][h] = mf_v4{0.0f, 0.0f, 0.0f, 0.0f};
  // Rows of one pass with groups of 64 or more columns: a lane's 64 columns
  // share one norm, so the levels go in unscaled and each accumulator is
  // scaled once at the end by its lane's norm (lane l's accumulator only
  // sums products with lane l's weights).  Otherwise every level is scaled
  // by its norm before its products.
  const bool late = k <= PC && G >= 64;
  float lnorm[MQ];
#pragma unroll
  for (int i = 0; i < MQ; ++i) lnorm[i] = 0.0f;

  for (int64_t p0 = 0; p0 < k; p0 += PC) {
    // 1. The pass's activations, coalesced: thread (rr, cb) loads float4s
    //    cb + TPR s (s < V / 4) of batch row rr, zeros past k or past the
    //    batch (such a float4 is read at the start of x instead).
    uint4 raw[V / 4];
#pragma unroll
    for (int i = 0; i < V / 4; ++i) {
      const int64_t c = p0 + 4 * static_cast<int64_t>(cb + TPR * i);
      const bool live = row_live && c < k;  // k % 4 == 0
      const uint4 v = *reinterpret_cast<const uint4*>(live ? xrow + c : a.x);
      raw[i] = live ? v : make_uint4(0u, 0u, 0u, 0u);
    }
    // 2. Codes and norms of the wave's quads for its slice of the pass:
    //    lane 4 b + q takes columns 64 b .. 64 b + 63 of the slice of row
    //    4 quad + q.  Lanes whose columns lie past k get norm 0 (their
    //    activations are 0 too), so nothing they read contributes.
    const int64_t c0 = p0 + static_cast<int64_t>(slice) * SLICE + 64 * bq;
    const bool slice_live = p0 + static_cast<int64_t>(slice) * SLICE < k;  // the same for the wave
    MfCodes<SB> codes[MQ] = {};
    uint32_t nrm[MQ][2] = {};
    {
      const int cvo = static_cast<int>(c0 * SB / 8);
      const int g0 = static_cast<int>(c0 >> log2g);
#pragma unroll
      for (int i = 0; i < MQ; ++i) {
        if (slice_live && i < nq) {
          codes[i].load(codes_src, roff_c[i] + cvo);
          nrm[i][0] = __builtin_amdgcn_raw_buffer_load_b16(norms_src, roff_n[i] + 2 * g0, 0, 0);
          nrm[i][1] = G == 32 ? __builtin_amdgcn_raw_buffer_load_b16(norms_src, roff_n[i] + 2 * g0 + 2, 0, 0) : 0u;
        }
      }
    }
    __syncthreads();  // the previous pass's activations are no longer read
    // 3. Through LDS to the rotation's layout: thread (rr, cb) reads back
    //    columns V cb .. V cb + V - 1 (both steps conflict-free: mf_pad),
    //    then rotates them and writes them to the very slots it read.  The
    //    many-matrix form loads activations rotated beforehand: it stops
    //    after the first write.
    {
      float* dst = xs + rr * RF4 * 4;
#pragma unroll
      for (int i = 0; i < V / 4; ++i) *reinterpret_cast<uint4*>(dst + 4 * mf_pad(cb + TPR * i)) = raw[i];
      hold_until_lds_written(raw);
    }
    __syncthreads();
    if constexpr (!MANY) {
    float xv[V];
    {
      const float* src = xs + rr * RF4 * 4;
#pragma unroll
      for (int i = 0; i < V / 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(src + 4 * mf_pad((V / 4) * cb + i));
        xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
      }
    }
    //    Butterfly stages of element stride 1 .. min(V, G)/2 inside the
    //    thread, then strides V .. G/2 across lanes (lane strides 1 .. 8).
#pragma unroll
    for (int hh = 1; hh < V; hh <<= 1) {
      if (hh < G) {
#pragma unroll
        for (int i = 0; i < V; i += 2 * hh)
#pragma unroll
          for (int j = i; j < i + hh; ++j) {
            const float u = xv[j], v = xv[j + hh];
            xv[j] = u + v;
            xv[j + hh] = u - v;
          }
      }
    }
    if (V < G) {
#pragma unroll
      for (int e = 0; e < V; ++e) xv[e] = dpp_stage<1>(xv[e], lane & 1);
    }
    if (2 * V < G) {
#pragma unroll
      for (int e = 0; e < V; ++e) xv[e] = dpp_stage<2>(xv[e], lane & 2);
    }
    if (4 * V < G) {
#pragma unroll
      for (int e = 0; e < V; ++e) xv[e] = dpp_stage<4>(xv[e], lane & 4);
    }
    if (8 * V < G) {
#pragma unroll
      for (int e = 0; e < V; ++e) xv[e] = dpp_stage<8>(xv[e], lane & 8);
    }
    {
      float* dst = xs + rr * RF4 * 4;
      uint4 ch[V / 4];
#pragma unroll
      for (int i = 0; i < V / 4; ++i) {
        ch[i] = make_uint4(__builtin_bit_cast(uint32_t, xv[4 * i]), __builtin_bit_cast(uint32_t, xv[4 * i + 1]),
                           __builtin_bit_cast(uint32_t, xv[4 * i + 2]), __builtin_bit_cast(uint32_t, xv[4 * i + 3]));
        *reinterpret_cast<uint4*>(dst + 4 * mf_pad((V / 4) * cb + i)) = ch[i];
      }
      hold_until_lds_written(ch);  // the stored chunks keep their registers until the LDS has them
    }
    __syncthreads();
    }
    // 4. Products: per 16-column chunk c of the lane's 64 columns, the
    //    chunk's activations (one 64-byte run per batch row half), then for
    //    every quad the 16 scaled levels and 16 NH matrix-core steps.
    if (slice_live) {
      float nscale[MQ][2];
#pragma unroll
      for (int i = 0; i < MQ; ++i) {
        const bool in0 = c0 < k, in1 = c0 + 32 < k;
        const float n0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(nrm[i][0])));
        const float n1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(nrm[i][1])));
        nscale[i][0] = in0 ? n0 : 0.0f;
        nscale[i][1] = G == 32 ? (in1 ? n1 : 0.0f) : nscale[i][0];
        lnorm[i] = nscale[i][0];
      }
      // Float4 16 b + 4 c + u of the slice sits at mf_pad(...) = 17 (f0 / 16) + 4 c + u.
      const float* xbase = xs + q * RF4 * 4 + 4 * mf_pad((slice * SLICE) / 4 + 16 * bq);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float xa[NH][16];
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const float* src = xbase + 4 * h * RF4 * 4;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float4 v = *reinterpret_cast<const float4*>(src + 4 * (4 * c + u));
            xa[h][4 * u] = v.x; xa[h][4 * u + 1] = v.y; xa[h][4 * u + 2] = v.z; xa[h][4 * u + 3] = v.w;
          }
        }
        // Quads in pairs: both quads' level reads are in flight together and
        // the steps alternate over 2 NH accumulators.  A wave with an odd
        // number of quads runs its last pair's second quad with norm 0 into
        // rows past the block (never stored).
#pragma unroll
        for (int i = 0; i < MQ; i += 2) {
          if (i < nq) {  // the same for the whole wave
            float lev0[16], lev1[16];
            LT::decode(codes[i].chunk(c), tb, lane_bytes, lev0);
            LT::decode(codes[i + 1].chunk(c), tb, lane_bytes, lev1);
            if (late) {
#pragma unroll
              for (int j = 0; j < 16; ++j)
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                  acc[i][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[h][j], lev0[j], acc[i][h], 0, 0, 0);
                  acc[i + 1][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[h][j], lev1[j], acc[i + 1][h], 0, 0, 0);
                }
            } else {
              const float s0 = nscale[i][c >> 1], s1 = nscale[i + 1][c >> 1];
#pragma unroll
              for (int j = 0; j < 16; ++j) {
                const float w0 = lev0[j] * s0, w1 = lev1[j] * s1;
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                  acc[i][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[h][j], w0, acc[i][h], 0, 0, 0);
                  acc[i + 1][h] = __builtin_amdgcn_mfma_f32_4x4x1f32(xa[h][j], w1, acc[i + 1][h], 0, 0, 0);
                }
              }
            }
          }
          // One pair at a time: otherwise the compiler hoists every quad's
          // table reads to the top and needs a register per level read.
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // 5. Sums: the four lanes of a 16-lane row that hold one (row, batch)
  //    value add up by DPP; lanes 16 j + q (j = 0-3) then leave their
  //    row's sum in LDS as partial 4 slice + j of that output, and one
  //    thread per output adds its 16 partials in order.  The activations'
  //    LDS is free once every wave is past its last products.
  __syncthreads();
  float* dump = xs;  // [kMfMaxRows][NP][NB]
#pragma unroll
  for (int i = 0; i < MQ; ++i)
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float v = late ? acc[i][h][m] * lnorm[i] : acc[i][h][m];
        acc[i][h][m] = mf_row_sum4(v);
      }
  if ((lane & 12) == 0) {
    const int part = 4 * slice + (lane >> 4);
#pragma unroll
    for (int i = 0; i < MQ; ++i) {
      const int r = 4 * (rsub + SUBSETS * i) + q;  // < 48
#pragma unroll
      for (int h = 0; h < NH; ++h)
        *reinterpret_cast<float4*>(dump + (r * NP + part) * NB + 4 * h) =
            make_float4(acc[i][h][0], acc[i][h][1], acc[i][h][2], acc[i][h][3]);
    }
    wait_lds_writes();  // the stored sums keep their registers until the LDS has them
#pragma unroll
    for (int i = 0; i < MQ; ++i)
#pragma unroll
      for (int h = 0; h < NH; ++h) hold_values(acc[i][h][0], acc[i][h][1], acc[i][h][2], acc[i][h][3]);
  }
  __syncthreads();
  const float inv_g = 1.0f / static_cast<float>(G);  // exact: a power of two
  for (int o = t; o < block_rows * NB; o += BLOCK) {
    const int r = o / NB, m = o % NB;
    if (b0 + m < a.batch) {
      const float* src = dump + r * NP * NB + m;
      float sum = src[0];
#pragma unroll
      for (int p = 1; p < NP; ++p) sum += src[p * NB];
      a.y[(b0 + m) * n_out + row_base + r] = sum * inv_g;
    }
  }
}


// ---- launchers ------------------------------------------------------------------

// Largest grid.y of one launch.
constexpr int64_t kMaxGridY = 65535;

// Rows per wave of the pair-table kernel (the most a wave's registers hold).
constexpr int kPairMaxRows = 8;

hipError_t launch_pair_rot(const MatvecArgs& a, const LevelTable& lv, int log2g, int rows_per_block, hipStream_t s) {
  const int64_t blocks = (a.n_out + rows_per_block - 1) / rows_per_block;
  // One batch row per grid row, at most kMaxGridY per launch.
  for (int64_t b0 = 0; b0 < a.batch; b0 += kMaxGridY) {
    MatvecArgs part = a;
    part.x = a.x + b0 * a.k;
    part.y = a.y + b0 * a.n_out;
    part.batch = a.batch - b0 < kMaxGridY ? a.batch - b0 : kMaxGridY;
    if (log2g == 5)
      hipLaunchKernelGGL((matvec_pair_rot_kernel<kPairMaxRows, true>), dim3(static_cast<unsigned>(blocks),
                         static_cast<unsigned>(part.batch)), dim3(kPairBlock), 0, s, part, lv, log2g, rows_per_block);
    else
      hipLaunchKernelGGL((matvec_pair_rot_kernel<kPairMaxRows, false>), dim3(static_cast<unsigned>(blocks),
                         static_cast<unsigned>(part.batch)), dim3(kPairBlock), 0, s, part, lv, log2g, rows_per_block);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_mfma_rot(const MatvecArgs& a, const LevelTable& lv, int sbits, int log2g, int rows_per_block,
                           hipStream_t s) {
  const int64_t blocks = (a.n_out + rows_per_block - 1) / rows_per_block;
  const int nh = a.batch > 4 ? 2 : 1;
  const int64_t nb = 4 * nh;
  // Batch chunks of 4 NH rows along grid.y, at most kMaxGridY per launch.
  for (int64_t c0 = 0; c0 * nb < a.batch; c0 += kMaxGridY) {
    MatvecArgs part = a;
    part.x = a.x + c0 * nb * a.k;
    part.y = a.y + c0 * nb * a.n_out;
    part.batch = a.batch - c0 * nb;
    const int64_t chunks = (part.batch + nb - 1) / nb;
    const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(chunks < kMaxGridY ? chunks : kMaxGridY));
#define CQ_MF(SB, NH) hipLaunchKernelGGL((matvec_mfma_kernel<SB, NH, false, 4096>), grid, dim3(kMfBlock), 0, s, part, lv, log2g, rows_per_block, MfMany{})
    if (nh == 2) {
      if (sbits == 2) CQ_MF(2, 2); else if (sbits == 3) CQ_MF(3, 2); else CQ_MF(4, 2);
    } else {
      if (sbits == 2) CQ_MF(2, 1); else if (sbits == 3) CQ_MF(3, 1); else CQ_MF(4, 1);
    }
#undef CQ_MF
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The many-matrix form: one launch per batch chunk of nb <= 8 rows over
// blocks row blocks (the prefix bstart built with rows_per_block), in passes
// of PC columns.
template <int PC>
hipError_t launch_mfma_many_pc(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks, int sbits,
                               const LevelTable& lv, const float* xr, int64_t b0, int nb, int log2g,
                               int rows_per_block, hipStream_t s) {
  const MfMany many{table, bstart, n, xr, b0, nb};
  MatvecArgs a{};
  const dim3 grid(static_cast<unsigned>(blocks));
#define CQ_MFM(SB, NH) hipLaunchKernelGGL((matvec_mfma_kernel<SB, NH, true, PC>), grid, dim3(PC / 8), 0, s, a, lv, log2g, rows_per_block, many)
  if (nb > 4) {
    if (sbits == 2) CQ_MFM(2, 2); else if (sbits == 3) CQ_MFM(3, 2); else CQ_MFM(4, 2);
  } else {
    if (sbits == 2) CQ_MFM(2, 1); else if (sbits == 3) CQ_MFM(3, 1); else CQ_MFM(4, 1);
  }
#undef CQ_MFM
  return hipGetLastError();
}

template <int SB, int NB>
hipError_t launch_rot_nb(const MatvecArgs& a, const LevelTable& lv, int log2g, int blocks_per_cu,
                         hipStream_t s) {
  // Rows per group (RB * NB <= 32 partial sums in registers) and units of
  // codes in flight (at most 32 dwords of codes per thread).
  constexpr int RB = NB <= 2 ? 8 : NB <= 4 ? 4 : 2;
  constexpr int PF = 2;
  // Row groups per block: the rotation of the block's activations is paid
  // once per block, so blocks are as large as filling the chip allows
  // (blocks_per_cu blocks per compute unit over all batch chunks).
  const int64_t groups = (a.n_out + RB - 1) / RB;
  const int64_t n_chunks = (a.batch + NB - 1) / NB;
  int64_t target = static_cast<int64_t>(device_cu_count()) * blocks_per_cu / (n_chunks < blocks_per_cu ? n_chunks : blocks_per_cu);
  target = target < 1 ? 1 : target;
  int64_t rg = (groups + target - 1) / target;
  rg = rg < 1 ? 1 : rg > 64 ? 64 : rg;
  const int64_t blocks = (groups + rg - 1) / rg;
  // Batch chunks of NB rows along grid.y, at most kMaxGridY per launch.
  for (int64_t c0 = 0; c0 * NB < a.batch; c0 += kMaxGridY) {
    MatvecArgs part = a;
    part.x = a.x + c0 * NB * a.k;
    part.y = a.y + c0 * NB * a.n_out;
    part.batch = a.batch - c0 * NB;
    const int64_t chunks = (part.batch + NB - 1) / NB;
    hipLaunchKernelGGL((matvec_rot_kernel<SB, NB, RB, PF>),
                       dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(chunks < kMaxGridY ? chunks : kMaxGridY)),
                       dim3(kRotBlock), 0, s, part, lv, log2g, static_cast<int>(rg));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int SB>
hipError_t launch_rot_sb(const MatvecArgs& a, const LevelTable& lv, int log2g, int blocks_per_cu,
                         hipStream_t s) {
  // Batch chunks (grid.y) of 8 rows (16 x 8 activations per thread, 214
  // VGPRs) or of at most 4.
  // From 16 rows, chunks of 8: the codes are decoded and the activations
  // rotated once per 8 rows (11008x4096 at batch 16: 63 us against 68 in
  // chunks of 4).  At batch 8 one chunk halves the blocks of this
  // latency-bound launch (40.5 us against 37.0), so it keeps two of 4.
  if (a.batch >= 16) return launch_rot_nb<SB, 8>(a, lv, log2g, blocks_per_cu, s);
  switch (a.batch >= 4 ? 4 : a.batch) {
    case 1: return launch_rot_nb<SB, 1>(a, lv, log2g, blocks_per_cu, s);
    case 2: return launch_rot_nb<SB, 2>(a, lv, log2g, blocks_per_cu, s);
    case 3: return launch_rot_nb<SB, 3>(a, lv, log2g, blocks_per_cu, s);
    default: return launch_rot_nb<SB, 4>(a, lv, log2g, blocks_per_cu, s);
  }
}

constexpr int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 256 ? 8 : 7; }

}  // namespace kr

// Longest rows of the pair-table kernel (its row offsets are 32-bit).
constexpr int64_t kPairMaxK = int64_t(1) << 26;

MatvecOnePlan matvec_one_plan(int sbits, int64_t n_out, int64_t k, int64_t batch) {
  // 2-bit fields at batch 1 take the pair-table kernel with about an equal
  // share of the rows for every compute unit (one block each; at most 8 rows
  // per wave, so a block takes at most 64).
  if (sbits == 2 && batch == 1 && k <= kPairMaxK && k % 64 == 0) {
    const int64_t cus = device_cu_count();
    int64_t rpb = (n_out + cus - 1) / cus;
    const int64_t cap = static_cast<int64_t>(kr::kPairWaves) * kr::kPairMaxRows;
    rpb = rpb < 1 ? 1 : rpb > cap ? cap : rpb;
    return MatvecOnePlan{static_cast<int>(rpb), 0, 0};
  }
  // Two or more batch rows take the matrix-core kernel: one block of up to
  // 48 rows per compute unit.  Rows of a multiple of 64 columns keep every
  // lane's 64-column run inside the row and its code loads aligned.
  if (batch >= 2 && k <= kPairMaxK && k % 64 == 0) {
    const int64_t cus = device_cu_count();
    int64_t rpb = (n_out + cus - 1) / cus;
    const int64_t cap = static_cast<int64_t>(kr::kMfSubsets) * 4 * kr::mf_quads(sbits, batch > 4 ? 2 : 1);
    rpb = rpb < 1 ? 1 : rpb > cap ? cap : rpb;
    return MatvecOnePlan{0, 0, static_cast<int>(rpb)};
  }
  return MatvecOnePlan{0, 2, 0};
}

int mfma_rows_cap(int sbits, int nb) { return kr::kMfSubsets * 4 * kr::mf_quads(sbits, nb > 4 ? 2 : 1); }

bool mfma_fits(int64_t k) { return k <= kPairMaxK && k % 64 == 0; }

hipError_t launch_mfma_many(const MatvecDesc* table, const int64_t* bstart, int n, int64_t blocks, int sbits,
                            const LevelTable& lv, const float* xr, int64_t b0, int nb, int log2g,
                            int rows_per_block, int pass_cols, hipStream_t stream) {
  if (blocks <= 0) return hipSuccess;
  if (nb < 1 || nb > 8 || sbits < 2 || sbits > 4 || rows_per_block < 1 || rows_per_block > mfma_rows_cap(sbits, nb))
    return hipErrorInvalidValue;
  if (pass_cols == 2048)
    return kr::launch_mfma_many_pc<2048>(table, bstart, n, blocks, sbits, lv, xr, b0, nb, log2g, rows_per_block, stream);
  if (pass_cols == 4096)
    return kr::launch_mfma_many_pc<4096>(table, bstart, n, blocks, sbits, lv, xr, b0, nb, log2g, rows_per_block, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_matvec_one(const MatvecArgs& a, int sbits, const LevelTable& lv, int group_size,
                             const MatvecOnePlan& plan, hipStream_t stream) {
  if (a.n_out <= 0 || a.batch <= 0) return hipSuccess;
  const int log2g = kr::log2_group(group_size);
  if ((1 << log2g) != group_size) return hipErrorInvalidValue;
  if (plan.mfma_rows_per_block) {
    if (a.k > kPairMaxK || a.k % 64 || sbits < 2 || sbits > 4 ||
        plan.mfma_rows_per_block > kr::kMfSubsets * 4 * kr::mf_quads(sbits, a.batch > 4 ? 2 : 1))
      return hipErrorInvalidValue;
    return kr::launch_mfma_rot(a, lv, sbits, log2g, plan.mfma_rows_per_block, stream);
  }
  if (plan.pair_rows_per_block) {
    if (sbits != 2 || a.k > kPairMaxK || a.k % 64 || plan.pair_rows_per_block > kr::kPairWaves * kr::kPairMaxRows)
      return hipErrorInvalidValue;
    return kr::launch_pair_rot(a, lv, log2g, plan.pair_rows_per_block, stream);
  }
  const int bpc = plan.blocks_per_cu > 0 ? plan.blocks_per_cu : 1;
  switch (sbits) {
    case 2: return kr::launch_rot_sb<2>(a, lv, log2g, bpc, stream);
    case 3: return kr::launch_rot_sb<3>(a, lv, log2g, bpc, stream);
    case 4: return kr::launch_rot_sb<4>(a, lv, log2g, bpc, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cq
