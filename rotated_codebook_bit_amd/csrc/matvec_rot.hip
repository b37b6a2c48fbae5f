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
// Two kernels:
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
//     block in a fixed order.
// Both are deterministic: every sum runs in a fixed order.

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

// ---- pair tables, one batch row per grid row ------------------------------------

constexpr int kPairWaves = 8;
constexpr int kPairBlock = kPairWaves * kWave;
// Rotated x of a tile in LDS: column c at float c + 2 (c / 16), so that the
// table build's reads (lane l reads columns 16 l + 2 w, +1) fall on distinct
// banks and the rotation's writes (lane l of wave w writes 128 w + 2 l, +1)
// stay conflict free.
constexpr int kTilePadded = kTile + kTile / 8;
__device__ __forceinline__ int xpad(int c) { return c + 2 * (c >> 4); }
// Tiles of rotated x held in LDS at once (72 KiB at most); longer rows are
// processed in windows of this many tiles.
constexpr int kMaxWindowTiles = 16;

template <int RPW, int PF>
__global__ void __launch_bounds__(kPairBlock, 2)
matvec_pair_rot_kernel(MatvecArgs a, LevelTable lv, int log2g, int window_tiles) {
  extern __shared__ __attribute__((aligned(16))) float xs[];  // window_tiles * kTilePadded
  __shared__ __attribute__((aligned(16))) float tab[8 * 16 * kWave];
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t k = a.k, n_out = a.n_out;
  const int64_t brow = blockIdx.y;  // batch row
  const int64_t row0 = static_cast<int64_t>(blockIdx.x) * (kPairWaves * RPW) + w * RPW;
  const int64_t row_bytes = k / 4, ngr = k >> log2g;
  const int64_t n_tiles = (k + kTile - 1) / kTile;
  const int G = 1 << log2g;
  const float* __restrict__ xrow = a.x + brow * k;

  // The wave's rows as buffer resources: rows past the end of the matrix lie
  // outside them and read as zero (their sums are never stored).  The host
  // sends a matrix here only when k <= 2^28, so RPW <= 16 rows of codes and
  // every offset below stay under 2^31.
  const int64_t rows_in = n_out - row0 < RPW ? (n_out - row0 > 0 ? n_out - row0 : 0) : RPW;
  const auto codes_src = rsrc(a.packed + (rows_in ? row0 * row_bytes : 0), rows_in * row_bytes);
  const auto norms_src = rsrc(a.norms + (rows_in ? row0 * ngr : 0), rows_in * ngr * 2);
  int soff_c[RPW], soff_n[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int rr = r < rows_in ? r : (rows_in > 0 ? static_cast<int>(rows_in) - 1 : 0);
    soff_c[r] = __builtin_amdgcn_readfirstlane(static_cast<int>(rr * row_bytes));
    soff_n[r] = __builtin_amdgcn_readfirstlane(static_cast<int>(2 * rr * ngr));
  }
  const float c0l = lv.c[0], c1l = lv.c[1], c2l = lv.c[2], c3l = lv.c[3];
  const uint32_t lane_bytes = 4u * static_cast<uint32_t>(lane);

  // Codes of tile t for the wave's rows, PF tiles in flight.  A lane without
  // columns in the tile offsets by 2^30, past every resource, and reads zero.
  uint32_t codes[PF][RPW];
  _Float16 norm[PF][RPW];
  auto issue = [&](int64_t t, uint32_t (&c)[RPW], _Float16 (&nv)[RPW]) {
    const int64_t c0 = t * kTile + kChunk * lane;
    const bool active = t < n_tiles && c0 < k;  // k % G == 0: whole chunks only
    const int coff = active ? static_cast<int>(c0 / 4) : (1 << 30);
    const int noff = active ? static_cast<int>(2 * (c0 >> log2g)) : (1 << 30);
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      c[r] = __builtin_amdgcn_raw_buffer_load_b32(codes_src, coff, soff_c[r], 2);  // nt: read once
      nv[r] = __builtin_bit_cast(_Float16, __builtin_amdgcn_raw_buffer_load_b16(norms_src, noff, soff_n[r], 0));
    }
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) issue(j, codes[j], norm[j]);

  float acc[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) acc[r] = 0.0f;

  // Butterfly signs of the cross-lane stages (lane stride s = 1 .. 32).
  float sgn[6];
#pragma unroll
  for (int i = 0; i < 6; ++i) sgn[i] = (lane >> i) & 1 ? -1.0f : 1.0f;
  const int in_wave = G < 2 * kWave ? G : 2 * kWave;  // butterfly width inside a wave

  for (int64_t w0 = 0; w0 < n_tiles; w0 += window_tiles) {
    const int nt = static_cast<int>(n_tiles - w0 < window_tiles ? n_tiles - w0 : window_tiles);
    __syncthreads();  // the previous window's rotated x is no longer read
    // Load the window's activations (two per thread per tile), all loads
    // first, then rotate and store each tile.
    float2 raw[kMaxWindowTiles];
#pragma unroll
    for (int i = 0; i < kMaxWindowTiles; ++i) {
      const int64_t c = (w0 + i) * kTile + 2 * threadIdx.x;
      raw[i] = i < nt && c < k ? *reinterpret_cast<const float2*>(xrow + c) : make_float2(0.0f, 0.0f);
    }
#pragma unroll
    for (int i = 0; i < kMaxWindowTiles; ++i) {
      if (i < nt) {
        float y0 = raw[i].x + raw[i].y, y1 = raw[i].x - raw[i].y;
#pragma unroll
        for (int st = 0; st < 6; ++st) {
          if ((2 << st) < in_wave) {
            y0 = xstage(y0, 1 << st, sgn[st]);
            y1 = xstage(y1, 1 << st, sgn[st]);
          }
        }
        *reinterpret_cast<float2*>(xs + i * kTilePadded + xpad(2 * threadIdx.x)) = make_float2(y0, y1);
        wait_lds_writes();  // the stored values keep their registers until the LDS has them
        hold_values(y0, y1);
      }
    }

    for (int i0 = 0; i0 < nt; i0 += PF) {
#pragma unroll
      for (int j = 0; j < PF; ++j) {
        const int i = i0 + j;
        if (i >= nt) break;  // the same for the whole block
        const int64_t t = w0 + i;
        const int64_t c0 = t * kTile + kChunk * lane;
        const bool active = c0 < k;
        __syncthreads();  // rotated x stored; the previous tile's table reads are done
        if (active) {
          // Pair w of this lane's chunk: columns 16 lane + 2 w, + 1 of the tile.
          const float* xt = xs + i * kTilePadded;
          const int c = kChunk * lane + 2 * w;
          float x0, x1;
          if (G > 2 * kWave) {
            // The last butterfly stage (stride 128) joins two waves' halves.
            const int lo = c & ~128;
            const float2 p = *reinterpret_cast<const float2*>(xt + xpad(lo));
            const float2 q = *reinterpret_cast<const float2*>(xt + xpad(lo + 128));
            x0 = c & 128 ? p.x - q.x : p.x + q.x;
            x1 = c & 128 ? p.y - q.y : p.y + q.y;
          } else {
            const float2 p = *reinterpret_cast<const float2*>(xt + xpad(c));
            x0 = p.x;
            x1 = p.y;
          }
          const float pa[4] = {c0l * x0, c1l * x0, c2l * x0, c3l * x0};
          const float cb[4] = {c0l, c1l, c2l, c3l};
          float e[16];
#pragma unroll
          for (int bb = 0; bb < 4; ++bb)
#pragma unroll
            for (int q = 0; q < 4; ++q) e[q + 4 * bb] = __builtin_fmaf(cb[bb], x1, pa[q]);
          float* dst = tab + (16 * w) * kWave + lane;
#pragma unroll
          for (int v = 0; v < 16; ++v) dst[v * kWave] = e[v];
          wait_lds_writes();
#pragma unroll
          for (int v = 0; v < 16; ++v) hold_values(e[v]);
        }
        __syncthreads();
        if (active) {
          const char* tb = reinterpret_cast<const char*>(tab);
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            const uint32_t cw = codes[j][r];
            const uint32_t ev = cw & 0x0F0F0F0Fu, od = (cw >> 4) & 0x0F0F0F0Fu;
            float s = 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              // Byte 0 of the address is the lane's (4 l), byte 1 the pair's
              // code v (its nibble, spread one per byte), bytes 2-3 zero.
              const uint32_t e = (q & 1) ? od : ev;
              const uint32_t addr = __builtin_amdgcn_perm(e, lane_bytes, 0x0C0C0000u | ((4u + (q >> 1)) << 8));
              const float v = *reinterpret_cast<const float*>(tb + addr + 4096 * q);
              s = q ? s + v : v;
            }
            acc[r] = __builtin_fmaf(static_cast<float>(norm[j][r]), s, acc[r]);
          }
        }
        issue(t + PF, codes[j], norm[j]);
      }
    }
  }

  // Reduce the RPW row sums over the 64 lanes: each exchange halves the
  // values a lane holds (the lane with the offset's bit set keeps the upper
  // half), then the remaining offsets sum within groups of 64 / RPW lanes.
  constexpr int kSteps = RPW >= 16 ? 4 : RPW >= 8 ? 3 : RPW >= 4 ? 2 : RPW >= 2 ? 1 : 0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) {
    const int o = 32 >> i, V = RPW >> i;
    const bool hi = lane & o;
#pragma unroll
    for (int jj = 0; jj < V / 2; ++jj) {
      const float lo_sum = acc[jj] + __shfl_xor(acc[jj], o, kWave);
      const float hi_sum = acc[jj + V / 2] + __shfl_xor(acc[jj + V / 2], o, kWave);
      acc[jj] = hi ? hi_sum : lo_sum;
    }
  }
  float s = acc[0];
#pragma unroll
  for (int o = 32 >> kSteps; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
  s *= 1.0f / static_cast<float>(G);  // exact: a power of two
  int r = 0;
#pragma unroll
  for (int i = 0; i < kSteps; ++i) r += ((lane >> (5 - i)) & 1) * (RPW >> (i + 1));
  if ((lane & (64 / RPW - 1)) == 0 && row0 + r < n_out) a.y[brow * n_out + row0 + r] = s;
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
//     holds level[v & 3], table 1 (4 KiB further) level[v >> 2];
//   4-bit fields: one code per nibble, one table;
//   3-bit fields: one 8-entry table, the code extracted by a shift.
template <int SB>
struct LaneTab {
  static constexpr int entries = SB == 3 ? 8 : 16;
  static constexpr int tables = SB == 2 ? 2 : 1;
  static constexpr int floats = tables * 16 * kWave;
  static __device__ __forceinline__ void fill(float* tab, const LevelTable& lv, int t) {
    for (int i = t; i < floats; i += kRotBlock) {
      const int tb = i / (16 * kWave), v = (i / kWave) % 16;
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
        v[2 * q + 1] = *reinterpret_cast<const float*>(tb + addr + 16 * 4 * kWave);
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
__global__ void __launch_bounds__(kRotBlock)
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
  // Rotated activations of this thread's 16 columns of pass p: the 16-point
  // butterfly inside the thread, then log2(G / 16) stages across the lanes
  // that share the group.
  auto load_x = [&](int p) __attribute__((always_inline)) {
    const int64_t c0 = static_cast<int64_t>(p) * kPass + kChunk * t;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bool live = c0 < k && b0 + b < a.batch;
      const float4* src = reinterpret_cast<const float4*>(a.x + (b0 + b) * k + c0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = live ? src[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        xv[b][4 * i] = v.x;
        xv[b][4 * i + 1] = v.y;
        xv[b][4 * i + 2] = v.z;
        xv[b][4 * i + 3] = v.w;
      }
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

  using CodeT = typename std::conditional<SB == 2, uint32_t, uint64_t>::type;
  CodeT codes[PF][RB];
  float scale[PF][RB];
  auto issue = [&](int u, CodeT (&c)[RB], float (&sc)[RB]) __attribute__((always_inline)) {
    const int g = u / n_pass, p = u - g * n_pass;
    const int64_t c0 = static_cast<int64_t>(p) * kPass + kChunk * t;
    const bool live = u < n_units && c0 < k;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      int64_t row = row_base + static_cast<int64_t>(g) * RB + r;
      row = row < n_out ? row : n_out - 1;  // rows past the end re-read the last; never stored
      c[r] = live ? static_cast<CodeT>(codes16<SB>(a.packed + row * row_bytes, c0)) : CodeT(0);
      sc[r] = live ? static_cast<float>(__builtin_bit_cast(_Float16, a.norms[row * ngr + (c0 >> log2g)])) * inv_g
                   : 0.0f;
    }
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) issue(j, codes[j], scale[j]);
  if (one_pass) load_x(0);

  float acc[RB][NB];
  for (int u0 = 0; u0 < n_units; u0 += PF) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int u = u0 + j;
      if (u >= n_units) break;  // the same for the whole block
      const int g = u / n_pass, p = u - g * n_pass;
      if (p == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) acc[r][b] = 0.0f;
      }
      if (!one_pass) load_x(p);
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
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[r][b] = __builtin_fmaf(scale[j][r], part[b], acc[r][b]);
      }
      issue(u + PF, codes[j], scale[j]);
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

// ---- launchers ------------------------------------------------------------------

// Largest grid.y of one launch.
constexpr int64_t kMaxGridY = 65535;

template <int RPW, int PF>
hipError_t launch_pair_rot(const MatvecArgs& a, const LevelTable& lv, int log2g, hipStream_t s) {
  constexpr int rows = kPairWaves * RPW;
  const int64_t blocks = (a.n_out + rows - 1) / rows;
  const int64_t n_tiles = (a.k + kTile - 1) / kTile;
  const int window = static_cast<int>(n_tiles < kMaxWindowTiles ? n_tiles : kMaxWindowTiles);
  const size_t lds = static_cast<size_t>(window) * kTilePadded * sizeof(float);
  // One batch row per grid row, at most kMaxGridY per launch.
  for (int64_t b0 = 0; b0 < a.batch; b0 += kMaxGridY) {
    MatvecArgs part = a;
    part.x = a.x + b0 * a.k;
    part.y = a.y + b0 * a.n_out;
    part.batch = a.batch - b0 < kMaxGridY ? a.batch - b0 : kMaxGridY;
    hipLaunchKernelGGL((matvec_pair_rot_kernel<RPW, PF>), dim3(static_cast<unsigned>(blocks),
                       static_cast<unsigned>(part.batch)), dim3(kPairBlock), lds, s, part, lv, log2g, window);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int SB, int NB>
hipError_t launch_rot_nb(const MatvecArgs& a, const LevelTable& lv, int log2g, int blocks_per_cu,
                         hipStream_t s) {
  // Rows per group (RB * NB <= 32 partial sums in registers) and units of
  // codes in flight (at most 32 dwords of codes per thread).
  constexpr int RB = NB <= 4 ? 8 : 4;
  constexpr int PF = SB == 2 ? 4 : NB <= 4 ? 2 : 3;
  // Row groups per block: the rotation of the block's activations is paid
  // once per block, so blocks are as large as filling the chip allows.
  const int64_t groups = (a.n_out + RB - 1) / RB;
  const int64_t target = static_cast<int64_t>(device_cu_count()) * blocks_per_cu;
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
  switch (a.batch >= 8 ? 8 : a.batch) {
    case 1: return launch_rot_nb<SB, 1>(a, lv, log2g, blocks_per_cu, s);
    case 2: return launch_rot_nb<SB, 2>(a, lv, log2g, blocks_per_cu, s);
    case 3: return launch_rot_nb<SB, 3>(a, lv, log2g, blocks_per_cu, s);
    case 4: return launch_rot_nb<SB, 4>(a, lv, log2g, blocks_per_cu, s);
    case 5: return launch_rot_nb<SB, 5>(a, lv, log2g, blocks_per_cu, s);
    case 6: return launch_rot_nb<SB, 6>(a, lv, log2g, blocks_per_cu, s);
    case 7: return launch_rot_nb<SB, 7>(a, lv, log2g, blocks_per_cu, s);
    default: return launch_rot_nb<SB, 8>(a, lv, log2g, blocks_per_cu, s);
  }
}

constexpr int log2_group(int g) { return g == 32 ? 5 : g == 64 ? 6 : g == 256 ? 8 : 7; }

}  // namespace kr

MatvecOnePlan matvec_one_plan(int sbits, int64_t n_out, int64_t k, int64_t batch) {
  // 2-bit fields at batch 1 take the pair-table kernel: the most rows per
  // wave (8, 4, 2) that still gives every compute unit two blocks.
  if (sbits == 2 && batch == 1 && k <= (int64_t(1) << 28)) {
    const int64_t target = 2 * static_cast<int64_t>(device_cu_count());
    for (int rpw = 8; rpw > 2; rpw /= 2)
      if ((n_out + kr::kPairWaves * rpw - 1) / (kr::kPairWaves * rpw) >= target) return MatvecOnePlan{rpw, 0};
    return MatvecOnePlan{2, 0};
  }
  return MatvecOnePlan{0, 1};
}

hipError_t launch_matvec_one(const MatvecArgs& a, int sbits, const LevelTable& lv, int group_size,
                             const MatvecOnePlan& plan, hipStream_t stream) {
  if (a.n_out <= 0 || a.batch <= 0) return hipSuccess;
  const int log2g = kr::log2_group(group_size);
  if ((1 << log2g) != group_size) return hipErrorInvalidValue;
  if (plan.pair_rows_per_wave) {
    if (sbits != 2 || a.k > (int64_t(1) << 28)) return hipErrorInvalidValue;
    switch (plan.pair_rows_per_wave) {
      case 2: return kr::launch_pair_rot<2, 8>(a, lv, log2g, stream);
      case 4: return kr::launch_pair_rot<4, 4>(a, lv, log2g, stream);
      case 8: return kr::launch_pair_rot<8, 2>(a, lv, log2g, stream);
      default: return hipErrorInvalidValue;
    }
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
