// CQ quantize kernels for gfx950.
//
// Method (web pages, by title and section):
//   "Cactus Quants CQ2-bit Quantization: Extreme Compression for Edge LLMs",
//     Group-wise Weight Partitioning (groups of 128 along the last axis, the
//     last group zero-padded), Hadamard Rotation, The CQ2-bit Implementation
//     Pipeline (pad, rotate, normalise, nearest level);
//   "How Quantization Codebooks Are Trained in Cactus Quants",
//     Iterative Refinement of Quantization Levels (decision boundaries are
//     the midpoints of neighbouring levels), Production Codebook Generation
//     and Caching (levels divided by sqrt(G), i.e. z = sqrt(G) y / ||y||
//     compared against N(0,1) levels);
//   "How CQ2-bit Quantization Contributes to Needle 2's Small Footprint",
//     Per-Group Storage Breakdown (indices + one fp16 norm per group).
//
// Mapping to the hardware
//   * One lane owns one whole group: all 7 butterfly stages of the 128-point
//     Walsh-Hadamard transform run in that lane's registers, with no
//     cross-lane traffic, and the group norm is a per-lane sum.
//   * A wave handles a batch of 64 consecutive groups.  The batch is copied
//     into a wave-private LDS buffer by direct-to-LDS loads
//     (global_load_lds_dwordx4): every load instruction moves 1 KiB of
//     contiguous HBM, so reads are fully coalesced although each lane later
//     needs a 256-byte (bf16) or 512-byte (fp32) stretch.  Each lane then reads
//     its group with ds_read_b128; chunk c of group g sits in physical chunk
//     slot c ^ (g & 15), which makes every such read conflict-free.
//   * The load of the next batch is issued right after the current batch has
//     been read out of LDS, so it overlaps the arithmetic.
//   * The butterfly is unnormalised (Y = H x with the +-1 Sylvester matrix).
//     z = sqrt(G) * (Y / sqrt(G)) / n = Y / n, so instead of dividing, the
//     thresholds are multiplied by the group norm n once per group.
//   * Three and four levels: two compares per element.  With mu the centre
//     and delta the half width of the outer pair of thresholds, and the
//     shifted value Y' = Y - mu*n,
//        h = [Y' > hmid*n],  q = [|Y'| > delta*n],
//        four levels: index = 2h + NOT(q XOR h);  three levels: 2h + NOT q.
//     Subtracting mu*n from every Y is the same as subtracting it from the
//     first element of the group before the transform (H maps e_0 to the
//     all-ones vector), so the shift costs one operation per group.
//   * Eight and sixteen levels: binary search over thresholds held in VGPRs.
//   * Bits are shifted into the packed word with add-with-carry from the
//     compare mask (acc = 2 acc + bit), LSB-first order per the ABI, so a
//     decision bit costs one compare and one add.

#include "cq_internal.h"

namespace cq {
namespace kq {

constexpr int kWaves = 4;
constexpr int kBlock = kWaves * kWave;
constexpr int kBlocksPerCu = 2;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

template <int L>
struct Shape {
  static constexpr int sbits = (L <= 4) ? 2 : (L == 8 ? 3 : 4);
  static constexpr int words = kGroup * sbits / 32;  // packed dwords per group
};

// Butterfly stages 2..7 (pairs at distance 2..64) in place; stage 1
// (distance 1) is done by the loader while the data is unpacked.
__device__ __forceinline__ void butterfly_from_stage2(float (&y)[kGroup]) {
#pragma unroll
  for (int h = 2; h < kGroup; h <<= 1) {
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

__device__ __forceinline__ uint32_t bit(bool b) { return b ? 1u : 0u; }

// acc * 2 + b in one add-with-carry whose carry-in is the wave's compare
// mask: the compare writes the mask straight into an SGPR pair and
// v_addc_co_u32 adds each lane's bit.  (Written as plain C++ the compiler
// materialises each bit with a select and merges it with shifts and ORs,
// about three times the instructions.)
__device__ __forceinline__ uint32_t shift_in(uint32_t acc, bool b) {
  const uint64_t mask = __builtin_amdgcn_ballot_w64(b);
  uint32_t r;
  uint64_t carry_out;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(acc), "s"(mask));
  return r;
}

// acc * 2 + [t > v] in two instructions with no mask register: t - v is
// negative (sign bit set) exactly when v > t, for every non-NaN t and v
// (a difference of two floats is zero only when they are equal, and
// rounding or flushing keeps its sign), and v_alignbit_b32 shifts that sign
// bit in: ({acc, d} >> 31) = (acc << 1) | (d >> 31).  Equal t and v give
// +0, bit 0, as the compare would.  Used for the two-compare decisions,
// where the mask form needs a wait state between each carry write and the
// next compare.  t is a rounded float32 threshold: the subtraction must
// not be contracted with the product that made t into one fma, which would
// compare against the unrounded product.
__device__ __forceinline__ uint32_t shift_in_gt(uint32_t acc, float v, float t) {
#pragma clang fp contract(off)
  const float d = t - v;
  return __builtin_amdgcn_alignbit(acc, __builtin_bit_cast(uint32_t, d), 31);
}

// Symmetric two-bit decisions (three levels, or four whose middle threshold
// is the centre of the outer pair: QuantParams::sym).  With the shifted
// value v and D = delta * ns, one product x = fma(v, k, +0), k = -2 / D,
// carries both decision bits in its top two bits:
//   bit 31 (sign)  = [v > 0]: k < 0, and the +0 addend turns the -0 of a
//                    zero product into +0, so v = +-0 gives 0;
//   bit 30         = [|x| >= 2] (exponent field >= 128, also for inf), i.e.
//                    |v| >= D up to the roundings of -2 / delta, of the
//                    (correctly rounded) division by ns and of the product:
//                    1.5 float32 ulps of the threshold, against 1 ulp for
//                    the compare with D = delta * ns.
// v_alignbit_b32 shifts both in at once: ({acc, x} >> 30) = acc << 2 | x >> 30.
// A word of 16 such pairs (s, q) becomes the index fields with one or two
// bitwise steps per word (finish_sym_word).
__device__ __forceinline__ uint32_t shift_in_pair(uint32_t acc, float v, float k) {
  const float x = __builtin_fmaf(v, k, 0.0f);
  return __builtin_amdgcn_alignbit(acc, __builtin_bit_cast(uint32_t, x), 30);
}

// (s, q) pairs -> index fields.  Four levels: s is the high bit h, and the
// low bit is NOT (q XOR h).  Three levels: h = s AND q, low bit NOT q.
template <int L>
__device__ __forceinline__ uint32_t finish_sym_word(uint32_t acc) {
  if constexpr (L == 4)
    return acc ^ (((acc >> 1) & 0x55555555u) ^ 0x55555555u);
  else
    return (acc & (acc << 1) & 0xAAAAAAAAu) | (~acc & 0x55555555u);
}

// Index by binary search over 7 thresholds (8 levels).
__device__ __forceinline__ uint32_t search8(float v, const float (&T)[kMaxLevels - 1]) {
  const bool b2 = v > T[3];
  const bool b1 = v > (b2 ? T[5] : T[1]);
  const float lo = b1 ? T[2] : T[0], hi = b1 ? T[6] : T[4];
  const bool b0 = v > (b2 ? hi : lo);
  return (bit(b2) << 2) | (bit(b1) << 1) | bit(b0);
}

// Index bits (b3, b2, b1, b0) by binary search over 15 thresholds.
__device__ __forceinline__ void search16(float v, const float (&T)[kMaxLevels - 1], bool& b3,
                                         bool& b2, bool& b1, bool& b0) {
  b3 = v > T[7];
  b2 = v > (b3 ? T[11] : T[3]);
  const float p0 = b3 ? T[9] : T[1], p1 = b3 ? T[13] : T[5];
  b1 = v > (b2 ? p1 : p0);
  const float r0 = b3 ? T[8] : T[0], r1 = b3 ? T[10] : T[2];
  const float r2 = b3 ? T[12] : T[4], r3 = b3 ? T[14] : T[6];
  const float s0 = b2 ? r2 : r0, s1 = b2 ? r3 : r1;
  b0 = v > (b1 ? s1 : s0);
}

// Stages after stage 1: the shift used by the two-compare decision, then
// butterfly stages 2..7.  y holds the stage-1 outputs, S the sum of squares
// of the group.  Returns the group norm; *ns is the scale the decisions use
// (the norm, or 1 for an all-zero group, whose z is 0: deciding with scale 1
// compares 0 against the thresholds themselves).
template <int L>
__device__ __forceinline__ float forward_group(float (&y)[kGroup], float S, const QuantParams& p,
                                               float* ns_out) {
  const float n = __builtin_sqrtf(S);
  const float ns = S > 0.0f ? n : 1.0f;
  if constexpr (L == 3 || L == 4) {
    const float sh = p.mu * ns;
    y[0] -= sh;
    y[1] -= sh;
  }
  butterfly_from_stage2(y);
  *ns_out = ns;
  return n;
}

// Everything after stage 1: shift, stages 2..7, decisions, packing.
// y holds the stage-1 outputs, S the sum of squares of the group.
template <int L>
__device__ __forceinline__ uint16_t finish_group(float (&y)[kGroup], float S, const QuantParams& p,
                                                 uint32_t (&words)[Shape<L>::words]) {
  float ns;
  const float n = forward_group<L>(y, S, p, &ns);
  if constexpr (L == 3 || L == 4) {
    if (p.sym) {  // the same for the whole launch
      const float k = p.neg2_over_delta / ns;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        uint32_t acc = 0;
#pragma unroll
        for (int pos = 15; pos >= 0; --pos) acc = shift_in_pair(acc, y[16 * wd + pos], k);
        words[wd] = finish_sym_word<L>(acc);
      }
      return __builtin_bit_cast(uint16_t, static_cast<_Float16>(n));
    }
    const float A = p.hmid * ns, D = p.delta * ns;
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      uint32_t acc = 0;
#pragma unroll
      for (int pos = 15; pos >= 0; --pos) {
        const float v = y[16 * wd + pos];
        acc = shift_in_gt(acc, v, A);
        acc = shift_in_gt(acc, __builtin_fabsf(v), D);
      }
      if constexpr (L == 4)
        acc ^= ((acc >> 1) & 0x55555555u) ^ 0x55555555u;
      else
        acc ^= 0x55555555u;
      words[wd] = acc;
    }
  } else if constexpr (L == 8) {
    float T[kMaxLevels - 1];
#pragma unroll
    for (int i = 0; i < 7; ++i) T[i] = p.thr[i] * ns;
#pragma unroll
    for (int i = 0; i < Shape<L>::words; ++i) words[i] = 0;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const uint32_t idx = search8(y[j], T);
      const int pos = 3 * j, wd = pos >> 5, off = pos & 31;
      words[wd] |= idx << off;
      if (off > 29) words[wd + 1] |= idx >> (32 - off);
    }
  } else {
    float T[kMaxLevels - 1];
#pragma unroll
    for (int i = 0; i < 15; ++i) T[i] = p.thr[i] * ns;
#pragma unroll
    for (int wd = 0; wd < 16; ++wd) {
      uint32_t acc = 0;
#pragma unroll
      for (int pos = 7; pos >= 0; --pos) {
        bool b3, b2, b1, b0;
        search16(y[8 * wd + pos], T, b3, b2, b1, b0);
        acc = shift_in(acc, b3);
        acc = shift_in(acc, b2);
        acc = shift_in(acc, b1);
        acc = shift_in(acc, b0);
      }
      words[wd] = acc;
    }
  }
  const _Float16 h = static_cast<_Float16>(n);
  return __builtin_bit_cast(uint16_t, h);
}

template <int L>
__device__ __forceinline__ void store_group(uint8_t* __restrict__ packed, uint16_t* __restrict__ norms,
                                            int64_t g, const uint32_t (&words)[Shape<L>::words],
                                            uint16_t n16, bool trits = false) {
  constexpr int W = Shape<L>::words;
  if constexpr (L == 3) {
    if (trits) {
      uint32_t t[13];
      fields_to_trits(words, t);
      uint16_t* dst = reinterpret_cast<uint16_t*>(packed + g * kTritBytes);
#pragma unroll
      for (int k = 0; k < 13; ++k) dst[k] = static_cast<uint16_t>(t[k]);
      norms[g] = n16;
      return;
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(packed + g * (W * 4));
#pragma unroll
  for (int i = 0; i < W / 4; ++i)
    dst[i] = make_uint4(words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]);
  norms[g] = n16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.lo * a.lo + a.hi * a.hi for a packed bf16 pair, in float32
// (v_dot2c_f32_bf16): the sum of squares of two elements in one instruction,
// straight from the packed pair.  The bf16 squares are exact in float32.
__device__ __forceinline__ float sumsq2_bf16(uint32_t a, float acc) {
  const bf16x2_t v = __builtin_bit_cast(bf16x2_t, a);
  return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

// Stage 1 from one 32-bit word holding elements 2i (low half) and 2i+1, plus
// the pair's contribution to the sum of squares.
__device__ __forceinline__ void stage1_bf16(uint32_t u, float& s, float& d, float& acc) {
  const float a = __builtin_bit_cast(float, u << 16);
  const float b = __builtin_bit_cast(float, u & 0xFFFF0000u);
  s = a + b;
  d = a - b;
  acc = sumsq2_bf16(u, acc);
}

// Buffer resource over [base, base + bytes): loads past the end return zero
// and stores past the end are dropped by the hardware, which handles the
// last, partial batch without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Groups of batch bt that exist (64 except for the last batch).
__device__ __forceinline__ int valid_in_batch(int64_t bt, int64_t n_groups) {
  const int64_t left = n_groups - bt * kWave;
  return static_cast<int>(left < kWave ? left : kWave);
}

// Where a batch's 64 groups lie: 16 slots of 4 consecutive groups, slot j
// at slot index first + j * step of the tensor.  Plain batches are
// contiguous (first = 16 bt, step = 1).  With bf16 input and 2- or 4-bit
// fields the full batches of a tensor are also taken S = kInterleaveBf16 at
// a time: batch r of such a super-batch owns slots r, r + S, ..., so that at
// any moment the neighbouring waves of the grid read neighbouring kilobytes.
// On the 7B-shaped bf16 model this cut quantize from 2.95-3.0 ms to 2.65 ms
// against 16 contiguous kilobytes per wave; S = 16 and 64 measured 2.7-2.8
// ms, widths that are not powers of two (24, 48) 2.9 ms.  Float32 input
// (2 KiB slots) was slower at every width (S = 8 / 16 / 32: 5.39 / 5.24 /
// 5.48 ms against 5.19) and keeps contiguous batches.  A slot's packed output is whole
// 128-byte lines at these widths (4 x 32 or 4 x 64 bytes), so no line is
// shared between waves; 3-bit fields (48 bytes a group) and trits keep the
// contiguous placement.  Norms are 8 bytes a slot, so a norm line is written
// by several waves (byte-masked stores; 1/128 of the traffic).
constexpr int kSlotGroups = 4;
constexpr int kSlots = kWave / kSlotGroups;
constexpr int kInterleaveBf16 = 32;
constexpr int kInterleaveF32 = 0;

struct Place {
  int64_t first;  // slot of the batch's first slot
  int step;       // slots between consecutive slots of the batch
};

// Super-batch width of a quantize launch (0: contiguous batches only).
template <int L, bool BF16, bool TRITS>
constexpr int interleave_width() {
  return (TRITS || Shape<L>::sbits == 3) ? 0 : (BF16 ? kInterleaveBf16 : kInterleaveF32);
}

template <int S>
__device__ __forceinline__ Place place_batch(int64_t bt, int64_t n_groups) {
  if constexpr (S > 0) {
    const int64_t full = n_groups / kWave;
    if (bt < full - full % S) return Place{(bt / S) * kSlots * S + bt % S, S};
  }
  return Place{bt * kSlots, 1};
}

// Offset, in groups from the batch's first group, of group g of the batch.
__device__ __forceinline__ int group_offset(int g, int step) {
  return (g / kSlotGroups) * step * kSlotGroups + g % kSlotGroups;
}

// DMA of batch bt into the wave's LDS buffer (see quantize_contig).
// Load instruction i fills LDS bytes [1024 i, 1024 i + 1024), i.e. kilobyte
// i % IPS of the batch's slot i / IPS (IPS kilobytes per slot).
template <int S, int GB, int NI, int R>
__device__ __forceinline__ void issue_batch(const uint8_t* __restrict__ w, int64_t bt,
                                            int64_t n_groups, uint8_t* buf,
                                            const uint32_t (&lane_part)[R]) {
  // Buffer-resource builtins exist only for the GPU target; the host pass
  // needs nothing but the kernel's signature for its launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  if constexpr (S == 0) {
    const auto src = make_rsrc(w + bt * kWave * GB, valid_in_batch(bt, n_groups) * GB);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_ptr_t)(buf + i * 1024), 16,
                                               i * 1024 + lane_part[i % R], 0, 0, 0);
  } else {
    constexpr int SLOT = kSlotGroups * GB;  // input bytes per slot
    constexpr int IPS = SLOT / 1024;
    const Place pl = place_batch<S>(bt, n_groups);
    const int bytes = pl.step == 1 ? valid_in_batch(bt, n_groups) * GB : ((kSlots - 1) * pl.step + 1) * SLOT;
    const auto src = make_rsrc(w + pl.first * SLOT, bytes);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_ptr_t)(buf + i * 1024), 16, lane_part[i % R],
                                               (i / IPS) * pl.step * SLOT + (i % IPS) * 1024, 0, 0);
  }
#endif
}

// Packed words and norm of every lane's group of batch bt.
template <int L, bool BF16, bool TRITS = false>
__device__ __forceinline__ void store_batch(uint8_t* __restrict__ packed, uint16_t* __restrict__ norms,
                                            int64_t bt, int64_t n_groups, int lane,
                                            const uint32_t (&words)[Shape<L>::words], uint16_t n16) {
  constexpr int PB = Shape<L>::words * 4;
#if defined(__HIP_DEVICE_COMPILE__)  // GPU-only builtins, as in issue_batch
  const int nv = valid_in_batch(bt, n_groups);
  const Place pl = place_batch<interleave_width<L, BF16, TRITS>()>(bt, n_groups);
  (void)pl;
  if constexpr (TRITS) {
    // 26 bytes per group at 2-byte alignment: 13 16-bit stores per lane.
    uint32_t t[13];
    fields_to_trits(words, t);
    const auto tdst = make_rsrc(packed + bt * kWave * kTritBytes, nv * kTritBytes);
#pragma unroll
    for (int k = 0; k < 13; ++k)
      __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(t[k]), tdst, lane * kTritBytes + 2 * k, 0, 0);
    const auto tndst = make_rsrc(norms + bt * kWave, nv * 2);
    __builtin_amdgcn_raw_buffer_store_b16(n16, tndst, lane * 2, 0, 0);
    return;
  }
  // Groups [g0, g0 + span) hold the batch; this lane's is `go` in.
  constexpr int S = interleave_width<L, BF16, TRITS>();
  const int span = S == 0 || pl.step == 1 ? nv : ((kSlots - 1) * pl.step + 1) * kSlotGroups;
  const int go = S == 0 ? lane : group_offset(lane, pl.step);
  const int64_t g0 = S == 0 ? bt * kWave : pl.first * kSlotGroups;
  const auto dst = make_rsrc(packed + g0 * PB, span * PB);
#pragma unroll
  for (int i = 0; i < PB / 16; ++i) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = {words[4 * i], words[4 * i + 1], words[4 * i + 2], words[4 * i + 3]};
    __builtin_amdgcn_raw_buffer_store_b128(v, dst, go * PB + 16 * i, 0, 0);
  }
  const auto ndst = make_rsrc(norms + g0, span * 2);
  __builtin_amdgcn_raw_buffer_store_b16(n16, ndst, go * 2, 0, 0);
#endif
}

// Fast path: every group is 128 contiguous elements (cols % 128 == 0).
//
// Per iteration a wave reads its 64 groups out of LDS, stores the results of
// its previous batch, issues the DMA of its next batch into the same buffer,
// and computes.  The compiler waits for the direct-to-LDS loads (with a full
// vmcnt(0)) right before the next LDS reads; deferring the stores by one
// iteration means that wait finds only long-finished stores in flight.
//
// Work is handed out by xcd_block's number: the 8 blocks of a 32-batch
// super-batch then share an L2, and so do the 16 waves that write the
// pieces of one 128-byte line of norms (8 bytes each, see store_batch): the
// pieces merge in that L2 instead of reaching HBM as partial lines from up
// to four L2s.  On the 7B-shaped bf16 model the norm stores alone had cost
// 4-5% of quantize's time (2.71 -> 2.61 ms without them, a timing-only
// build); the renumbering took it from 2.73 to 2.66 ms at four batches per
// wave, and to 2.47 ms with one batch per wave (quant_batches_per_wave).
// Storing each slot's four norms as one 8-byte piece (lane 4j after two DPP
// exchanges) measured 2.52 ms there, so the norms keep their 2-byte stores.
//
// One launch covers either one tensor (MANY = false: job.w, job.packed,
// job.norms, job.n_groups) or a table of tensors whose column counts are
// multiples of 128 (MANY = true: job.t, with the batches of each tensor
// numbered consecutively; a tensor's last batch may be partial).
struct QuantJob {
  const uint8_t* w;
  uint8_t* packed;
  uint16_t* norms;
  int64_t n_groups;
  TensorTable<QuantDesc> t;
  int64_t n_batches;
};

// Input and outputs of one 64-group batch: local batch bt of a tensor with
// n_groups groups.
struct QBatch {
  const uint8_t* w;
  uint8_t* packed;
  uint16_t* norms;
  int64_t bt;
  int64_t n_groups;
};

// Batch b of the launch.  d carries the tensor index of the wave's previous
// batch (batches only increase, so the search starts there).
template <bool MANY>
__device__ __forceinline__ QBatch resolve(const QuantJob& j, int64_t b, int& d) {
  if constexpr (!MANY) {
    return QBatch{j.w, j.packed, j.norms, b, j.n_groups};
  } else {
    d = find_unit(j.t.start, d, j.t.n, b);
    // Field by field: each is then a scalar load (an aggregate copy is not).
    const QuantDesc* q = j.t.desc + d;
    return QBatch{load_const(&q->w), load_const(&q->packed), load_const(&q->norms),
                  b - load_const(j.t.start + d), load_const(&q->rows) * (load_const(&q->cols) / kGroup)};
  }
}

// Resident blocks per CU: two for bf16 input (64 KiB of LDS each), one for
// float32 input (128 KiB).
constexpr int blocks_per_cu(bool bf16_in) { return bf16_in ? kBlocksPerCu : 1; }

// Waves per block of the contiguous kernels (7B-shaped model, ms at 4 / 2 /
// 1 waves per block): quantize from bf16 2.69 / 2.76 / 2.82, from float32
// 5.15 / 4.98 / 5.35; fake quant bf16 -> bf16 5.21 / 5.10 / 4.93.
constexpr int quant_waves(bool bf16_in) { return bf16_in ? kWaves : kWaves / 2; }
constexpr int fake_waves() { return 1; }
// The smallest grid a mid-size tensor gets, in blocks of w waves: as many
// waves per CU as blocks_per_cu blocks of kWaves waves.
constexpr int floor_blocks_per_cu(bool bf16_in, int w) { return blocks_per_cu(bf16_in) * kWaves / w; }

// Batches per wave of the grid (each wave strides by the grid).  A grid of a
// few batches per wave measured 4-7% faster on the 7B-shaped model than a
// resident grid of blocks_per_cu blocks per CU that loops over all batches.
// With the block sizes above (ms at 1 / 2 / 4 / 8 batches per wave), without
// the XCD block order (xcd_block): quantize from bf16 2.76 / 2.72 / 2.70 /
// 2.74, from float32 4.78 / 4.84 / 4.96 / 5.23; fake quant bf16 -> bf16
// 4.88 / 4.75 / 4.93 / 5.06.  With it, quantize from bf16 at 1 / 2 / 3 / 4 /
// 8 batches per wave took 2.47 / 2.53 / 2.59 / 2.66 / 2.77 ms (one box, one
// process; 2-wave blocks at one batch per wave 2.49), so bf16 takes a
// covering grid.  Smaller tensors get at least the resident grid's waves
// (spread_blocks).
constexpr int quant_batches_per_wave(bool) { return 1; }
// The multi-tensor launch resolves each batch's tensor by a binary search
// that starts from the wave's previous tensor, so a wave's later batches
// find theirs in a step or two.  The 7B-shaped model as 225 tensors in one
// call (ms per call at 1 / 2 / 4 batches per wave, one box): 2.66 / 2.53 /
// 2.63-2.65.  The XCD block order did not move dequantize or fake quant
// beyond the run-to-run spread (about 1%), so they keep plain numbering.
constexpr int kManyBatchesPerWave = 2;
constexpr int fake_batches_per_wave() { return 2; }

template <int L, bool BF16, bool MANY, bool TRITS = false>
__global__ void __launch_bounds__(quant_waves(BF16) * kWave, blocks_per_cu(BF16))
quantize_contig(QuantJob job, QuantParams p) {
  constexpr int W = quant_waves(BF16);
  constexpr int GB = BF16 ? 256 : 512;  // input bytes per group
  constexpr int CPG = GB / 16;          // 16-byte chunks per group
  constexpr int WAVE_BYTES = kWave * GB;
  constexpr int NI = WAVE_BYTES / 1024;  // 1 KiB load instructions per batch
  __shared__ __attribute__((aligned(16))) uint8_t lds[W * WAVE_BYTES];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  // Blocks have 1 to W waves (quant_grid).
  const int waves = __builtin_amdgcn_readfirstlane(blockDim.x / kWave);
  uint8_t* const buf = lds + wave * WAVE_BYTES;
  const int64_t n_batches = job.n_batches;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * waves;
  int64_t batch = static_cast<int64_t>(xcd_block(blockIdx.x, gridDim.x)) * waves + wave;
  if (batch >= n_batches) return;
  int d = 0;

  // Load instruction i, lane l fills LDS slot 64 i + l (16 bytes each): group
  // gs = GPI*i + q with q = l / CPG, physical chunk cl = l % CPG, which holds
  // logical chunk cl ^ (gs & 15).  Since q < GPI and GPI*i is a multiple of
  // GPI, cl ^ (gs & 15) = (cl ^ q) ^ ((GPI*i) & 15), so the source offset is
  // 1024*i plus a lane part that repeats every R = 16/GPI instructions.
  constexpr int GPI = kWave / CPG;  // groups per load instruction
  constexpr int R = 16 / GPI;
  uint32_t lane_part[R];
  {
    const int q = lane / CPG, cl = lane % CPG;
#pragma unroll
    for (int r = 0; r < R; ++r)
      lane_part[r] = static_cast<uint32_t>(q * GB + 16 * ((cl ^ q) ^ ((GPI * r) & 15)));
  }



  // This lane's group occupies bytes [lane*GB, lane*GB + GB) of the buffer;
  // logical chunk c sits at (lane*GB + 16*(lane & 15)) ^ (16*c).
  const uint32_t rd_base = static_cast<uint32_t>(lane * GB + 16 * (lane & 15));



  uint32_t words[Shape<L>::words];
  uint16_t n16 = 0;
  bool have_prev = false;  // results of batch `prev` are waiting in words / n16
  QBatch cur = resolve<MANY>(job, batch, d), prev = cur;
  constexpr int S = interleave_width<L, BF16, TRITS>();
  issue_batch<S, GB, NI, R>(cur.w, cur.bt, cur.n_groups, buf, lane_part);
  for (;;) {
    uint32_t raw[GB / 4];
#pragma unroll
    for (int c = 0; c < CPG; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(buf + (rd_base ^ (16u * c)));
      raw[4 * c] = v.x;
      raw[4 * c + 1] = v.y;
      raw[4 * c + 2] = v.z;
      raw[4 * c + 3] = v.w;
    }
    wait_lgkm0();  // the buffer is free once every lane has its group
    // Keep the deferred stores (and the next DMA) after the LDS reads, i.e.
    // after the loop-head wait, instead of letting them float above it.
    asm volatile("" ::: "memory");
    if (have_prev) store_batch<L, BF16, TRITS>(prev.packed, prev.norms, prev.bt, prev.n_groups, lane, words, n16);
    const int64_t next = batch + stride;
    QBatch nxt = cur;
    if (next < n_batches) {
      nxt = resolve<MANY>(job, next, d);
      issue_batch<S, GB, NI, R>(nxt.w, nxt.bt, nxt.n_groups, buf, lane_part);
    }

    float y[kGroup];
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 64; i += 4) {
        stage1_bf16(raw[i], y[2 * i], y[2 * i + 1], s0);
        stage1_bf16(raw[i + 1], y[2 * i + 2], y[2 * i + 3], s1);
        stage1_bf16(raw[i + 2], y[2 * i + 4], y[2 * i + 5], s2);
        stage1_bf16(raw[i + 3], y[2 * i + 6], y[2 * i + 7], s3);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 128; i += 4) {
        const float a0 = __builtin_bit_cast(float, raw[i]), b0 = __builtin_bit_cast(float, raw[i + 1]);
        const float a1 = __builtin_bit_cast(float, raw[i + 2]), b1 = __builtin_bit_cast(float, raw[i + 3]);
        y[i] = a0 + b0;
        y[i + 1] = a0 - b0;
        y[i + 2] = a1 + b1;
        y[i + 3] = a1 - b1;
        s0 = __builtin_fmaf(a0, a0, s0);
        s1 = __builtin_fmaf(b0, b0, s1);
        s2 = __builtin_fmaf(a1, a1, s2);
        s3 = __builtin_fmaf(b1, b1, s3);
      }
    }
    n16 = finish_group<L>(y, (s0 + s1) + (s2 + s3), p, words);
    prev = cur;
    have_prev = true;
    cur = nxt;
    batch = next;
    if (batch >= n_batches) break;
  }
  store_batch<L, BF16, TRITS>(prev.packed, prev.norms, prev.bt, prev.n_groups, lane, words, n16);
}

// Decisions and packed fields of a lane's 32 elements (ragged kernels):
// y holds the lane's butterfly outputs, ns the decision scale.  The lane's
// elements 32q .. 32q+31 fill a contiguous quarter of the group's packed
// bits, Shape<L>::sbits dwords, in the same LSB-first order as finish_group.
template <int L>
__device__ __forceinline__ void decide_quarter(const float (&y)[kQuadElems], float ns, const QuantParams& p,
                                               uint32_t (&words)[Shape<L>::sbits]) {
  if constexpr (L == 3 || L == 4) {
    if (p.sym) {
      const float k = p.neg2_over_delta / ns;
#pragma unroll
      for (int wd = 0; wd < 2; ++wd) {
        uint32_t acc = 0;
#pragma unroll
        for (int pos = 15; pos >= 0; --pos) acc = shift_in_pair(acc, y[16 * wd + pos], k);
        words[wd] = finish_sym_word<L>(acc);
      }
      return;
    }
    const float A = p.hmid * ns, D = p.delta * ns;
#pragma unroll
    for (int wd = 0; wd < 2; ++wd) {
      uint32_t acc = 0;
#pragma unroll
      for (int pos = 15; pos >= 0; --pos) {
        const float v = y[16 * wd + pos];
        acc = shift_in_gt(acc, v, A);
        acc = shift_in_gt(acc, __builtin_fabsf(v), D);
      }
      if constexpr (L == 4)
        acc ^= ((acc >> 1) & 0x55555555u) ^ 0x55555555u;
      else
        acc ^= 0x55555555u;
      words[wd] = acc;
    }
  } else if constexpr (L == 8) {
    float T[kMaxLevels - 1];
#pragma unroll
    for (int i = 0; i < 7; ++i) T[i] = p.thr[i] * ns;
#pragma unroll
    for (int i = 0; i < 3; ++i) words[i] = 0;
#pragma unroll
    for (int j = 0; j < kQuadElems; ++j) {
      const uint32_t idx = search8(y[j], T);
      const int pos = 3 * j, wd = pos >> 5, off = pos & 31;
      words[wd] |= idx << off;
      if (off > 29) words[wd + 1] |= idx >> (32 - off);
    }
  } else {
    float T[kMaxLevels - 1];
#pragma unroll
    for (int i = 0; i < 15; ++i) T[i] = p.thr[i] * ns;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      uint32_t acc = 0;
#pragma unroll
      for (int pos = 7; pos >= 0; --pos) {
        bool b3, b2, b1, b0;
        search16(y[8 * wd + pos], T, b3, b2, b1, b0);
        acc = shift_in(acc, b3);
        acc = shift_in(acc, b2);
        acc = shift_in(acc, b1);
        acc = shift_in(acc, b0);
      }
      words[wd] = acc;
    }
  }
}

// Front half of a ragged-path group in quad form: load the lane's 32
// elements, stage 1 and the quad's sum of squares, the two-compare shift
// (lane 0 holds the group's first pair), stages 2..7.  Returns the group
// norm; *ns is the decision scale, as in forward_group.
template <int L, bool BF16, bool WIDE>
__device__ __forceinline__ float quad_forward(const uint8_t* __restrict__ w, const QuadPlace& pl, int q,
                                              const QuantParams& p, float (&y)[kQuadElems], float* ns_out) {
  float x[kQuadElems];
  quad_load<BF16, WIDE>(w, pl.first, pl.valid, q, x);
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int i = 0; i < kQuadElems; i += 2) {
    y[i] = x[i] + x[i + 1];
    y[i + 1] = x[i] - x[i + 1];
    s0 = __builtin_fmaf(x[i], x[i], s0);
    s1 = __builtin_fmaf(x[i + 1], x[i + 1], s1);
  }
  const float S = quad_sum(s0 + s1);
  const float n = __builtin_sqrtf(S);
  const float ns = S > 0.0f ? n : 1.0f;
  if constexpr (L == 3 || L == 4) {
    const float sh = q == 0 ? p.mu * ns : 0.0f;
    y[0] -= sh;
    y[1] -= sh;
  }
  quad_butterfly_in_lane<2>(y);
  quad_butterfly_across<1>(y, q);
  quad_butterfly_across<2>(y, q);
  *ns_out = ns;
  return n;
}

// Unit u of a ragged launch: its group within its tensor and that tensor's
// pointers and width.  With MANY, u indexes the concatenation of the
// table's tensors (t.start holds group prefixes); without, the plain
// arguments describe the one tensor.
template <bool MANY>
__device__ __forceinline__ void ragged_unit(const TensorTable<QuantDesc>& t, int64_t u, const uint8_t*& w,
                                            uint8_t*& packed, uint16_t*& norms, int64_t& cols, int64_t& gl) {
  gl = u;
  if constexpr (MANY) {
    const int d = find_unit(t.start, 0, t.n, u);
    const QuantDesc* qd = t.desc + d;
    w = load_const(&qd->w);
    packed = load_const(&qd->packed);
    norms = load_const(&qd->norms);
    cols = load_const(&qd->cols);
    gl = u - load_const(t.start + d);
  }
}

// General path: rows whose length is not a multiple of 128; the last group
// of each row is zero-padded.  A quad of lanes takes one group (quad form
// of the transform, see quad_load and quad_butterfly_across); each lane
// decides and packs its own 32 elements and stores its quarter of the
// group's packed bytes, lane 0 the norm.  One-wave blocks take 16 groups per
// step of a grid-stride loop (quad_blocks).
template <int L, bool BF16, bool MANY, bool TRITS, bool WIDE>
__global__ void __launch_bounds__(kWave)
quantize_ragged(const uint8_t* __restrict__ w, int64_t rows, int64_t cols, QuantParams p,
                uint8_t* __restrict__ packed, uint16_t* __restrict__ norms,
                TensorTable<QuantDesc> t, int64_t total) {
  constexpr int SW = Shape<L>::sbits;      // packed dwords per lane
  constexpr int PB = Shape<L>::words * 4;  // packed bytes per group
  const int q = threadIdx.x & 3;
  const int64_t n_units = MANY ? total : rows * ((cols + kGroup - 1) / kGroup);
  const int64_t n_steps = (n_units + kQuadGroups - 1) / kQuadGroups;
  for (int64_t s = blockIdx.x; s < n_steps; s += gridDim.x) {
    int64_t u = s * kQuadGroups + (threadIdx.x >> 2);
    const bool live = u < n_units;
    if (!live) u = n_units - 1;  // the quad computes on a real group and stores nothing
    const uint8_t* src = w;
    uint8_t* pk = packed;
    uint16_t* nm = norms;
    int64_t c = cols, gl;
    ragged_unit<MANY>(t, u, src, pk, nm, c, gl);
    const QuadPlace pl = quad_place(gl, c);
    float y[kQuadElems], ns;
    const float n = quad_forward<L, BF16, WIDE>(src, pl, q, p, y, &ns);
    uint32_t words[SW];
    decide_quarter<L>(y, ns, p, words);
    const uint16_t n16 = __builtin_bit_cast(uint16_t, static_cast<_Float16>(n));
    if constexpr (TRITS) {
      // The quad's eight field dwords, then trit bytes; lane q writes the
      // byte pairs k = q, q + 4, ... (13 pairs, 26 bytes, 2-byte aligned).
      uint32_t all[8] = {quad_bcast<0>(words[0]), quad_bcast<0>(words[1]), quad_bcast<1>(words[0]),
                         quad_bcast<1>(words[1]), quad_bcast<2>(words[0]), quad_bcast<2>(words[1]),
                         quad_bcast<3>(words[0]), quad_bcast<3>(words[1])};
      uint32_t tr[13];
      fields_to_trits(all, tr);
      uint16_t* dst = reinterpret_cast<uint16_t*>(pk + gl * kTritBytes);
#pragma unroll
      for (int k = 0; k < 13; ++k)
        if (live && (k & 3) == q) dst[k] = static_cast<uint16_t>(tr[k]);
    } else if (live) {
      uint8_t* dst = pk + gl * PB + q * (4 * SW);
      if constexpr (SW == 2) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
      } else if constexpr (SW == 4) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
      } else {
#pragma unroll
        for (int i = 0; i < SW; ++i) reinterpret_cast<uint32_t*>(dst)[i] = words[i];
      }
    }
    if (live && q == 0) nm[gl] = n16;
  }
}

// ---------------------------------------------------------------------------
// Fused fake quantization: quantize, then reconstruct with the unrounded
// float32 norm, with no packed intermediate (the pages' quantizer returns the
// reconstructed tensor: "Cactus Quants CQ2-bit Quantization: Extreme
// Compression for Edge LLMs", section The CQ2-bit Implementation Pipeline;
// it is the forward of the straight-through estimator, section Training with
// Quantization).
// x_hat = (n / G) * H levels[idx]  (n unrounded; 1/G = 2^-7 is exact).
// ---------------------------------------------------------------------------

// y[j] <- level of element j's decision (N(0,1) units), in place.
template <int L>
__device__ __forceinline__ void levels_in_place(float (&y)[kGroup], float ns, const QuantParams& p,
                                                const LevelTable& lv, const float* lut) {
  if constexpr (L == 3 || L == 4) {
    const float A = p.hmid * ns, D = p.delta * ns;
    // Four levels: index = 2h + NOT(q XOR h); three levels: 2h + NOT q.
    const float lo = lv.c[0], mid = lv.c[1], hi = lv.c[L - 1], mid2 = lv.c[L == 4 ? 2 : 1];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const float v = y[j];
      const bool h = v > A, q = __builtin_fabsf(v) > D;
      y[j] = q ? (h ? hi : lo) : (h ? mid2 : mid);
    }
  } else if constexpr (L == 8) {
    float T[kMaxLevels - 1];
#pragma unroll
    for (int i = 0; i < 7; ++i) T[i] = p.thr[i] * ns;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) y[j] = lut[search8(y[j], T)];
  } else {
    float T[kMaxLevels - 1];
#pragma unroll
    for (int i = 0; i < 15; ++i) T[i] = p.thr[i] * ns;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      bool b3, b2, b1, b0;
      search16(y[j], T, b3, b2, b1, b0);
      y[j] = lut[(bit(b3) << 3) | (bit(b2) << 2) | (bit(b1) << 1) | bit(b0)];
    }
  }
}

__device__ __forceinline__ void butterfly_all(float (&y)[kGroup]) {
#pragma unroll
  for (int i = 0; i < kGroup; i += 2) {
    const float a = y[i], b = y[i + 1];
    y[i] = a + b;
    y[i + 1] = a - b;
  }
  butterfly_from_stage2(y);
}

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void store16(const uint4& v, __amdgpu_buffer_rsrc_t dst, uint32_t voff,
                                        uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)  // buffer builtins exist only for the GPU target
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, dst, voff, soff, 0);
#endif
}

// Stage 1 and the sum of squares from the raw words of one group.
template <bool BF16>
__device__ __forceinline__ float stage1_group(const uint32_t (&raw)[BF16 ? 64 : 128], float (&y)[kGroup]) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
  if constexpr (BF16) {
#pragma unroll
    for (int i = 0; i < 64; i += 4) {
      stage1_bf16(raw[i], y[2 * i], y[2 * i + 1], s0);
      stage1_bf16(raw[i + 1], y[2 * i + 2], y[2 * i + 3], s1);
      stage1_bf16(raw[i + 2], y[2 * i + 4], y[2 * i + 5], s2);
      stage1_bf16(raw[i + 3], y[2 * i + 6], y[2 * i + 7], s3);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 128; i += 4) {
      const float a0 = __builtin_bit_cast(float, raw[i]), b0 = __builtin_bit_cast(float, raw[i + 1]);
      const float a1 = __builtin_bit_cast(float, raw[i + 2]), b1 = __builtin_bit_cast(float, raw[i + 3]);
      y[i] = a0 + b0;
      y[i + 1] = a0 - b0;
      y[i + 2] = a1 + b1;
      y[i + 3] = a1 - b1;
      s0 = __builtin_fmaf(a0, a0, s0);
      s1 = __builtin_fmaf(b0, b0, s1);
      s2 = __builtin_fmaf(a1, a1, s2);
      s3 = __builtin_fmaf(b1, b1, s3);
    }
  }
  return (s0 + s1) + (s2 + s3);
}

// Fast path (cols % 128 == 0).  Input as in quantize_contig (DMA into a
// wave-private LDS buffer, next batch issued right after the current one is
// read out); the reconstructed groups leave through a second, smaller LDS
// buffer in phases of 32 bytes per group so that consecutive lanes store
// consecutive bytes.
template <int L, bool BF16IN, bool BF16OUT>
__global__ void __launch_bounds__(fake_waves() * kWave, blocks_per_cu(BF16IN))
fakequant_contig(const uint8_t* __restrict__ w, int64_t n_groups, QuantParams p, LevelTable lv,
                 uint8_t* __restrict__ out) {
  constexpr int W = fake_waves();
  constexpr int GB = BF16IN ? 256 : 512;  // input bytes per group
  constexpr int CPG = GB / 16;
  constexpr int WAVE_BYTES = kWave * GB;
  constexpr int NI = WAVE_BYTES / 1024;
  constexpr int OB = BF16OUT ? 2 : 4;     // output bytes per element
  constexpr int GOB = kGroup * OB;        // output bytes per group
  // Bytes per group per phase: 64 (half a 128-byte line per piece) where
  // the LDS allows it, else 32 (8 and 16 levels with bf16 input keep their
  // 64-byte level table and stay within two blocks per CU).
  constexpr int PB = (L <= 4 || !BF16IN) ? 64 : 32;
  constexpr int PE = PB / OB;             // elements per group per phase
  constexpr int CPP = PB / 16;            // 16-byte chunks per group per phase
  constexpr int GPB = 256 / PB;           // groups per 256-byte LDS row
  constexpr int GPO = kWave / CPP;        // groups per store instruction
  constexpr int OWB = kWave * PB;         // output staging bytes per wave
  constexpr int NIO = OWB / 1024;         // store instructions per phase
  __shared__ __attribute__((aligned(16))) uint8_t lds[W * WAVE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t olds[W * OWB];
  float* lut = nullptr;  // level table for the 8- and 16-level searches only
  if constexpr (L >= 8) {
    __shared__ float lut_s[kMaxLevels];
    if (threadIdx.x < kMaxLevels) {
      const float v = level_at(lv, threadIdx.x);
      lut_s[threadIdx.x] = v;
      wait_lds_writes();  // the value keeps its register until stored
      hold_values(v);
    }
    lut = lut_s;
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  uint8_t* const buf = lds + wave * WAVE_BYTES;
  uint8_t* const obuf = olds + wave * OWB;
  const int64_t n_batches = (n_groups + kWave - 1) / kWave;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * W;
  int64_t batch = static_cast<int64_t>(blockIdx.x) * W + wave;
  if (batch >= n_batches) return;

  constexpr int GPI = kWave / CPG;
  constexpr int R = 16 / GPI;
  uint32_t lane_part[R];
  {
    const int q = lane / CPG, cl = lane % CPG;
#pragma unroll
    for (int r = 0; r < R; ++r)
      lane_part[r] = static_cast<uint32_t>(q * GB + 16 * ((cl ^ q) ^ ((GPI * r) & 15)));
  }
  const uint32_t rd_base = static_cast<uint32_t>(lane * GB + 16 * (lane & 15));
  const int swz_w = (lane / GPB) & (CPP - 1);
  const int gq = lane / CPP, cc = lane % CPP;
  const uint32_t st_lane = static_cast<uint32_t>(gq * GOB + 16 * cc);

  issue_batch<0, GB, NI, R>(w, batch, n_groups, buf, lane_part);
  for (;;) {
    uint32_t raw[GB / 4];
#pragma unroll
    for (int c = 0; c < CPG; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(buf + (rd_base ^ (16u * c)));
      raw[4 * c] = v.x;
      raw[4 * c + 1] = v.y;
      raw[4 * c + 2] = v.z;
      raw[4 * c + 3] = v.w;
    }
    wait_lgkm0();
    asm volatile("" ::: "memory");
    const int64_t next = batch + stride;
    if (next < n_batches) issue_batch<0, GB, NI, R>(w, next, n_groups, buf, lane_part);

    float y[kGroup];
    const float S = stage1_group<BF16IN>(raw, y);
    float ns;
    const float n = forward_group<L>(y, S, p, &ns);
    levels_in_place<L>(y, ns, p, lv, lut);
    butterfly_all(y);
    const float sc = n * (1.0f / kGroup);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) y[j] *= sc;

    const auto dst = make_rsrc(out + batch * kWave * GOB, valid_in_batch(batch, n_groups) * GOB);
#pragma unroll
    for (int ph = 0; ph < kGroup / PE; ++ph) {
      uint4 ch[CPP];
#pragma unroll
      for (int c = 0; c < CPP; ++c) {
        if constexpr (BF16OUT) {
          const int e = PE * ph + 8 * c;
          ch[c].x = f32_to_bf16_rne(y[e]) | (f32_to_bf16_rne(y[e + 1]) << 16);
          ch[c].y = f32_to_bf16_rne(y[e + 2]) | (f32_to_bf16_rne(y[e + 3]) << 16);
          ch[c].z = f32_to_bf16_rne(y[e + 4]) | (f32_to_bf16_rne(y[e + 5]) << 16);
          ch[c].w = f32_to_bf16_rne(y[e + 6]) | (f32_to_bf16_rne(y[e + 7]) << 16);
        } else {
          const int e = PE * ph + 4 * c;
          ch[c] = make_uint4(__builtin_bit_cast(uint32_t, y[e]), __builtin_bit_cast(uint32_t, y[e + 1]),
                             __builtin_bit_cast(uint32_t, y[e + 2]), __builtin_bit_cast(uint32_t, y[e + 3]));
        }
      }
#pragma unroll
      for (int c = 0; c < CPP; ++c) *reinterpret_cast<uint4*>(obuf + lane * PB + 16 * (c ^ swz_w)) = ch[c];
#pragma unroll
      for (int i = 0; i < NIO; ++i) {
        const int gs = GPO * i + gq;
        const int sw = (gs / GPB) & (CPP - 1);
        const uint4 v = *reinterpret_cast<const uint4*>(obuf + gs * PB + 16 * (cc ^ sw));
        store16(v, dst, st_lane + ph * PB, static_cast<uint32_t>(GPO * i * GOB));
      }
      // After the gather reads (which complete after the writes), so the wait
      // adds nothing to the phase.
      hold_until_lds_written(ch);
    }
    batch = next;
    if (batch >= n_batches) break;
  }
}

// Levels of a lane's 32 decisions, in place (ragged fake quant; the same
// decisions as decide_quarter).
template <int L>
__device__ __forceinline__ void levels_quarter(float (&y)[kQuadElems], float ns, const QuantParams& p,
                                               const LevelTable& lv, const float* lut) {
  if constexpr (L == 3 || L == 4) {
    const float A = p.hmid * ns, D = p.delta * ns;
    const float lo = lv.c[0], mid = lv.c[1], hi = lv.c[L - 1], mid2 = lv.c[L == 4 ? 2 : 1];
#pragma unroll
    for (int j = 0; j < kQuadElems; ++j) {
      const float v = y[j];
      const bool h = v > A, q = __builtin_fabsf(v) > D;
      y[j] = q ? (h ? hi : lo) : (h ? mid2 : mid);
    }
  } else if constexpr (L == 8) {
    float T[kMaxLevels - 1];
#pragma unroll
    for (int i = 0; i < 7; ++i) T[i] = p.thr[i] * ns;
#pragma unroll
    for (int j = 0; j < kQuadElems; ++j) y[j] = lut[search8(y[j], T)];
  } else {
    float T[kMaxLevels - 1];
#pragma unroll
    for (int i = 0; i < 15; ++i) T[i] = p.thr[i] * ns;
#pragma unroll
    for (int j = 0; j < kQuadElems; ++j) {
      bool b3, b2, b1, b0;
      search16(y[j], T, b3, b2, b1, b0);
      y[j] = lut[(bit(b3) << 3) | (bit(b2) << 2) | (bit(b1) << 1) | bit(b0)];
    }
  }
}

// General path: rows of any length, in quad form (see quantize_ragged): the
// quad's forward transform, each lane's levels, the 7-stage transform back,
// the unrounded norm / 128, and each lane writes its existing elements.
template <int L, bool BF16IN, bool BF16OUT, bool WIDE>
__global__ void __launch_bounds__(kWave)
fakequant_ragged(const uint8_t* __restrict__ w, int64_t rows, int64_t cols, QuantParams p,
                 LevelTable lv, uint8_t* __restrict__ out) {
  __shared__ float lut[kMaxLevels];
  if (threadIdx.x < kMaxLevels) {
    const float v = level_at(lv, threadIdx.x);
    lut[threadIdx.x] = v;
    wait_lds_writes();  // the value keeps its register until stored
    hold_values(v);
  }
  __syncthreads();
  const int q = threadIdx.x & 3;
  const int64_t n_units = rows * ((cols + kGroup - 1) / kGroup);
  const int64_t n_steps = (n_units + kQuadGroups - 1) / kQuadGroups;
  for (int64_t s = blockIdx.x; s < n_steps; s += gridDim.x) {
    int64_t u = s * kQuadGroups + (threadIdx.x >> 2);
    const bool live = u < n_units;
    if (!live) u = n_units - 1;
    const QuadPlace pl = quad_place(u, cols);
    float y[kQuadElems], ns;
    const float n = quad_forward<L, BF16IN, WIDE>(w, pl, q, p, y, &ns);
    levels_quarter<L>(y, ns, p, lv, lut);
    quad_butterfly_in_lane<1>(y);
    quad_butterfly_across<1>(y, q);
    quad_butterfly_across<2>(y, q);
    const float sc = n * (1.0f / kGroup);
#pragma unroll
    for (int j = 0; j < kQuadElems; ++j) y[j] *= sc;
    if (live) quad_store<BF16OUT, WIDE>(out, pl.first, pl.valid, q, y);
  }
}

template <int L, bool BF16IN, bool BF16OUT>
hipError_t launch_fq(const void* w, int64_t rows, int64_t cols, const QuantParams& p,
                     const LevelTable& lv, void* out, hipStream_t s) {
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  uint8_t* ob = static_cast<uint8_t*>(out);
  if (cols % kGroup == 0) {
    const int64_t n_groups = rows * (cols / kGroup);
    const int64_t n_batches = (n_groups + kWave - 1) / kWave;
    constexpr int W = fake_waves();
    const int blocks = spread_blocks(n_batches, W, fake_batches_per_wave(), floor_blocks_per_cu(BF16IN, W));
    hipLaunchKernelGGL((fakequant_contig<L, BF16IN, BF16OUT>), dim3(blocks), dim3(W * kWave), 0, s, wb,
                       n_groups, p, lv, ob);
  } else {
    const int blocks = quad_blocks(rows * ((cols + kGroup - 1) / kGroup));
    // 16-byte pieces need whole pieces on both sides (16-byte aligned base
    // pointers are required by the caller).
    if (cols % wide_elems(BF16IN) == 0 && cols % wide_elems(BF16OUT) == 0)
      hipLaunchKernelGGL((fakequant_ragged<L, BF16IN, BF16OUT, true>), dim3(blocks), dim3(kWave), 0, s, wb, rows,
                         cols, p, lv, ob);
    else
      hipLaunchKernelGGL((fakequant_ragged<L, BF16IN, BF16OUT, false>), dim3(blocks), dim3(kWave), 0, s, wb, rows,
                         cols, p, lv, ob);
  }
  return hipGetLastError();
}

template <int L>
hipError_t launch_fq_types(const void* w, bool bf16_in, int64_t rows, int64_t cols,
                           const QuantParams& p, const LevelTable& lv, void* out, bool bf16_out,
                           hipStream_t s) {
  if (bf16_in)
    return bf16_out ? launch_fq<L, true, true>(w, rows, cols, p, lv, out, s)
                    : launch_fq<L, true, false>(w, rows, cols, p, lv, out, s);
  return bf16_out ? launch_fq<L, false, true>(w, rows, cols, p, lv, out, s)
                  : launch_fq<L, false, false>(w, rows, cols, p, lv, out, s);
}

// Grid of the contiguous quantize kernel: a few batches per wave in blocks of
// quant_waves waves; a call with fewer than that many batches per CU takes
// smaller blocks, one batch per wave, so its batches spread over more CUs.
template <bool BF16>
ContigGrid quant_grid(int64_t n_batches, int per_wave = quant_batches_per_wave(BF16)) {
  constexpr int W = quant_waves(BF16);
  return contig_grid(n_batches, W, per_wave, floor_blocks_per_cu(BF16, W));
}

template <int L, bool BF16, bool TRITS>
hipError_t launch_l(const void* w, int64_t rows, int64_t cols, const QuantParams& p,
                    uint8_t* packed, uint16_t* norms, hipStream_t s) {
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  if (cols % kGroup == 0) {
    const int64_t n_groups = rows * (cols / kGroup);
    const int64_t n_batches = (n_groups + kWave - 1) / kWave;
    // Each wave loops over a few batches, so the next batch's DMA overlaps
    // the current arithmetic.
    const ContigGrid g = quant_grid<BF16>(n_batches);
    const QuantJob job{wb, packed, norms, n_groups, TensorTable<QuantDesc>{nullptr, nullptr, 0}, n_batches};
    hipLaunchKernelGGL((quantize_contig<L, BF16, false, TRITS>), dim3(g.blocks), dim3(g.waves * kWave), 0, s, job,
                       p);
  } else {
    const int blocks = quad_blocks(rows * ((cols + kGroup - 1) / kGroup));
    const TensorTable<QuantDesc> none{nullptr, nullptr, 0};
    if (cols % wide_elems(BF16) == 0)
      hipLaunchKernelGGL((quantize_ragged<L, BF16, false, TRITS, true>), dim3(blocks), dim3(kWave), 0, s, wb,
                         rows, cols, p, packed, norms, none, int64_t{0});
    else
      hipLaunchKernelGGL((quantize_ragged<L, BF16, false, TRITS, false>), dim3(blocks), dim3(kWave), 0, s, wb,
                         rows, cols, p, packed, norms, none, int64_t{0});
  }
  return hipGetLastError();
}

template <int L, bool BF16, bool TRITS>
hipError_t launch_many_l(const QuantParams& p, TensorTable<QuantDesc> contig, int64_t contig_batches,
                         TensorTable<QuantDesc> ragged, int64_t ragged_groups, int64_t ragged_cols_gcd,
                         hipStream_t s) {
  if (contig_batches > 0) {
    const ContigGrid g = quant_grid<BF16>(contig_batches, kManyBatchesPerWave);
    const QuantJob job{nullptr, nullptr, nullptr, 0, contig, contig_batches};
    hipLaunchKernelGGL((quantize_contig<L, BF16, true, TRITS>), dim3(g.blocks), dim3(g.waves * kWave), 0, s, job,
                       p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (ragged_groups > 0) {
    // The 16-byte form needs every ragged tensor's width to be a multiple
    // of the piece (their gcd is).
    const int blocks = quad_blocks(ragged_groups);
    if (ragged_cols_gcd % wide_elems(BF16) == 0)
      hipLaunchKernelGGL((quantize_ragged<L, BF16, true, TRITS, true>), dim3(blocks), dim3(kWave), 0, s, nullptr,
                         int64_t{0}, int64_t{0}, p, nullptr, nullptr, ragged, ragged_groups);
    else
      hipLaunchKernelGGL((quantize_ragged<L, BF16, true, TRITS, false>), dim3(blocks), dim3(kWave), 0, s,
                         nullptr, int64_t{0}, int64_t{0}, p, nullptr, nullptr, ragged, ragged_groups);
  }
  return hipGetLastError();
}

// Trit storage exists for the three-level code only.
template <int L>
hipError_t launch_many_dtype(bool bf16, bool trits, const QuantParams& p, TensorTable<QuantDesc> contig,
                             int64_t contig_batches, TensorTable<QuantDesc> ragged,
                             int64_t ragged_groups, int64_t ragged_cols_gcd, hipStream_t s) {
  if constexpr (L == 3) {
    if (trits)
      return bf16 ? launch_many_l<L, true, true>(p, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, s)
                  : launch_many_l<L, false, true>(p, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, s);
  }
  if (trits) return hipErrorInvalidValue;
  return bf16 ? launch_many_l<L, true, false>(p, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, s)
              : launch_many_l<L, false, false>(p, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, s);
}

template <int L>
hipError_t launch_dtype(const void* w, bool bf16, bool trits, int64_t rows, int64_t cols,
                        const QuantParams& p, uint8_t* packed, uint16_t* norms, hipStream_t s) {
  if constexpr (L == 3) {
    if (trits)
      return bf16 ? launch_l<L, true, true>(w, rows, cols, p, packed, norms, s)
                  : launch_l<L, false, true>(w, rows, cols, p, packed, norms, s);
  }
  if (trits) return hipErrorInvalidValue;
  return bf16 ? launch_l<L, true, false>(w, rows, cols, p, packed, norms, s)
              : launch_l<L, false, false>(w, rows, cols, p, packed, norms, s);
}

}  // namespace kq

hipError_t launch_fake_quant(const void* w, bool bf16_in, int64_t rows, int64_t cols,
                             const QuantParams& p, const LevelTable& lv, void* out, bool bf16_out,
                             hipStream_t stream) {
  switch (p.n_levels) {
    case 3: return kq::launch_fq_types<3>(w, bf16_in, rows, cols, p, lv, out, bf16_out, stream);
    case 4: return kq::launch_fq_types<4>(w, bf16_in, rows, cols, p, lv, out, bf16_out, stream);
    case 8: return kq::launch_fq_types<8>(w, bf16_in, rows, cols, p, lv, out, bf16_out, stream);
    case 16: return kq::launch_fq_types<16>(w, bf16_in, rows, cols, p, lv, out, bf16_out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize(const void* w, bool bf16, bool trits, int64_t rows, int64_t cols,
                           const QuantParams& p, uint8_t* packed, uint16_t* norms,
                           hipStream_t stream) {
  switch (p.n_levels) {
    case 3: return kq::launch_dtype<3>(w, bf16, trits, rows, cols, p, packed, norms, stream);
    case 4: return kq::launch_dtype<4>(w, bf16, trits, rows, cols, p, packed, norms, stream);
    case 8: return kq::launch_dtype<8>(w, bf16, trits, rows, cols, p, packed, norms, stream);
    case 16: return kq::launch_dtype<16>(w, bf16, trits, rows, cols, p, packed, norms, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize_many(bool bf16, bool trits, const QuantParams& p, TensorTable<QuantDesc> contig,
                                int64_t contig_batches, TensorTable<QuantDesc> ragged,
                                int64_t ragged_groups, int64_t ragged_cols_gcd, hipStream_t stream) {
  switch (p.n_levels) {
    case 3: return kq::launch_many_dtype<3>(bf16, trits, p, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, stream);
    case 4: return kq::launch_many_dtype<4>(bf16, trits, p, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, stream);
    case 8: return kq::launch_many_dtype<8>(bf16, trits, p, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, stream);
    case 16: return kq::launch_many_dtype<16>(bf16, trits, p, contig, contig_batches, ragged, ragged_groups, ragged_cols_gcd, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cq
