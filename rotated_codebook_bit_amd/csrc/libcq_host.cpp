// libcq host side: argument validation, layout and size accounting, the
// Lloyd-Max codebook, per-call constants, and kernel dispatch.
//
// Method sources (web pages, by title and section):
//   "Cactus Quants CQ2-bit Quantization: Extreme Compression for Edge LLMs"
//       - Group-wise Weight Partitioning; The CQ2-bit Implementation Pipeline
//   "How CQ2-bit Quantization Contributes to Needle 2's Small Footprint"
//       - Per-Group Storage Breakdown; Binary Serialization
//   "How Quantization Codebooks Are Trained in Cactus Quants: Lloyd-Max on
//    Gaussian Data"
//       - Gaussian Sampling and Initialization; Iterative Refinement of
//         Quantization Levels; Ternary Special Case Handling

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <numeric>
#include <vector>

#include "../../include/libcq.h"
#include "cq_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Levels of a bit-width; -1 if unsupported.
int levels_for_bits(int bits, bool host_only) {
  if (bits == CQ_TERNARY || bits == CQ_TERNARY_TRITS) return 3;
  if (bits == 2 || bits == 3 || bits == 4) return 1 << bits;
  if (bits == 1 && host_only) return 2;
  return -1;
}

// Bits of one index in the bit-field layouts (the ternary code uses 2-bit
// fields; its trit storage has no fields, see group_bytes).
int storage_bits(int bits) { return (bits == CQ_TERNARY || bits == CQ_TERNARY_TRITS) ? 2 : bits; }

int check_bits(int bits, bool host_only, int* n_levels) {
  int l = levels_for_bits(bits, host_only);
  if (l < 0) return fail(CQ_ERR_ARG, "unsupported bits=%d", bits);
  if (n_levels) *n_levels = l;
  return CQ_OK;
}

int check_group(int group_size, bool device) {
  if (device) {
    if (group_size != cq::kGroup)
      return fail(CQ_ERR_UNSUPPORTED, "group_size=%d: this call supports 128", group_size);
  } else if (!is_pow2(group_size) || group_size < 8 || group_size > 4096) {
    // From 8 up, a group's packed indices fill whole bytes at every width.
    return fail(CQ_ERR_ARG, "group_size=%d must be a power of two in [8, 4096]", group_size);
  }
  return CQ_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  auto x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

const float* builtin_levels(int bits);

// Validates a caller's codebook; NULL selects the built-in table of the
// width (n_levels is then ignored) and `levels` is pointed at it.
int check_levels(const float*& levels, int n_levels, int expect, int bits) {
  if (!levels) {
    levels = builtin_levels(bits);
    return CQ_OK;
  }
  if (n_levels != expect)
    return fail(CQ_ERR_ARG, "n_levels=%d, this bit-width needs %d", n_levels, expect);
  for (int i = 0; i < n_levels; ++i) {
    if (!std::isfinite(levels[i])) return fail(CQ_ERR_ARG, "levels[%d] is not finite", i);
    if (i && !(levels[i] > levels[i - 1]))
      return fail(CQ_ERR_ARG, "levels must be strictly ascending (index %d)", i);
  }
  return CQ_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The codec calls (quantize, dequantize, fake quantization, their
// multi-tensor forms, repacking) run group sizes 32, 64, 128 and 256.
int check_codec_group(int group_size, int bits) {
  (void)bits;
  if (group_size != 32 && group_size != 64 && group_size != cq::kGroup && group_size != 256)
    return fail(CQ_ERR_UNSUPPORTED, "group_size=%d: these kernels support 32, 64, 128 and 256", group_size);
  return CQ_OK;
}

// Packed bytes per group: G * sbits / 8, or ceil(G / 5) for trit storage.
int64_t group_bytes(int bits, int group_size) {
  if (bits == CQ_TERNARY_TRITS) return ceil_div(group_size, 5);
  return static_cast<int64_t>(group_size) * storage_bits(bits) / 8;
}

// Storage code of the dequantize launchers: field width, or trits.
int storage_code(int bits) { return bits == CQ_TERNARY_TRITS ? cq::kTritStorage : storage_bits(bits); }

// Alignment the kernels need for packed indices: 16 bytes for bit fields at
// G = 128 (128-bit accesses), 4 bytes at the other group sizes (32-bit
// accesses; their groups are multiples of 4 bytes, so every offset inside a
// serialized blob qualifies), 2 bytes for trit storage (16-bit accesses; a
// group is 26 bytes, so tensors inside a blob sit at even offsets).
size_t packed_align(int bits, int group_size) {
  if (bits == CQ_TERNARY_TRITS) return group_size == cq::kGroup ? 2 : 1;
  return group_size == cq::kGroup ? 16 : 4;
}

int reject_trits(int bits) {
  if (bits == CQ_TERNARY_TRITS)
    return fail(CQ_ERR_UNSUPPORTED, "trit storage: convert it with cq_repack to CQ_TERNARY first");
  return CQ_OK;
}

// Byte range [lo, hi) of one buffer of a multi-tensor call.
struct Span {
  uintptr_t lo, hi;
  int tensor;
};

Span span(const void* p, size_t bytes, int tensor) {
  const auto a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes, tensor};
}

// Index of a tensor whose buffers conflict (two outputs overlap, or an input
// overlaps an output), or -1.  Inputs may overlap each other.
int first_conflict(std::vector<Span> outs, const std::vector<Span>& ins) {
  std::sort(outs.begin(), outs.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < outs.size(); ++i)
    if (outs[i].lo < outs[i - 1].hi) return outs[i].tensor;
  for (const Span& in : ins) {
    // The last output starting before the input ends is the only candidate:
    // outputs are disjoint and sorted.
    auto it = std::lower_bound(outs.begin(), outs.end(), in.hi,
                               [](const Span& o, uintptr_t v) { return o.lo < v; });
    if (it != outs.begin() && std::prev(it)->hi > in.lo) return in.tensor;
  }
  return -1;
}

int hip_status(hipError_t e, const char* what);

// 1-D Lloyd-Max (k-means) with L levels on sorted samples x, as "How
// Quantization Codebooks Are Trained in Cactus Quants: Lloyd-Max on Gaussian
// Data" describes it (sections Gaussian Sampling and Initialization and
// Iterative Refinement of Quantization Levels): level k starts at the sorted
// sample floor((k + 1/2) n / L); each round puts the boundaries at the
// midpoints of neighbouring levels, gives every sample to the cell whose
// lower boundary it strictly exceeds (a sample equal to a boundary stays in
// the lower cell) and moves each level to the mean of its cell; an empty
// cell keeps its level.  Cells are contiguous runs of the sorted array, so a
// round needs only the L-1 split positions.  Writes the sorted levels as
// float32.
//
// mirrored: the samples are symmetric about 0 (x[n-1-i] = -x[i]).  The
// upper half of the levels then starts at the mirror images of the lower
// half's order statistics (x[n-1-i] rather than the sample at the upper
// quantile's own index, which is one position off the mirror), so every
// round keeps the partition symmetric; the result is symmetrised once more
// to drop differences of summation order.  With the plain start the 2-bit
// levels settle on an asymmetric fixed point (a few samples just above 0
// stay in the lower cell; the inner levels then differ by 8.5e-5).
void lloyd_max_sorted(const std::vector<double>& x, int L, int iters, float* levels_out, bool mirrored) {
  const int64_t n = static_cast<int64_t>(x.size());
  std::vector<double> c(L);
  for (int k = 0; k < L; ++k) c[k] = x[((2 * static_cast<int64_t>(k) + 1) * n) / (2 * L)];
  if (mirrored)
    for (int k = L / 2; k < L; ++k) c[k] = x[n - 1 - ((2 * static_cast<int64_t>(L - 1 - k) + 1) * n) / (2 * L)];
  std::vector<int64_t> start(L + 1);
  for (int it = 0; it < iters; ++it) {
    start[0] = 0;
    start[L] = n;
    for (int k = 1; k < L; ++k) {
      const double edge = 0.5 * (c[k - 1] + c[k]);
      // First sample strictly above the boundary.
      start[k] = std::upper_bound(x.begin(), x.end(), edge) - x.begin();
    }
    for (int k = 0; k < L; ++k) {
      const int64_t lo = start[k], hi = start[k + 1];
      if (hi <= lo) continue;  // empty cell keeps its level
      long double sum = 0.0L;
      for (int64_t i = lo; i < hi; ++i) sum += x[i];
      c[k] = static_cast<double>(sum / static_cast<long double>(hi - lo));
    }
  }
  std::sort(c.begin(), c.end());
  if (mirrored) {
    for (int k = 0; k < L / 2; ++k) {
      const double h = 0.5 * (c[L - 1 - k] - c[k]);
      c[k] = -h;
      c[L - 1 - k] = h;
    }
    if (L % 2) c[L / 2] = 0.0;
  }
  for (int k = 0; k < L; ++k) levels_out[k] = static_cast<float>(c[k]);
}

// ---- Built-in codebook ---------------------------------------------------------
//
// The training recipe of the codebook page (400,000 standard-normal samples,
// quantile initialisation, 200 Lloyd-Max rounds), run once per width on
// samples from this library's own deterministic generator:
//   - uniform 64-bit words from SplitMix64 (G. Steele, D. Lea, C. Flood,
//     "Fast Splittable Pseudorandom Number Generators", OOPSLA 2014) with
//     state 0: the state advances by 0x9E3779B97F4A7C15 and each output is
//     the state mixed by z ^= z >> 30, z *= 0xBF58476D1CE4E5B9,
//     z ^= z >> 27, z *= 0x94D049BB133111EB, z ^= z >> 31;
//   - a uniform double u = ((w >> 11) + 1) * 2^-53 in (0, 1] per word;
//   - normals by the Box-Muller transform of consecutive (u1, u2):
//     sqrt(-2 ln u1) * cos(2 pi u2), then sqrt(-2 ln u1) * sin(2 pi u2);
//   - each normal is used together with its negation (antithetic pairs), so
//     the 400,000 samples are 100,000 Box-Muller pairs and the sample set
//     is symmetric about 0.  Without it a finite sample's Lloyd-Max fixed
//     point shifts with the sample's own asymmetry: the first 400,000
//     normals of this generator put the 2-bit levels 7e-3 off the Gaussian
//     optimum, their symmetrised half within 1.5e-3.
// The ternary width has the fixed table of the page's section Ternary Special
// Case Handling.  The tables are built on first use and never change.
constexpr int64_t kBuiltinSamples = 400000;  // a multiple of 4
constexpr int kBuiltinIters = 200;
const float kTernaryLevels[3] = {-1.2240064f, 0.0f, 1.2240064f};

uint64_t splitmix64(uint64_t& state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

std::vector<double> builtin_samples() {
  std::vector<double> x(kBuiltinSamples);
  uint64_t state = 0;
  const double two_pi = 6.283185307179586476925286766559;
  for (int64_t i = 0; i < kBuiltinSamples; i += 4) {
    const double u1 = static_cast<double>((splitmix64(state) >> 11) + 1) * 0x1.0p-53;
    const double u2 = static_cast<double>((splitmix64(state) >> 11) + 1) * 0x1.0p-53;
    const double r = std::sqrt(-2.0 * std::log(u1));
    const double z0 = r * std::cos(two_pi * u2), z1 = r * std::sin(two_pi * u2);
    x[i] = z0;
    x[i + 1] = -z0;
    x[i + 2] = z1;
    x[i + 3] = -z1;
  }
  std::sort(x.begin(), x.end());
  return x;
}

struct BuiltinTables {
  float lv[5][cq::kMaxLevels];  // index = bits (1..4)
  BuiltinTables() {
    const std::vector<double> x = builtin_samples();
    for (int bits = 1; bits <= 4; ++bits) lloyd_max_sorted(x, 1 << bits, kBuiltinIters, lv[bits], true);
  }
};

const float* builtin_levels(int bits) {
  if (bits == CQ_TERNARY || bits == CQ_TERNARY_TRITS) return kTernaryLevels;
  static const BuiltinTables tables;  // built once, thread-safe (C++11 static init)
  return tables.lv[bits];
}

// Device table of one multi-tensor call: descriptors of the fast-path
// (cols % 128 == 0) and ragged tensors, with their work-unit prefixes, in one
// stream-ordered allocation.
template <class D>
struct ManyTables {
  std::vector<D> contig, ragged;
  std::vector<int64_t> bstart{0}, gstart{0};  // 64-group batches / groups
  int64_t ragged_gcd = 0;                       // gcd of the ragged tensors' column counts
  uint8_t* ws = nullptr;
  cq::TensorTable<D> tc{}, tr{};

  void add(const D& d, int64_t n_groups, bool fast) {
    if (fast) {
      contig.push_back(d);
      bstart.push_back(bstart.back() + ceil_div(n_groups, cq::kWave));
    } else {
      ragged.push_back(d);
      gstart.push_back(gstart.back() + n_groups);
      ragged_gcd = std::gcd(ragged_gcd, d.cols);
    }
  }
  bool empty() const { return contig.empty() && ragged.empty(); }

  // Allocates the workspace on `s` and uploads the tables.
  int upload(hipStream_t s) {
    auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
    const size_t b0 = up(contig.size() * sizeof(D)), b1 = up(bstart.size() * 8);
    const size_t b2 = up(ragged.size() * sizeof(D)), b3 = up(gstart.size() * 8);
    int rc = hip_status(hipMallocAsync(reinterpret_cast<void**>(&ws), b0 + b1 + b2 + b3, s),
                        "table alloc");
    if (rc) return rc;
    auto* dc = reinterpret_cast<D*>(ws);
    auto* sc = reinterpret_cast<int64_t*>(ws + b0);
    auto* dr = reinterpret_cast<D*>(ws + b0 + b1);
    auto* sr = reinterpret_cast<int64_t*>(ws + b0 + b1 + b2);
    tc = cq::TensorTable<D>{dc, sc, static_cast<int>(contig.size())};
    tr = cq::TensorTable<D>{dr, sr, static_cast<int>(ragged.size())};
    if (!contig.empty()) {
      rc = hip_status(cq::upload(contig.data(), contig.size() * sizeof(D), dc, s), "table upload");
      if (!rc) rc = hip_status(cq::upload(bstart.data(), bstart.size() * 8, sc, s), "table upload");
    }
    if (!rc && !ragged.empty()) {
      rc = hip_status(cq::upload(ragged.data(), ragged.size() * sizeof(D), dr, s), "table upload");
      if (!rc) rc = hip_status(cq::upload(gstart.data(), gstart.size() * 8, sr, s), "table upload");
    }
    return rc;
  }
  int release(hipStream_t s) { return ws ? hip_status(hipFreeAsync(ws, s), "table free") : CQ_OK; }
};

// Decision constants for the quantize kernels.  The index of a value z is
// the number of midpoint thresholds strictly below it.  For three and four
// levels the kernels decide with two compares around the centre mu of the
// outer thresholds (half width delta):
//   high bit h = [z - mu > hmid]       (hmid = t_mid - mu; three levels: delta)
//   q          = [|z - mu| > delta]    (outside the outer pair)
//   four levels: low bit = NOT (q XOR h);  three levels: low bit = NOT q.
cq::QuantParams make_quant_params(const float* levels, int n_levels) {
  cq::QuantParams p{};
  p.n_levels = n_levels;
  double t[cq::kMaxLevels - 1];
  for (int i = 0; i + 1 < n_levels; ++i) {
    t[i] = 0.5 * (static_cast<double>(levels[i]) + static_cast<double>(levels[i + 1]));
    p.thr[i] = static_cast<float>(t[i]);
  }
  if (n_levels == 3) {
    double mu = 0.5 * (t[0] + t[1]), d = 0.5 * (t[1] - t[0]);
    p.mu = static_cast<float>(mu);
    p.delta = static_cast<float>(d);
    p.hmid = static_cast<float>(d);
  } else if (n_levels == 4) {
    double mu = 0.5 * (t[0] + t[2]), d = 0.5 * (t[2] - t[0]);
    p.mu = static_cast<float>(mu);
    p.delta = static_cast<float>(d);
    p.hmid = static_cast<float>(t[1] - mu);
  }
  if (n_levels == 3 || (n_levels == 4 && p.hmid == 0.0f)) {
    const float k = static_cast<float>(-2.0 / static_cast<double>(p.delta));
    p.neg2_over_delta = k;
    p.sym = std::isfinite(k) ? 1 : 0;
  }
  return p;
}

// Trit storage at group sizes other than 128: the 2-bit field kernels with a
// stream-ordered workspace of fields (G / 4 bytes per group), converted by
// cq_repack's kernels.
int quantize_trits_g(const void* w, bool bf16, int64_t rows, int64_t cols, int group_size,
                     const cq::QuantParams& p, uint8_t* packed, uint16_t* norms, hipStream_t s) {
  const int64_t ng = rows * ceil_div(cols, group_size);
  uint8_t* ws = nullptr;
  int rc = hip_status(hipMallocAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(ng) * (group_size / 4), s),
                      "workspace alloc");
  if (rc) return rc;
  rc = hip_status(cq::launch_quantize_g(group_size, w, bf16, rows, cols, p, ws, norms, s), "quantize launch");
  if (!rc) rc = hip_status(cq::launch_repack(ws, true, packed, ng, group_size, s), "repack launch");
  const int rc2 = hip_status(hipFreeAsync(ws, s), "workspace free");
  return rc ? rc : rc2;
}

int dequantize_trits_g(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols, int group_size,
                       const cq::LevelTable& lv, void* out, bool bf16_out, hipStream_t s) {
  const int64_t ng = rows * ceil_div(cols, group_size);
  uint8_t* ws = nullptr;
  int rc = hip_status(hipMallocAsync(reinterpret_cast<void**>(&ws), static_cast<size_t>(ng) * (group_size / 4), s),
                      "workspace alloc");
  if (rc) return rc;
  rc = hip_status(cq::launch_repack(packed, false, ws, ng, group_size, s), "repack launch");
  if (!rc)
    rc = hip_status(cq::launch_dequantize_g(group_size, ws, norms, rows, cols, 2, lv, out, bf16_out, s),
                    "dequantize launch");
  const int rc2 = hip_status(hipFreeAsync(ws, s), "workspace free");
  return rc ? rc : rc2;
}


cq::LevelTable make_table(const float* levels, int n_levels) {
  cq::LevelTable t{};
  t.n_levels = n_levels;
  for (int i = 0; i < n_levels; ++i) t.c[i] = levels[i];
  return t;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return CQ_OK;
}

}  // namespace

namespace cq {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace cq

extern "C" {

const char* cq_version(void) { return "libcq 0.1 (gfx950)"; }

const char* cq_last_error(void) { return g_last_error; }

const char* cq_status_str(int status) {
  switch (status) {
    case CQ_OK: return "ok";
    case CQ_ERR_NULL: return "null pointer";
    case CQ_ERR_ARG: return "invalid argument";
    case CQ_ERR_ALIGN: return "misaligned pointer";
    case CQ_ERR_UNSUPPORTED: return "unsupported";
    case CQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int cq_layout(int64_t rows, int64_t cols, int bits, int group_size, int64_t* n_groups,
              int64_t* packed_bytes) {
  g_last_error[0] = 0;
  int rc;
  if ((rc = check_bits(bits, true, nullptr))) return rc;
  if ((rc = check_group(group_size, false))) return rc;
  if (rows < 0 || cols < 0) return fail(CQ_ERR_ARG, "negative size");
  int64_t g = rows * ceil_div(cols, group_size);
  if (n_groups) *n_groups = g;
  if (packed_bytes) *packed_bytes = g * group_bytes(bits, group_size);
  return CQ_OK;
}

int cq_model_bytes(int n_tensors, const int64_t* rows, const int64_t* cols, int bits,
                   int group_size, uint64_t* bytes_out) {
  g_last_error[0] = 0;
  int rc;
  if (!bytes_out) return fail(CQ_ERR_NULL, "bytes_out is NULL");
  if (n_tensors < 0) return fail(CQ_ERR_ARG, "n_tensors < 0");
  if (n_tensors > 0 && (!rows || !cols)) return fail(CQ_ERR_NULL, "rows/cols is NULL");
  if ((rc = check_bits(bits, true, nullptr))) return rc;
  if ((rc = check_group(group_size, false))) return rc;
  const uint64_t per_group = static_cast<uint64_t>(group_bytes(bits, group_size)) + 2;
  uint64_t total = 0;
  for (int i = 0; i < n_tensors; ++i) {
    if (rows[i] < 0 || cols[i] < 0) return fail(CQ_ERR_ARG, "tensor %d has a negative size", i);
    total += static_cast<uint64_t>(rows[i]) * static_cast<uint64_t>(ceil_div(cols[i], group_size)) *
             per_group;
  }
  *bytes_out = total;
  return CQ_OK;
}

int cq_codebook(int bits, float* levels_out, int* n_levels) {
  g_last_error[0] = 0;
  int L, rc;
  if (!levels_out || !n_levels) return fail(CQ_ERR_NULL, "levels_out/n_levels is NULL");
  if ((rc = check_bits(bits, true, &L))) return rc;
  std::memcpy(levels_out, builtin_levels(bits), static_cast<size_t>(L) * sizeof(float));
  *n_levels = L;
  return CQ_OK;
}

int cq_codebook_train(int bits, const double* samples, int64_t n_samples, int iters, float* levels_out,
                      int* n_levels) {
  g_last_error[0] = 0;
  int L, rc;
  if (!levels_out || !n_levels) return fail(CQ_ERR_NULL, "levels_out/n_levels is NULL");
  if ((rc = check_bits(bits, true, &L))) return rc;
  if (bits == CQ_TERNARY || bits == CQ_TERNARY_TRITS) {
    std::memcpy(levels_out, kTernaryLevels, sizeof(kTernaryLevels));
    *n_levels = 3;
    return CQ_OK;
  }
  if (!samples) return fail(CQ_ERR_NULL, "samples is NULL");
  if (n_samples < L) return fail(CQ_ERR_ARG, "need at least %d samples", L);
  if (iters < 0) return fail(CQ_ERR_ARG, "iters < 0");
  for (int64_t i = 0; i < n_samples; ++i)
    if (!std::isfinite(samples[i])) return fail(CQ_ERR_ARG, "sample %lld is not finite", (long long)i);
  std::vector<double> x(samples, samples + n_samples);
  std::sort(x.begin(), x.end());
  lloyd_max_sorted(x, L, iters, levels_out, false);
  *n_levels = L;
  return CQ_OK;
}

int cq_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols, int bits, int group_size,
                const float* levels, int n_levels, uint8_t* packed, uint16_t* norms,
                void* stream) {
  g_last_error[0] = 0;
  int L, rc;
  if ((rc = check_bits(bits, false, &L))) return rc;
  if (w_dtype != CQ_F32 && w_dtype != CQ_BF16) return fail(CQ_ERR_ARG, "unknown w_dtype %d", w_dtype);
  if (rows < 0 || cols < 0) return fail(CQ_ERR_ARG, "negative size");
  if ((rc = check_codec_group(group_size, bits))) return rc;
  if ((rc = check_levels(levels, n_levels, L, bits))) return rc;
  if (rows == 0 || cols == 0) return CQ_OK;
  if (!w || !packed || !norms) return fail(CQ_ERR_NULL, "w/packed/norms is NULL");
  if (!aligned(w, 16) || !aligned(packed, packed_align(bits, group_size)) || !aligned(norms, 2))
    return fail(CQ_ERR_ALIGN, "w needs 16-byte, packed 16-byte (G != 128: 4-byte; trits: 2-byte, any at G != 128), norms 2-byte alignment");
  const int64_t ng = rows * ceil_div(cols, group_size);
  const size_t in_bytes = static_cast<size_t>(rows * cols) * (w_dtype == CQ_F32 ? 4 : 2);
  const size_t pk_bytes = static_cast<size_t>(ng * group_bytes(bits, group_size));
  const size_t nm_bytes = static_cast<size_t>(ng) * 2;
  if (overlap(w, in_bytes, packed, pk_bytes) || overlap(w, in_bytes, norms, nm_bytes) ||
      overlap(packed, pk_bytes, norms, nm_bytes))
    return fail(CQ_ERR_ARG, "input and output buffers overlap");
  const cq::QuantParams p = make_quant_params(levels, L);
  if (group_size != cq::kGroup && bits == CQ_TERNARY_TRITS)
    return quantize_trits_g(w, w_dtype == CQ_BF16, rows, cols, group_size, p, packed, norms,
                            static_cast<hipStream_t>(stream));
  if (group_size != cq::kGroup)
    return hip_status(cq::launch_quantize_g(group_size, w, w_dtype == CQ_BF16, rows, cols, p, packed, norms,
                                            static_cast<hipStream_t>(stream)),
                      "quantize launch");
  return hip_status(cq::launch_quantize(w, w_dtype == CQ_BF16, bits == CQ_TERNARY_TRITS, rows, cols, p,
                                        packed, norms,
                                        static_cast<hipStream_t>(stream)),
                    "quantize launch");
}

int cq_quantize_many(int n, const cq_quant_desc* descs, int w_dtype, int bits, int group_size,
                     const float* levels, int n_levels, void* stream) {
  g_last_error[0] = 0;
  int L, rc;
  if ((rc = check_bits(bits, false, &L))) return rc;
  if (w_dtype != CQ_F32 && w_dtype != CQ_BF16) return fail(CQ_ERR_ARG, "unknown w_dtype %d", w_dtype);
  if (n < 0) return fail(CQ_ERR_ARG, "n < 0");
  if ((rc = check_codec_group(group_size, bits))) return rc;
  if ((rc = check_levels(levels, n_levels, L, bits))) return rc;
  if (n == 0) return CQ_OK;
  if (!descs) return fail(CQ_ERR_NULL, "descs is NULL");
  const size_t esz = w_dtype == CQ_F32 ? 4 : 2;
  const int64_t gb = group_bytes(bits, group_size);
  ManyTables<cq::QuantDesc> t;
  std::vector<Span> outs, ins;
  for (int i = 0; i < n; ++i) {
    const cq_quant_desc& d = descs[i];
    if (d.rows < 0 || d.cols < 0) return fail(CQ_ERR_ARG, "tensor %d: negative size", i);
    if (d.rows == 0 || d.cols == 0) continue;
    if (!d.w || !d.packed || !d.norms) return fail(CQ_ERR_NULL, "tensor %d: w/packed/norms is NULL", i);
    if (!aligned(d.w, 16) || !aligned(d.packed, packed_align(bits, group_size)) || !aligned(d.norms, 2))
      return fail(CQ_ERR_ALIGN, "tensor %d: w needs 16-byte, packed 16-byte (G != 128: 4-byte; trits: 2-byte, any at G != 128), norms 2-byte alignment", i);
    const int64_t ng = d.rows * ceil_div(d.cols, group_size);
    ins.push_back(span(d.w, static_cast<size_t>(d.rows * d.cols) * esz, i));
    outs.push_back(span(d.packed, static_cast<size_t>(ng * gb), i));
    outs.push_back(span(d.norms, static_cast<size_t>(ng) * 2, i));
    t.add(cq::QuantDesc{static_cast<const uint8_t*>(d.w), d.packed, d.norms, d.rows, d.cols}, ng,
          d.cols % group_size == 0);
  }
  const int bad = first_conflict(outs, ins);
  if (bad >= 0) return fail(CQ_ERR_ARG, "tensor %d: buffers overlap another buffer of the call", bad);
  if (t.empty()) return CQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const cq::QuantParams p = make_quant_params(levels, L);
  if (group_size != cq::kGroup) {
    // Other group sizes: the single-tensor kernels, one launch per tensor.
    for (int i = 0; i < n && !rc; ++i) {
      const cq_quant_desc& d = descs[i];
      if (d.rows == 0 || d.cols == 0) continue;
      rc = bits == CQ_TERNARY_TRITS
               ? quantize_trits_g(d.w, w_dtype == CQ_BF16, d.rows, d.cols, group_size, p, d.packed, d.norms, s)
               : hip_status(cq::launch_quantize_g(group_size, d.w, w_dtype == CQ_BF16, d.rows, d.cols, p,
                                                  d.packed, d.norms, s),
                            "quantize launch");
    }
    return rc;
  }
  rc = t.upload(s);
  if (!rc)
    rc = hip_status(cq::launch_quantize_many(w_dtype == CQ_BF16, bits == CQ_TERNARY_TRITS, p, t.tc, t.bstart.back(), t.tr,
                                             t.gstart.back(), t.ragged_gcd, s),
                    "quantize launch");
  const int rc2 = t.release(s);
  return rc ? rc : rc2;
}

int cq_dequantize_many(int n, const cq_dequant_desc* descs, int bits, int group_size,
                       const float* levels, int n_levels, int out_dtype, void* stream) {
  g_last_error[0] = 0;
  int L, rc;
  if ((rc = check_bits(bits, false, &L))) return rc;
  if (out_dtype != CQ_F32 && out_dtype != CQ_BF16)
    return fail(CQ_ERR_ARG, "unknown out_dtype %d", out_dtype);
  if (n < 0) return fail(CQ_ERR_ARG, "n < 0");
  if ((rc = check_codec_group(group_size, bits))) return rc;
  if ((rc = check_levels(levels, n_levels, L, bits))) return rc;
  if (n == 0) return CQ_OK;
  if (!descs) return fail(CQ_ERR_NULL, "descs is NULL");
  const size_t esz = out_dtype == CQ_F32 ? 4 : 2;
  const int64_t gb = group_bytes(bits, group_size);
  ManyTables<cq::DequantDesc> t;
  std::vector<Span> outs, ins;
  for (int i = 0; i < n; ++i) {
    const cq_dequant_desc& d = descs[i];
    if (d.rows < 0 || d.cols < 0) return fail(CQ_ERR_ARG, "tensor %d: negative size", i);
    if (d.rows == 0 || d.cols == 0) continue;
    if (!d.packed || !d.norms || !d.out) return fail(CQ_ERR_NULL, "tensor %d: packed/norms/out is NULL", i);
    if (!aligned(d.out, 16) || !aligned(d.packed, packed_align(bits, group_size)) || !aligned(d.norms, 2))
      return fail(CQ_ERR_ALIGN, "tensor %d: out needs 16-byte, packed 16-byte (G != 128: 4-byte; trits: 2-byte, any at G != 128), norms 2-byte alignment", i);
    const int64_t ng = d.rows * ceil_div(d.cols, group_size);
    ins.push_back(span(d.packed, static_cast<size_t>(ng * gb), i));
    ins.push_back(span(d.norms, static_cast<size_t>(ng) * 2, i));
    outs.push_back(span(d.out, static_cast<size_t>(d.rows * d.cols) * esz, i));
    t.add(cq::DequantDesc{d.packed, d.norms, static_cast<uint8_t*>(d.out), d.rows, d.cols}, ng,
          d.cols % group_size == 0);
  }
  const int bad = first_conflict(outs, ins);
  if (bad >= 0) return fail(CQ_ERR_ARG, "tensor %d: buffers overlap another buffer of the call", bad);
  if (t.empty()) return CQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const cq::LevelTable lv = make_table(levels, L);
  if (group_size != cq::kGroup) {
    // Other group sizes: the single-tensor kernels, one launch per tensor.
    for (int i = 0; i < n && !rc; ++i) {
      const cq_dequant_desc& d = descs[i];
      if (d.rows == 0 || d.cols == 0) continue;
      rc = bits == CQ_TERNARY_TRITS
               ? dequantize_trits_g(d.packed, d.norms, d.rows, d.cols, group_size, lv, d.out, out_dtype == CQ_BF16, s)
               : hip_status(cq::launch_dequantize_g(group_size, d.packed, d.norms, d.rows, d.cols,
                                                    storage_bits(bits), lv, d.out, out_dtype == CQ_BF16, s),
                            "dequantize launch");
    }
    return rc;
  }
  rc = t.upload(s);
  if (!rc)
    rc = hip_status(cq::launch_dequantize_many(storage_code(bits), lv, out_dtype == CQ_BF16, t.tc, t.bstart.back(), t.tr,
                                               t.gstart.back(), t.ragged_gcd, s),
                    "dequantize launch");
  const int rc2 = t.release(s);
  return rc ? rc : rc2;
}

// Validates one matrix of a product call (sizes, pointers, alignment,
// overlap of y with the inputs).
static int check_matvec_desc(const cq_matvec_desc& d, int i, int64_t batch, int sb, int group_size) {
  if (d.n_out < 0 || d.k < 0) return fail(CQ_ERR_ARG, "matrix %d: negative size", i);
  if (d.k % group_size)
    return fail(CQ_ERR_UNSUPPORTED, "matrix %d: k=%lld is not a multiple of %d", i, (long long)d.k,
                group_size);
  if (d.n_out == 0) return CQ_OK;
  if (!d.y) return fail(CQ_ERR_NULL, "matrix %d: y is NULL", i);
  if (!aligned(d.y, 16)) return fail(CQ_ERR_ALIGN, "matrix %d: y needs 16-byte alignment", i);
  if (d.k == 0) return CQ_OK;
  if (!d.packed || !d.norms || !d.x) return fail(CQ_ERR_NULL, "matrix %d: packed/norms/x is NULL", i);
  if (!aligned(d.x, 16) || !aligned(d.packed, 16) || !aligned(d.norms, 2))
    return fail(CQ_ERR_ALIGN, "matrix %d: x, packed need 16-byte, norms 2-byte alignment", i);
  const int64_t ng = d.n_out * (d.k / group_size);
  const size_t y_bytes = static_cast<size_t>(batch * d.n_out) * 4;
  const size_t pk_bytes = static_cast<size_t>(ng) * group_size * sb / 8;
  if (overlap(d.y, y_bytes, d.packed, pk_bytes) || overlap(d.y, y_bytes, d.norms, ng * 2) ||
      overlap(d.y, y_bytes, d.x, static_cast<size_t>(batch * d.k) * 4))
    return fail(CQ_ERR_ARG, "matrix %d: input and output buffers overlap", i);
  return CQ_OK;
}

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
static uint32_t bf16_rne_host(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

int cq_dequant_gemm_many(int n, const cq_matvec_desc* descs, int bits, int group_size,
                         const float* levels, int n_levels, int64_t batch, void* stream) {
  g_last_error[0] = 0;
  int L, rc;
  if ((rc = check_bits(bits, false, &L))) return rc;
  if ((rc = reject_trits(bits))) return rc;
  if (n < 0) return fail(CQ_ERR_ARG, "n < 0");
  if (batch < 1) return fail(CQ_ERR_ARG, "batch must be >= 1");
  if ((rc = check_codec_group(group_size, bits))) return rc;
  if ((rc = check_levels(levels, n_levels, L, bits))) return rc;
  if (n == 0) return CQ_OK;
  if (!descs) return fail(CQ_ERR_NULL, "descs is NULL");
  const int sb = storage_bits(bits);
  std::vector<Span> outs, ins;
  for (int i = 0; i < n; ++i) {
    const cq_matvec_desc& d = descs[i];
    if (d.n_out < 0 || d.k < 0) return fail(CQ_ERR_ARG, "matrix %d: negative size", i);
    // The GEMM runs 128-column tiles whatever the group size.
    const int64_t kmul = group_size > cq::kGroup ? group_size : cq::kGroup;
    if (d.k % kmul)
      return fail(CQ_ERR_UNSUPPORTED, "matrix %d: k=%lld is not a multiple of %lld", i, (long long)d.k,
                  (long long)kmul);
    if (d.n_out == 0) continue;
    if (!d.y) return fail(CQ_ERR_NULL, "matrix %d: y is NULL", i);
    if (!aligned(d.y, 16)) return fail(CQ_ERR_ALIGN, "matrix %d: y needs 16-byte alignment", i);
    outs.push_back(span(d.y, static_cast<size_t>(batch * d.n_out) * 4, i));
    if (d.k == 0) continue;
    if (!d.packed || !d.norms || !d.x) return fail(CQ_ERR_NULL, "matrix %d: packed/norms/x is NULL", i);
    if (!aligned(d.x, 16) || !aligned(d.packed, 16) || !aligned(d.norms, 2))
      return fail(CQ_ERR_ALIGN, "matrix %d: x, packed need 16-byte, norms 2-byte alignment", i);
    const int64_t ng = d.n_out * (d.k / group_size);
    ins.push_back(span(d.packed, static_cast<size_t>(ng) * group_size * sb / 8, i));
    ins.push_back(span(d.norms, static_cast<size_t>(ng) * 2, i));
    ins.push_back(span(d.x, static_cast<size_t>(batch * d.k) * 4, i));
  }
  const int bad = first_conflict(outs, ins);
  if (bad >= 0) return fail(CQ_ERR_ARG, "matrix %d: y overlaps another buffer of the call", bad);
  hipStream_t s = static_cast<hipStream_t>(stream);

  cq::SplitLevels sl{};
  for (int i = 0; i < L; ++i) {
    const uint32_t hi = bf16_rne_host(levels[i]);
    float hv;
    const uint32_t hb = hi << 16;
    std::memcpy(&hv, &hb, 4);
    sl.hi[i] = hi;
    sl.lo[i] = bf16_rne_host(levels[i] - hv);
  }
  const int64_t bm = cq::gemm_block_rows(batch, group_size), bn = cq::gemm_block_cols();
  const int64_t mpad = ceil_div(batch, bm) * bm;
  std::vector<cq::GemmDesc> act;
  for (int i = 0; i < n; ++i) {
    const cq_matvec_desc& d = descs[i];
    if (d.n_out == 0) continue;
    if (d.k == 0) {
      if ((rc = hip_status(cq::launch_zero(d.y, batch * d.n_out, s), "zero launch"))) return rc;
      continue;
    }
    act.push_back(cq::GemmDesc{d.packed, d.norms, d.x, d.y, d.n_out, d.k, mpad, 0, nullptr, 1, 0});
  }
  if (act.empty()) return CQ_OK;
  const int na = static_cast<int>(act.size());
  // When the call's output tiles would not give every CU two blocks, each
  // tile's 128-groups are split into `split` ranges (one block each) whose
  // partial sums a reduction launch adds in range order.
  int64_t tiles = 0;
  for (const cq::GemmDesc& g : act) tiles += (mpad / bm) * ceil_div(g.n_out, bn);
  const int64_t target = 2 * static_cast<int64_t>(cq::device_cu_count());
  const int64_t split = tiles >= target ? 1 : ceil_div(target, tiles);
  std::vector<int64_t> ustart{0}, bstart{0}, ostart{0}, part_off;
  int64_t xs = 0, parts = 0;  // bf16 values; partial-sum floats
  for (cq::GemmDesc& g : act) {
    const int64_t ngr = g.k / cq::kGroup;  // 128-column tiles
    g.xs_off = xs;
    g.gps = ceil_div(ngr, split);
    g.ksplit = ceil_div(ngr, g.gps);  // every range non-empty
    xs += ngr * mpad * 2 * cq::kGroup;
    ustart.push_back(ustart.back() + (g.k / group_size) * mpad);  // rotation units: (group, row)
    bstart.push_back(bstart.back() + (mpad / bm) * ceil_div(g.n_out, bn) * g.ksplit);
    ostart.push_back(ostart.back() + batch * g.n_out);
    part_off.push_back(parts);
    if (split > 1) parts += g.ksplit * batch * g.n_out;
  }
  auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t tb = up(na * sizeof(cq::GemmDesc)), sb_ = up((na + 1) * 8);
  const size_t xb = up(static_cast<size_t>(xs) * 2);
  const size_t ws_bytes = tb + 3 * sb_ + xb + static_cast<size_t>(parts) * 4;
  uint8_t* ws = nullptr;
  if ((rc = hip_status(hipMallocAsync(reinterpret_cast<void**>(&ws), ws_bytes, s), "workspace alloc")))
    return rc;
  auto* table = reinterpret_cast<cq::GemmDesc*>(ws);
  auto* u_dev = reinterpret_cast<int64_t*>(ws + tb);
  auto* b_dev = reinterpret_cast<int64_t*>(ws + tb + sb_);
  auto* o_dev = reinterpret_cast<int64_t*>(ws + tb + 2 * sb_);
  auto* xs_dev = reinterpret_cast<uint16_t*>(ws + tb + 3 * sb_);
  auto* part_dev = reinterpret_cast<float*>(ws + tb + 3 * sb_ + xb);
  if (split > 1)
    for (int i = 0; i < na; ++i) act[i].part = part_dev + part_off[i];
  rc = hip_status(cq::upload(act.data(), na * sizeof(cq::GemmDesc), table, s), "table upload");
  if (!rc) rc = hip_status(cq::upload(ustart.data(), (na + 1) * 8, u_dev, s), "table upload");
  if (!rc) rc = hip_status(cq::upload(bstart.data(), (na + 1) * 8, b_dev, s), "table upload");
  if (!rc && split > 1) rc = hip_status(cq::upload(ostart.data(), (na + 1) * 8, o_dev, s), "table upload");
  if (!rc)
    rc = hip_status(cq::launch_split_rotate(table, u_dev, na, ustart[na], batch, group_size, xs_dev, s),
                    "rotate launch");
  if (!rc)
    rc = hip_status(cq::launch_gemm(table, b_dev, na, bstart[na], sb, sl, xs_dev, batch, group_size, s),
                    "gemm launch");
  if (!rc && split > 1)
    rc = hip_status(cq::launch_gemm_reduce(table, o_dev, na, ostart[na], batch, s), "reduce launch");
  const int rc2 = hip_status(hipFreeAsync(ws, s), "workspace free");
  return rc ? rc : rc2;
}

int cq_dequant_gemm(const uint8_t* packed, const uint16_t* norms, int64_t n_out, int64_t k, int bits,
                    int group_size, const float* levels, int n_levels, const float* x, int64_t batch,
                    float* y, void* stream) {
  const cq_matvec_desc d{packed, norms, n_out, k, x, y};
  return cq_dequant_gemm_many(1, &d, bits, group_size, levels, n_levels, batch, stream);
}

int cq_repack(const uint8_t* src, int src_bits, uint8_t* dst, int dst_bits, int64_t n_groups,
              int group_size, void* stream) {
  g_last_error[0] = 0;
  int rc;
  const bool to_trits = src_bits == CQ_TERNARY && dst_bits == CQ_TERNARY_TRITS;
  const bool to_fields = src_bits == CQ_TERNARY_TRITS && dst_bits == CQ_TERNARY;
  if (!to_trits && !to_fields)
    return fail(CQ_ERR_ARG, "cq_repack converts between CQ_TERNARY and CQ_TERNARY_TRITS (got %d -> %d)",
                src_bits, dst_bits);
  if (n_groups < 0) return fail(CQ_ERR_ARG, "n_groups < 0");
  if ((rc = check_codec_group(group_size, CQ_TERNARY_TRITS))) return rc;
  if (n_groups == 0) return CQ_OK;
  if (!src || !dst) return fail(CQ_ERR_NULL, "src/dst is NULL");
  const uint8_t* fields = to_trits ? src : dst;
  const uint8_t* trits = to_trits ? dst : src;
  if (!aligned(fields, packed_align(CQ_TERNARY, group_size)) ||
      !aligned(trits, packed_align(CQ_TERNARY_TRITS, group_size)))
    return fail(CQ_ERR_ALIGN, "2-bit fields need 16-byte (G != 128: 4-byte), trit storage 2-byte (G != 128: any) alignment");
  if (overlap(src, static_cast<size_t>(n_groups * group_bytes(src_bits, group_size)), dst,
              static_cast<size_t>(n_groups * group_bytes(dst_bits, group_size))))
    return fail(CQ_ERR_ARG, "src and dst overlap");
  return hip_status(cq::launch_repack(src, to_trits, dst, n_groups, group_size, static_cast<hipStream_t>(stream)),
                    "repack launch");
}

int cq_blob_layout(int n_tensors, const int64_t* rows, const int64_t* cols, int bits, int group_size,
                   int64_t* packed_offsets, int64_t* norm_offsets, int64_t* total_bytes) {
  g_last_error[0] = 0;
  int rc;
  if (n_tensors < 0) return fail(CQ_ERR_ARG, "n_tensors < 0");
  if (n_tensors > 0 && (!rows || !cols)) return fail(CQ_ERR_NULL, "rows/cols is NULL");
  if ((rc = check_bits(bits, true, nullptr))) return rc;
  if ((rc = check_group(group_size, false))) return rc;
  const int64_t per_group = group_bytes(bits, group_size);
  int64_t packed_total = 0, norms_total = 0;
  for (int i = 0; i < n_tensors; ++i) {
    if (rows[i] < 0 || cols[i] < 0) return fail(CQ_ERR_ARG, "tensor %d has a negative size", i);
    packed_total += rows[i] * ceil_div(cols[i], group_size) * per_group;
  }
  // An odd index section (trit storage with 7- or 13-byte groups) is followed
  // by one pad byte, so the binary16 norms start at an even offset.
  const int64_t norms_start = packed_total + packed_total % 2;
  int64_t p = 0;
  for (int i = 0; i < n_tensors; ++i) {
    const int64_t ng = rows[i] * ceil_div(cols[i], group_size);
    if (packed_offsets) packed_offsets[i] = p;
    if (norm_offsets) norm_offsets[i] = norms_start + norms_total;
    p += ng * per_group;
    norms_total += 2 * ng;
  }
  if (total_bytes) *total_bytes = norms_start + norms_total;
  return CQ_OK;
}

int cq_fake_quant(const void* w, int w_dtype, int64_t rows, int64_t cols, int bits,
                  int group_size, const float* levels, int n_levels, void* out, int out_dtype,
                  void* stream) {
  g_last_error[0] = 0;
  int L, rc;
  if ((rc = check_bits(bits, false, &L))) return rc;
  if (w_dtype != CQ_F32 && w_dtype != CQ_BF16) return fail(CQ_ERR_ARG, "unknown w_dtype %d", w_dtype);
  if (out_dtype != CQ_F32 && out_dtype != CQ_BF16)
    return fail(CQ_ERR_ARG, "unknown out_dtype %d", out_dtype);
  if (rows < 0 || cols < 0) return fail(CQ_ERR_ARG, "negative size");
  if ((rc = check_codec_group(group_size, bits))) return rc;
  if ((rc = check_levels(levels, n_levels, L, bits))) return rc;
  if (rows == 0 || cols == 0) return CQ_OK;
  if (!w || !out) return fail(CQ_ERR_NULL, "w/out is NULL");
  if (!aligned(w, 16) || !aligned(out, 16))
    return fail(CQ_ERR_ALIGN, "w and out need 16-byte alignment");
  const size_t in_bytes = static_cast<size_t>(rows * cols) * (w_dtype == CQ_F32 ? 4 : 2);
  const size_t out_bytes = static_cast<size_t>(rows * cols) * (out_dtype == CQ_F32 ? 4 : 2);
  const bool in_place = w == out && w_dtype == out_dtype;
  if (!in_place && overlap(w, in_bytes, out, out_bytes))
    return fail(CQ_ERR_ARG, "w and out overlap (only out == w with equal dtypes is allowed)");
  const cq::QuantParams p = make_quant_params(levels, L);
  const cq::LevelTable lv = make_table(levels, L);
  if (group_size != cq::kGroup)
    return hip_status(cq::launch_fake_quant_g(group_size, w, w_dtype == CQ_BF16, rows, cols, p, lv, out,
                                              out_dtype == CQ_BF16, static_cast<hipStream_t>(stream)),
                      "fake-quant launch");
  return hip_status(cq::launch_fake_quant(w, w_dtype == CQ_BF16, rows, cols, p, lv, out,
                                          out_dtype == CQ_BF16, static_cast<hipStream_t>(stream)),
                    "fake-quant launch");
}

int cq_dequantize(const uint8_t* packed, const uint16_t* norms, int64_t rows, int64_t cols,
                  int bits, int group_size, const float* levels, int n_levels, void* out,
                  int out_dtype, void* stream) {
  g_last_error[0] = 0;
  int L, rc;
  if ((rc = check_bits(bits, false, &L))) return rc;
  if (out_dtype != CQ_F32 && out_dtype != CQ_BF16)
    return fail(CQ_ERR_ARG, "unknown out_dtype %d", out_dtype);
  if (rows < 0 || cols < 0) return fail(CQ_ERR_ARG, "negative size");
  if ((rc = check_codec_group(group_size, bits))) return rc;
  if ((rc = check_levels(levels, n_levels, L, bits))) return rc;
  if (rows == 0 || cols == 0) return CQ_OK;
  if (!packed || !norms || !out) return fail(CQ_ERR_NULL, "packed/norms/out is NULL");
  if (!aligned(out, 16) || !aligned(packed, packed_align(bits, group_size)) || !aligned(norms, 2))
    return fail(CQ_ERR_ALIGN, "out needs 16-byte, packed 16-byte (G != 128: 4-byte; trits: 2-byte, any at G != 128), norms 2-byte alignment");
  const int64_t ng = rows * ceil_div(cols, group_size);
  const size_t out_bytes = static_cast<size_t>(rows * cols) * (out_dtype == CQ_F32 ? 4 : 2);
  const size_t pk_bytes = static_cast<size_t>(ng * group_bytes(bits, group_size));
  if (overlap(out, out_bytes, packed, pk_bytes) || overlap(out, out_bytes, norms, ng * 2))
    return fail(CQ_ERR_ARG, "input and output buffers overlap");
  const cq::LevelTable lv = make_table(levels, L);
  if (group_size != cq::kGroup && bits == CQ_TERNARY_TRITS)
    return dequantize_trits_g(packed, norms, rows, cols, group_size, lv, out, out_dtype == CQ_BF16,
                              static_cast<hipStream_t>(stream));
  if (group_size != cq::kGroup)
    return hip_status(cq::launch_dequantize_g(group_size, packed, norms, rows, cols, storage_bits(bits), lv,
                                              out, out_dtype == CQ_BF16, static_cast<hipStream_t>(stream)),
                      "dequantize launch");
  return hip_status(cq::launch_dequantize(packed, norms, rows, cols, storage_code(bits), lv, out,
                                          out_dtype == CQ_BF16, static_cast<hipStream_t>(stream)),
                    "dequantize launch");
}

int cq_dequant_matvec(const uint8_t* packed, const uint16_t* norms, int64_t n_out, int64_t k,
                      int bits, int group_size, const float* levels, int n_levels, const float* x,
                      int64_t batch, float* y, void* stream) {
  g_last_error[0] = 0;
  int L, rc;
  if ((rc = check_bits(bits, false, &L))) return rc;
  if ((rc = reject_trits(bits))) return rc;
  if (batch < 1) return fail(CQ_ERR_ARG, "batch must be >= 1");
  if ((rc = check_codec_group(group_size, bits))) return rc;
  if ((rc = check_levels(levels, n_levels, L, bits))) return rc;
  const cq_matvec_desc d{packed, norms, n_out, k, x, y};
  if ((rc = check_matvec_desc(d, 0, batch, storage_bits(bits), group_size))) return rc;
  if (k > (int64_t(1) << 28))
    return fail(CQ_ERR_UNSUPPORTED, "k=%lld: the single-matrix product takes k <= 2^28", (long long)k);
  if (n_out == 0) return CQ_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (k == 0) return hip_status(cq::launch_zero(y, batch * n_out, s), "zero launch");
  // One launch: the descriptor is a kernel argument and every block rotates
  // the activations it consumes.
  const int sb = storage_bits(bits);
  const cq::MatvecArgs a{packed, norms, x, y, n_out, k, batch};
  return hip_status(cq::launch_matvec_one(a, sb, make_table(levels, L), group_size,
                                          cq::matvec_one_plan(sb, n_out, k, batch), s),
                    "matvec launch");
}

int cq_dequant_matvec_many(int n, const cq_matvec_desc* descs, int bits, int group_size,
                           const float* levels, int n_levels, int64_t batch, void* stream) {
  return cq::matvec_many_impl(n, descs, bits, group_size, levels, n_levels, batch, stream, nullptr, 0);
}

}  // extern "C"

namespace cq {

// The multi-matrix product with its workspace either stream-ordered
// (fixed_ws == nullptr: hipMallocAsync / hipFreeAsync on the stream) or a
// fixed one of fixed_cap bytes whose device address fixed_ws returns
// (nothing allocated; a call that needs more is rejected before anything is
// enqueued, and fixed_ws is called only once the call is known to run).
// Device copies of the descriptor tables of the multi-matrix product, one per
// (device, stream), reused when a call's tables equal the previous call's on
// that stream byte for byte: a decode loop runs the product over the same
// matrices and buffers at every step, and the upload (kernel launches of
// 48 descriptors each, 4.6 us apiece; five for 225 matrices) is then
// skipped.  A table is rewritten only after the stream has waited for the
// event recorded after its last use, so readers still running from an
// earlier stream with the same handle cannot see a half-written table.  The
// entries live until the process ends.
struct TableCache {
  std::vector<uint8_t> host;  // the bytes the device copy holds
  uint8_t* dev = nullptr;
  size_t cap = 0;
  hipEvent_t last_use = nullptr;
};
std::mutex g_table_cache_mutex;
std::map<std::pair<int, hipStream_t>, TableCache> g_table_cache;

int matvec_many_impl(int n, const cq_matvec_desc* descs, int bits, int group_size, const float* levels,
                     int n_levels, int64_t batch, void* stream, int (*fixed_ws)(uint8_t**), size_t fixed_cap) {
  g_last_error[0] = 0;
  int L, rc;
  if ((rc = check_bits(bits, false, &L))) return rc;
  if ((rc = reject_trits(bits))) return rc;
  if (n < 0) return fail(CQ_ERR_ARG, "n < 0");
  if (batch < 1) return fail(CQ_ERR_ARG, "batch must be >= 1");
  if ((rc = check_codec_group(group_size, bits))) return rc;
  if ((rc = check_levels(levels, n_levels, L, bits))) return rc;
  if (n == 0) return CQ_OK;
  if (!descs) return fail(CQ_ERR_NULL, "descs is NULL");
  const int sb = storage_bits(bits);
  for (int i = 0; i < n; ++i)
    if ((rc = check_matvec_desc(descs[i], i, batch, sb, group_size))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const cq::LevelTable lv = make_table(levels, L);

  // Matrices with k = 0 produce zeros; the rest go to the descriptor table.
  std::vector<cq::MatvecDesc> act;
  std::vector<int> zero_k;
  for (int i = 0; i < n; ++i) {
    const cq_matvec_desc& d = descs[i];
    if (d.n_out == 0) continue;
    if (d.k == 0) {
      zero_k.push_back(i);
      continue;
    }
    act.push_back(cq::MatvecDesc{d.packed, d.norms, d.x, d.y, d.n_out, d.k, 0});
  }
  const int na = static_cast<int>(act.size());
  if (na == 0) {
    for (int i : zero_k)
      if ((rc = hip_status(cq::launch_zero(descs[i].y, batch * descs[i].n_out, s), "zero launch"))) return rc;
    return CQ_OK;
  }
  // Batch rows go through the product kernel in chunks of `chunk` rows.
  const int chunk = cq::matvec_chunk(sb, batch, act.data(), na);
  const int nb_full = static_cast<int>(batch < chunk ? batch : chunk);
  const int nb_last = static_cast<int>(batch - chunk * ((batch - 1) / chunk));
  const cq::MatvecPlan plan0 = cq::matvec_plan(sb, nb_full, act.data(), na);
  const cq::MatvecPlan plan1 = cq::matvec_plan(sb, nb_last, act.data(), na);
  const int rb0 = plan0.rows_per_block, rb1 = plan1.rows_per_block;
  std::vector<int64_t> gstart(na + 1), bstart0(na + 1), bstart1(na + 1);
  int64_t xr_floats = 0;
  for (int i = 0; i < na; ++i) {
    act[i].xr_offset = xr_floats;
    xr_floats += batch * act[i].k;
    gstart[i + 1] = gstart[i] + batch * (act[i].k / group_size);
    bstart0[i + 1] = bstart0[i] + (act[i].n_out + rb0 - 1) / rb0;
    bstart1[i + 1] = bstart1[i] + (act[i].n_out + rb1 - 1) / rb1;
  }
  auto round_up = [](size_t v) { return (v + 255) & ~size_t(255); };
  const size_t table_b = round_up(na * sizeof(cq::MatvecDesc));
  const size_t start_b = round_up((na + 1) * sizeof(int64_t));
  const size_t ws_bytes = table_b + 3 * start_b + static_cast<size_t>(xr_floats) * sizeof(float);
  if (fixed_ws && ws_bytes > fixed_cap)
    return fail(CQ_ERR_UNSUPPORTED,
                "this call needs %zu bytes of workspace (the descriptor table and batch * sum(k) rotated "
                "activations); the fixed workspace holds %zu",
                ws_bytes, fixed_cap);
  uint8_t* ws = nullptr;
  if (fixed_ws && (rc = fixed_ws(&ws))) return rc;
  for (int i : zero_k)
    if ((rc = hip_status(cq::launch_zero(descs[i].y, batch * descs[i].n_out, s), "zero launch"))) return rc;
  // Tables: in the fixed workspace, or in this stream's cached copy.
  const size_t tables_bytes = table_b + 3 * start_b;
  std::unique_lock<std::mutex> cache_lock;
  TableCache* tc = nullptr;
  bool upload_tables = true;
  uint8_t* tabs = ws;
  uint8_t* xr_mem = ws + tables_bytes;
  if (!fixed_ws) {
    std::vector<uint8_t> host(tables_bytes, 0);
    std::memcpy(host.data(), act.data(), na * sizeof(cq::MatvecDesc));
    std::memcpy(host.data() + table_b, gstart.data(), (na + 1) * sizeof(int64_t));
    std::memcpy(host.data() + table_b + start_b, bstart0.data(), (na + 1) * sizeof(int64_t));
    std::memcpy(host.data() + table_b + 2 * start_b, bstart1.data(), (na + 1) * sizeof(int64_t));
    int dev = 0;
    if ((rc = hip_status(hipGetDevice(&dev), "get device"))) return rc;
    cache_lock = std::unique_lock<std::mutex>(g_table_cache_mutex);
    tc = &g_table_cache[{dev, s}];
    if (!tc->last_use && (rc = hip_status(hipEventCreateWithFlags(&tc->last_use, hipEventDisableTiming), "event")))
      return rc;
    if (tc->dev && tc->host == host) {
      upload_tables = false;
    } else {
      // Earlier readers of the copy finish before it is rewritten or freed.
      if (tc->dev && (rc = hip_status(hipStreamWaitEvent(s, tc->last_use, 0), "event wait"))) return rc;
      if (tc->cap < tables_bytes) {
        if (tc->dev && (rc = hip_status(hipFreeAsync(tc->dev, s), "table free"))) return rc;
        tc->dev = nullptr;
        tc->cap = 0;
        tc->host.clear();
        if ((rc = hip_status(hipMallocAsync(reinterpret_cast<void**>(&tc->dev), tables_bytes, s), "table alloc")))
          return rc;
        tc->cap = tables_bytes;
      }
      tc->host = std::move(host);
    }
    tabs = tc->dev;
    const size_t xr_bytes = static_cast<size_t>(xr_floats) * sizeof(float);
    if ((rc = hip_status(hipMallocAsync(reinterpret_cast<void**>(&xr_mem), xr_bytes, s), "workspace alloc"))) {
      tc->host.clear();  // the upload below is not enqueued
      return rc;
    }
    ws = xr_mem;
  }
  auto* table = reinterpret_cast<cq::MatvecDesc*>(tabs);
  auto* g_dev = reinterpret_cast<int64_t*>(tabs + table_b);
  auto* b0_dev = reinterpret_cast<int64_t*>(tabs + table_b + start_b);
  auto* b1_dev = reinterpret_cast<int64_t*>(tabs + table_b + 2 * start_b);
  auto* xr = reinterpret_cast<float*>(xr_mem);
  for (int first = 0; first < na && !rc && upload_tables; first += cq::kDescPerInit) {
    cq::DescChunk c{};
    c.first = first;
    c.count = na - first < cq::kDescPerInit ? na - first : cq::kDescPerInit;
    c.last_chunk = first + c.count == na ? 1 : 0;
    for (int i = 0; i < c.count; ++i) c.d[i] = act[first + i];
    for (int i = 0; i < c.count + c.last_chunk; ++i) {
      c.gstart[i] = gstart[first + i];
      c.bstart0[i] = bstart0[first + i];
      c.bstart1[i] = bstart1[first + i];
    }
    rc = hip_status(cq::launch_table_init(c, table, g_dev, b0_dev, b1_dev, s), "table launch");
  }
  if (!rc) rc = hip_status(cq::launch_rotate(table, g_dev, na, gstart[na], group_size, xr, s), "rotate launch");
  for (int64_t b0 = 0; b0 < batch && !rc; b0 += chunk) {
    const int nb = static_cast<int>(batch - b0 < chunk ? batch - b0 : chunk);
    const bool full = nb == nb_full;
    rc = hip_status(cq::launch_matvec(table, full ? b0_dev : b1_dev, na, full ? bstart0[na] : bstart1[na],
                                      sb, lv, xr, b0, nb, full ? plan0 : plan1, group_size, s),
                    "matvec launch");
  }
  if (tc) {
    if (rc && upload_tables) tc->host.clear();  // the device copy may be incomplete
    const int rc3 = hip_status(hipEventRecord(tc->last_use, s), "event record");
    rc = rc ? rc : rc3;
  }
  const int rc2 = fixed_ws ? CQ_OK : hip_status(hipFreeAsync(ws, s), "workspace free");
  return rc ? rc : rc2;
}

int report(int status, const char* msg) { return fail(status, "%s", msg); }

}  // namespace cq

