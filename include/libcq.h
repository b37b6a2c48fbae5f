/*
 * libcq - Cactus-Quants (CQ) rotated-codebook weight quantizer for AMD
 * MI355X (gfx950).  C ABI.
 *
 * The method (sources are web pages, cited by title and section):
 *   - weights are cut into groups of G consecutive values along the last axis
 *     (G = 128 unless stated), the last group of a row zero-padded
 *     ("Cactus Quants CQ2-bit Quantization: Extreme Compression for Edge
 *     LLMs", section Group-wise Weight Partitioning);
 *   - each group is rotated by the orthonormal Walsh-Hadamard matrix
 *     (same page, section Hadamard Rotation);
 *   - the rotated values are normalised by the group's L2 norm and snapped to
 *     the nearest level of a fixed Lloyd-Max codebook for N(0,1), whose levels
 *     are used divided by sqrt(G)
 *     ("How Quantization Codebooks Are Trained in Cactus Quants: Lloyd-Max on
 *     Gaussian Data", sections Iterative Refinement of Quantization Levels and
 *     Production Codebook Generation and Caching);
 *   - storage is the packed indices plus one binary16 norm per group
 *     ("How CQ2-bit Quantization Contributes to Needle 2's Small Footprint",
 *     sections Per-Group Storage Breakdown and Binary Serialization);
 *   - dequantization looks the levels up, rescales and rotates back
 *     (first page, section The CQ2-bit Implementation Pipeline).
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers unless the argument says "host".
 *   - A tensor of any rank is passed as rows x cols: rows is the product of
 *     the leading dimensions, cols the last (grouping) dimension.  Rows are
 *     contiguous, row-major.
 *   - bits is one of CQ_TERNARY, CQ_TERNARY_TRITS, 2, 3, 4 (1 is accepted by
 *     the host-only calls).  Storage bits per index (sbits): 2 for CQ_TERNARY,
 *     else bits.
 *   - Packed layout: packed[rows][ceil(cols/G)][B] bytes with B = G*sbits/8
 *     bytes per group; inside a group, index j occupies bits
 *     [sbits*j, sbits*j + sbits) of a little-endian bit stream (least
 *     significant bit first).  CQ_TERNARY_TRITS instead stores B = ceil(G/5)
 *     bytes per group (26 at G = 128): index j is base-3 digit j % 5 of byte
 *     j / 5, least significant digit first, unused digits of the last byte
 *     zero.  Groups are in row-major order.
 *   - Norm layout: norms[rows][ceil(cols/G)], IEEE binary16 bit patterns,
 *     round to nearest even from the float32 norm; norms above 65504 store
 *     +Inf.
 *   - levels (host, nullable): n_levels float32 codebook levels in N(0,1)
 *     units (before the 1/sqrt(G) scaling), strictly ascending.  n_levels
 *     must be 3 for CQ_TERNARY and CQ_TERNARY_TRITS, 2^bits otherwise.
 *     NULL selects the built-in table of the width (the levels cq_codebook
 *     returns); n_levels is then ignored.
 *   - group_size: the device calls take 32, 64, 128 or 256 ("Cactus Quants
 *     CQ2-bit Quantization: Extreme Compression for Edge LLMs", FAQ on group
 *     size); the GEMM calls also need k to be a multiple of 128 (of 256 at
 *     group size 256).
 *     Host-only calls take any power of two from 8 to 4096 (so a group's
 *     packed indices fill whole bytes).
 *   - Device calls validate every argument first, then enqueue their kernels
 *     on `stream` (a hipStream_t; NULL = the null stream) and return without
 *     waiting.  On a validation error nothing is enqueued.  Asynchronous
 *     faults surface at the caller's next synchronisation.  Buffers must stay
 *     alive until the stream has passed the call.
 *   - rows*cols == 0 (or n_out == 0) is a successful no-op; a product with
 *     k == 0 writes zeros to y (an empty sum).
 *   - Alignment: w, out, packed, x, y must be 16-byte aligned; norms 2-byte;
 *     packed at group sizes other than 128 4-byte; packed in trit storage
 *     (CQ_TERNARY_TRITS) 2-byte at group size 128, any at the others.
 *   - Inputs and outputs must not overlap (cq_fake_quant allows out == w).
 *     Non-finite inputs give unspecified but deterministic results.
 *   - Return value: CQ_OK (0) or a negative cq_status.  cq_last_error()
 *     returns a thread-local message for the last failing call.
 *   - Ownership: the caller owns every buffer.  The library keeps no pointer
 *     after a call returns.
 */
#ifndef LIBCQ_H
#define LIBCQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CQ_OK = 0,
  CQ_ERR_NULL = -1,        /* a required pointer is NULL */
  CQ_ERR_ARG = -2,         /* bad bits, sizes, dtype, levels or overlap */
  CQ_ERR_ALIGN = -3,       /* misaligned pointer */
  CQ_ERR_UNSUPPORTED = -4, /* valid request this build does not implement */
  CQ_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed */
} cq_status;

typedef enum { CQ_F32 = 0, CQ_BF16 = 1 } cq_dtype;

/* Bit-width code of the three-level ("1.58-bit") codebook
 * ("How Quantization Codebooks Are Trained in Cactus Quants", section Ternary
 * Special Case Handling). */
#define CQ_TERNARY 158
/* The same three-level code stored five indices per byte: ceil(G/5) bytes
 * per group, 26 per 128-group, 1.625 bits per weight before the norm (the
 * 2-bit field form takes 32 bytes).  Accepted by the host calls,
 * cq_quantize(_many), cq_dequantize(_many) and cq_fake_quant at every group
 * size; the product calls decode the field form (convert with cq_repack). */
#define CQ_TERNARY_TRITS 159
#define CQ_GROUP 128
#define CQ_MAX_LEVELS 16

/* Sizes of the quantized form of one rows x cols tensor: the last axis is
 * zero-padded to a multiple of the group size and cut into groups ("Cactus
 * Quants CQ2-bit Quantization: Extreme Compression for Edge LLMs", section
 * Group-wise Weight Partitioning), each stored as packed indices ("How
 * CQ2-bit Quantization Contributes to Needle 2's Small Footprint", section
 * Per-Group Storage Breakdown).
 * n_groups = rows * ceil(cols / group_size);
 * packed_bytes = n_groups * B (B the bytes per group of the packed layout
 * above: group_size * sbits / 8, or ceil(group_size / 5) for trit storage).
 * Host only, pure.
 * Either output pointer may be NULL. */
int cq_layout(int64_t rows, int64_t cols, int bits, int group_size,
              int64_t* n_groups, int64_t* packed_bytes);

/* Storage size of a set of tensors: for every group, B bytes of indices (as
 * in cq_layout) plus 2 bytes of binary16 norm, and nothing else
 * ("How CQ2-bit Quantization Contributes to Needle 2's Small Footprint",
 * section Per-Group Storage Breakdown).  rows/cols are host arrays of
 * n_tensors entries.  Padded groups count in full.  Host only, pure. */
int cq_model_bytes(int n_tensors, const int64_t* rows, const int64_t* cols,
                   int bits, int group_size, uint64_t* bytes_out);

/* The built-in codebook of a width: float32 levels in N(0,1) units written
 * to levels_out (host, room for CQ_MAX_LEVELS), their count to *n_levels
 * (host).  These are the levels every call uses when its `levels` argument
 * is NULL.
 * CQ_TERNARY and CQ_TERNARY_TRITS: the fixed levels -1.2240064, 0, 1.2240064
 * ("How Quantization Codebooks Are Trained in Cactus Quants: Lloyd-Max on
 * Gaussian Data", section Ternary Special Case Handling).  Widths 1-4: the
 * same page's recipe (sections Gaussian Sampling and Initialization,
 * Iterative Refinement of Quantization Levels, Production Codebook
 * Generation and Caching): 1-D Lloyd-Max with 2^bits levels, 200 rounds,
 * on 400,000 standard-normal samples.  The pages draw the samples from a
 * seeded NumPy generator; this library draws them from its own documented
 * deterministic generator: SplitMix64 words from state 0, each turned into
 * a uniform u = ((w >> 11) + 1) * 2^-53 in (0, 1], consecutive pairs
 * (u1, u2) turned into sqrt(-2 ln u1) cos(2 pi u2) and
 * sqrt(-2 ln u1) sin(2 pi u2) (Box-Muller), each normal taken with its
 * negation (100,000 pairs, a sample set symmetric about 0).  Computed on
 * first use, cached,
 * immutable.  The levels are within sampling noise of the Gaussian Lloyd-Max
 * optimum (2 bits: about +-0.4528, +-1.510), not bit-identical to the
 * pages' own draws.  Host only. */
int cq_codebook(int bits, float* levels_out, int* n_levels);

/* Lloyd-Max on caller-supplied samples: the training recipe of
 * cq_codebook run on the n_samples host doubles `samples` for `iters`
 * rounds: sort, quantile initialisation at sorted position
 * floor((k + 1/2) n / L), then per round midpoint boundaries, assignment
 * (a sample equal to a boundary goes to the lower cell) and cell means; an
 * empty cell keeps its level; result sorted ("How Quantization Codebooks
 * Are Trained in Cactus Quants", sections Gaussian Sampling and
 * Initialization and Iterative Refinement of Quantization Levels).  The
 * ternary widths return the fixed table and ignore the samples.  Host only;
 * samples is not modified. */
int cq_codebook_train(int bits, const double* samples, int64_t n_samples, int iters,
                      float* levels_out, int* n_levels);

/* Quantize w (rows x cols, dtype w_dtype = CQ_F32 or CQ_BF16) into packed
 * indices and binary16 norms (layouts above), the steps of "Cactus Quants
 * CQ2-bit Quantization: Extreme Compression for Edge LLMs", section The
 * CQ2-bit Implementation Pipeline: pad and group, rotate each group by the
 * orthonormal Walsh-Hadamard matrix, normalise by the group's L2 norm,
 * snap to the nearest level, store indices and the binary16 norm ("How
 * CQ2-bit Quantization Contributes to Needle 2's Small Footprint", section
 * Per-Group Storage Breakdown).  levels (host, nullable: built-in table).
 * Each group's index j is the number of decision thresholds (midpoints of
 * neighbouring levels, "How Quantization Codebooks Are Trained in Cactus
 * Quants", section Iterative Refinement of Quantization Levels) strictly
 * below sqrt(G) * y_j / ||y|| (y the rotated group); an all-zero group uses
 * 0 for that value.  The decision is taken in float32; values within about
 * 1e-6 of a threshold may land on either side. */
int cq_quantize(const void* w, int w_dtype, int64_t rows, int64_t cols,
                int bits, int group_size, const float* levels, int n_levels,
                uint8_t* packed, uint16_t* norms, void* stream);

/* Dequantize packed indices + binary16 norms to out (rows x cols, dtype
 * out_dtype = CQ_F32 or CQ_BF16, pad columns not written): look the levels
 * up, rescale by the stored norm and rotate back ("Cactus Quants CQ2-bit
 * Quantization: Extreme Compression for Edge LLMs", section The CQ2-bit
 * Implementation Pipeline), i.e.
 * x_hat = (norm / G) * H * levels[idx] with H the +-1 Sylvester-Hadamard
 * matrix, which equals (norm/sqrt(G)) * levels[idx] times the orthonormal
 * Hadamard matrix.  Computed in float32 (bf16 output rounds to nearest
 * even).  levels (host, nullable: built-in table). */
int cq_dequantize(const uint8_t* packed, const uint16_t* norms, int64_t rows,
                  int64_t cols, int bits, int group_size, const float* levels,
                  int n_levels, void* out, int out_dtype, void* stream);

/* Serialized layout of n_tensors quantized tensors (rows/cols host arrays),
 * in the order of "How CQ2-bit Quantization Contributes to Needle 2's Small
 * Footprint", section Binary Serialization: the packed indices of every
 * tensor, tensor after tensor, then the binary16 norms of every tensor in the
 * same order, with no header.  When the indices take an odd number of bytes
 * (trit storage at group sizes whose groups are 7 or 13 bytes) one pad byte
 * follows them, which cq_quantize_many does not write.  Writes the byte
 * offset of tensor i's packed indices to packed_offsets[i] and of its norms
 * to norm_offsets[i] (host arrays of n_tensors entries, each may be NULL)
 * and the blob size to *total_bytes (may be NULL), which equals
 * cq_model_bytes plus that pad byte.  Every packed offset meets the call's
 * packed alignment (a multiple of 16 at group size 128, of 4 at the others,
 * of 2 in trit storage at 128, any otherwise) and every norm offset is even,
 * so a 16-byte aligned blob can take cq_quantize_many's outputs directly.
 * Host only, pure. */
int cq_blob_layout(int n_tensors, const int64_t* rows, const int64_t* cols, int bits,
                   int group_size, int64_t* packed_offsets, int64_t* norm_offsets,
                   int64_t* total_bytes);

/* One tensor of cq_quantize_many (device pointers, layouts as cq_quantize). */
typedef struct {
  const void* w;     /* rows x cols, the call's w_dtype */
  int64_t rows;
  int64_t cols;
  uint8_t* packed;   /* [rows][ceil(cols/G)][B], B as in cq_layout */
  uint16_t* norms;   /* [rows][ceil(cols/G)] */
} cq_quant_desc;

/* cq_quantize over n tensors (descs: host array) sharing w_dtype, bits and
 * levels, e.g. every weight of a model, in one call (a parameter tree
 * quantized as in "Cactus Quants CQ2-bit Quantization: Extreme Compression
 * for Edge LLMs", section The CQ2-bit Implementation Pipeline).  At group
 * size 128: one launch for all the tensors whose cols is a multiple of G
 * plus one for the others, instead of one launch per tensor; at 32, 64 and
 * 256, cq_quantize's kernels once per tensor.  Results are identical to
 * cq_quantize on each tensor.  Pointing packed/norms at the offsets of cq_blob_layout writes
 * the serialized blob in place.  Every descriptor is validated as
 * cq_quantize validates its arguments (the first failing tensor is reported;
 * nothing is enqueued then); no output may overlap another output or any
 * input of the call (CQ_ERR_ARG).  Empty tensors are skipped.  At group
 * size 128 takes 48 bytes per tensor of stream-ordered device memory for
 * the descriptor table (hipMallocAsync / hipFreeAsync on `stream`). */
int cq_quantize_many(int n, const cq_quant_desc* descs, int w_dtype, int bits, int group_size,
                     const float* levels, int n_levels, void* stream);

/* One tensor of cq_dequantize_many (device pointers, layouts as
 * cq_dequantize). */
typedef struct {
  const uint8_t* packed;
  const uint16_t* norms;
  int64_t rows;
  int64_t cols;
  void* out;         /* rows x cols, the call's out_dtype */
} cq_dequant_desc;

/* cq_dequantize over n tensors (descs: host array) in one call, the inverse
 * of cq_quantize_many (for example all tensors of a serialized blob).  Same
 * launch structure, validation, overlap rule and workspace as
 * cq_quantize_many; results identical to cq_dequantize on each tensor. */
int cq_dequantize_many(int n, const cq_dequant_desc* descs, int bits, int group_size,
                       const float* levels, int n_levels, int out_dtype, void* stream);

/* Fake quantization: out = the reconstruction of w after quantization, in
 * one pass with no packed intermediate.  This is the quantize-then-rebuild
 * transform of "Cactus Quants CQ2-bit Quantization: Extreme Compression for
 * Edge LLMs", section The CQ2-bit Implementation Pipeline, and the forward
 * of its straight-through estimator (same page, section Training with
 * Quantization).  Indices are chosen exactly as cq_quantize chooses them;
 * the reconstruction is x_hat = (n / G) * H * levels[idx] with n the float32
 * group norm BEFORE binary16 rounding (so it differs from cq_dequantize of
 * cq_quantize's output by that rounding, at most 2^-11 relative per group).
 * w and out are rows x cols in w_dtype / out_dtype (CQ_F32 or CQ_BF16; bf16
 * output rounds to nearest even), both 16-byte aligned.  out == w with
 * w_dtype == out_dtype (in place) is allowed: every group is read in full
 * before it is written.  Any other overlap is CQ_ERR_ARG.  levels (host,
 * nullable: built-in table). */
int cq_fake_quant(const void* w, int w_dtype, int64_t rows, int64_t cols, int bits,
                  int group_size, const float* levels, int n_levels, void* out, int out_dtype,
                  void* stream);

/* y = x . W_hat^T for the quantized n_out x k matrix W (packed + norms as
 * produced by cq_quantize with rows = n_out, cols = k), x float32
 * [batch][k], y float32 [batch][n_out].  k must be a multiple of G
 * (CQ_ERR_UNSUPPORTED otherwise), batch >= 1.  The activations are rotated
 * once per group and dotted with the looked-up levels: because the
 * orthonormal Hadamard matrix is symmetric and its own inverse,
 * x_g . W_hat_g = (norm / G) * <H x_g, levels[idx]> with H the +-1
 * Sylvester-Hadamard matrix.  float32 accumulation in a fixed order
 * (deterministic).  One kernel launch (for batches up to 524,280 rows),
 * and no memory beyond the call's buffers: each thread block rotates the
 * activations it uses ("How Needle 2 Model Compresses to a Single Binary",
 * section Stage 3: the weights are decoded on the fly inside the product).
 * k <= 2^28 (CQ_ERR_UNSUPPORTED otherwise).  Results equal those of
 * cq_dequant_matvec_many on the same matrix to the product tolerance (the
 * two may sum in different orders). */
int cq_dequant_matvec(const uint8_t* packed, const uint16_t* norms, int64_t n_out,
                      int64_t k, int bits, int group_size, const float* levels,
                      int n_levels, const float* x, int64_t batch, float* y,
                      void* stream);

/* One matrix of cq_dequant_matvec_many (all pointers device pointers):
 * y [batch][n_out] = x [batch][k] . W_hat^T with W given by packed/norms as
 * cq_quantize produced them for rows = n_out, cols = k. */
typedef struct {
  const uint8_t* packed;
  const uint16_t* norms;
  int64_t n_out;
  int64_t k;
  const float* x;
  float* y;
} cq_matvec_desc;

/* cq_dequant_matvec for n matrices (descs: host array) that share bits,
 * levels and batch: the whole set runs as one activation-rotation launch and
 * one product launch per 8 batch rows (per batch row for large 2-bit calls
 * of 1 to 4 rows), e.g. every weight matrix of a model for one decode step
 * ("How Needle 2 Model Compresses to a Single Binary", section Stage 3: the
 * runtime decodes the packed tensors on the fly).  Each descriptor is
 * validated as cq_dequant_matvec validates its arguments (the first failing
 * one is reported; nothing is enqueued then).  Takes sum(batch*k)*4 bytes
 * of stream-ordered device memory for the rotated activations
 * (hipMallocAsync / hipFreeAsync on `stream`).  The device copy of the
 * descriptor table (about 80 bytes per matrix) is kept per (device, stream)
 * until the process ends: a later call on the same stream with the same
 * descriptors reuses it without an upload, and a call with other
 * descriptors rewrites it once the stream has passed the copy's last use.
 * Results are deterministic (fixed reduction order). */
int cq_dequant_matvec_many(int n, const cq_matvec_desc* descs, int bits, int group_size,
                           const float* levels, int n_levels, int64_t batch, void* stream);

/* cq_dequant_matvec_many for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, validation, kernels and results (bit for
 * bit), but the workspace lives in a fixed array of this library, 16 MiB
 * per GPU (held from the library's load until the process ends), and the
 * call allocates nothing.  The workspace a call needs is a descriptor table
 * of about 80 bytes per matrix plus sum(batch * k) * 4 bytes of rotated
 * activations (4.6 MB for the 225 matrices of a 7B-parameter model at
 * batch 1); a call that needs more than 16 MiB returns CQ_ERR_UNSUPPORTED
 * before anything is enqueued (use cq_dequant_matvec_many then).  Every
 * call on a GPU uses that GPU's one workspace: calls that overlap on the
 * same GPU (on different streams or host threads) race and must be
 * serialized by the caller; calls in order on one stream are safe. */
int cq_dequant_matvec_many_noalloc(int n, const cq_matvec_desc* descs, int bits, int group_size,
                                   const float* levels, int n_levels, int64_t batch, void* stream);

/* Batched product y = x . W_hat^T on the matrix cores, for the same inputs,
 * layouts, validation and workspace rules as cq_dequant_matvec (x float32
 * [batch][k], y float32 [batch][n_out], k a multiple of G), meant for larger
 * batches such as a prefill pass (the decode-time matvec is the batch-1 case;
 * "Performance Differences Between 2-Bit and 4-Bit Quantization in Needle",
 * section Practical Code Comparison, runs the quantized weights in an
 * ordinary forward product).  The activations are rotated once per group and
 * split into two bf16 halves (hi = bf16(v), lo = bf16(v - hi)); the levels
 * likewise; each product is taken as hi*hi + hi*lo + lo*hi by bf16 MFMAs with
 * float32 accumulation, then scaled by norm / G per (row, group).  Each
 * product is then within about 3 * 2^-16 of its float32 value, so
 * |y - exact| <= about 5e-5 * ||x_b|| * ||W_hat_n||.  Deterministic (fixed
 * order).  Workspace: 4 * batch * k bytes per matrix, with batch rounded up
 * to 32 (batches of at most 32) or 64, stream-ordered (hipMallocAsync /
 * hipFreeAsync on `stream`). */
int cq_dequant_gemm(const uint8_t* packed, const uint16_t* norms, int64_t n_out,
                    int64_t k, int bits, int group_size, const float* levels,
                    int n_levels, const float* x, int64_t batch, float* y,
                    void* stream);

/* cq_dequant_gemm for n matrices sharing bits, levels and batch (descs: host
 * array, as for cq_dequant_matvec_many): one rotation launch and one product
 * launch for the whole set.  No y may overlap another buffer of the call. */
int cq_dequant_gemm_many(int n, const cq_matvec_desc* descs, int bits, int group_size,
                         const float* levels, int n_levels, int64_t batch, void* stream);

/* Converts n_groups groups of three-level indices between the 2-bit field
 * form (CQ_TERNARY, G/4 bytes per group: 32 at G = 128, 16-byte aligned;
 * 4-byte aligned at other G) and trit storage (CQ_TERNARY_TRITS, ceil(G/5)
 * bytes per group: 26 at G = 128, 2-byte aligned; any alignment at other
 * G), in either direction (src_bits -> dst_bits; any other pair is
 * CQ_ERR_ARG), for group_size 32, 64, 128 or 256.  Lossless for indices
 * 0..2; a field holding 3 or a trit byte above 242 (neither is ever written
 * by cq_quantize) converts to unspecified in-range values.  src and dst must
 * not overlap. */
int cq_repack(const uint8_t* src, int src_bits, uint8_t* dst, int dst_bits, int64_t n_groups,
              int group_size, void* stream);

/* Static description of a status code. */
const char* cq_status_str(int status);

/* Thread-local detail message of the last failing call on this thread
 * ("" if none). */
const char* cq_last_error(void);

/* Library version string. */
const char* cq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBCQ_H */
