// Host-to-device copies of small tables (descriptor tables, prefix sums) as
// kernel arguments.  A kernel launch copies its argument block when it is
// enqueued, so the copy is stream-ordered and asynchronous without pinned
// staging memory, and the caller's host buffer is free once the call returns.

#include "cq_internal.h"

namespace cq {
namespace {

constexpr int kUploadWords = 1016;  // 4,064 bytes per launch (the argument block holds 4 KiB)

struct UploadChunk {
  uint32_t w[kUploadWords];
  uint32_t n_words;
};
static_assert(sizeof(UploadChunk) <= 4096, "kernel arguments stay within 4 KiB");

__global__ void __launch_bounds__(256) upload_kernel(UploadChunk c, uint32_t* __restrict__ dst) {
  for (uint32_t i = threadIdx.x; i < c.n_words; i += blockDim.x) dst[i] = c.w[i];
}

}  // namespace

hipError_t upload(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  if (bytes % 4) return hipErrorInvalidValue;
  const uint32_t* s = static_cast<const uint32_t*>(src);
  uint32_t* d = static_cast<uint32_t*>(dst);
  size_t words = bytes / 4;
  while (words > 0) {
    UploadChunk c{};
    c.n_words = static_cast<uint32_t>(words < kUploadWords ? words : kUploadWords);
    for (uint32_t i = 0; i < c.n_words; ++i) c.w[i] = s[i];
    hipLaunchKernelGGL(upload_kernel, dim3(1), dim3(256), 0, stream, c, d);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    s += c.n_words;
    d += c.n_words;
    words -= c.n_words;
  }
  return hipSuccess;
}

}  // namespace cq
