// cq_dequant_matvec_many_noalloc: the multi-matrix product with its
// workspace in a fixed device array of this library instead of memory
// allocated per call, for callers that cannot allocate (code under stream
// capture, tight serving loops).
//
// The workspace is the file-scope array `scratch` below, kScratchBytes per
// GPU, held from the library's load until the process ends.  In host code
// the array's name is only a stand-in for its device address: the device
// address is obtained once per device with hipGetSymbolAddress (with that
// device current) and kept in g_scratch; only that pointer is ever passed
// to kernels.  Every call on a GPU uses that GPU's copy, so calls that
// overlap on one GPU (different streams, or another host thread) race on
// it; each call writes all of the workspace it reads (the descriptor table
// and the rotated activations) before reading it, so nothing needs clearing.

#include <mutex>

#include "cq_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;  // 16 MiB per GPU
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint8_t* g_scratch[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up on first use.
int scratch_address(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return cq::report(CQ_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return cq::report(CQ_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return cq::report(CQ_ERR_HIP, "hipGetSymbolAddress of the fixed workspace failed");
    g_scratch[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch[dev];
  return CQ_OK;
}

}  // namespace

extern "C" int cq_dequant_matvec_many_noalloc(int n, const cq_matvec_desc* descs, int bits, int group_size,
                                              const float* levels, int n_levels, int64_t batch, void* stream) {
  // Validation and the workspace size check come first and need no device;
  // the address is looked up only for a call that will run.
  return cq::matvec_many_impl(n, descs, bits, group_size, levels, n_levels, batch, stream, scratch_address,
                              kScratchBytes);
}
