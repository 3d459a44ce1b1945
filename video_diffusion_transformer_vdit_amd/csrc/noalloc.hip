// Device scratch of the allocation-free fp8 pre-pass entry point
// (vdit_attn_quant_fp8_noalloc).
//
// The pre-pass keeps per-block V statistics (and, with one K mean per head,
// K partial sums) between its three launches.  vdit_attn_quant_fp8 takes that
// scratch as a caller-owned workspace; the allocation-free entry point uses
// this file-scope array instead, for callers that cannot allocate (code
// under graph capture, tight serving loops).  Each GPU the library runs on
// holds its own copy at its own address until the process ends.  In host
// code the name `scratch` is only a host-side stand-in, so the device address
// is looked up once per device with hipGetSymbolAddress and only that
// address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launchers.h"

// Sized for the pre-pass of the 720p workload (40 heads x 75,600 tokens,
// one K mean per 64-token block: 96.9 MB); 0.05% of an MI355X's 288 GB.
static constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace vdit {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (stream != nullptr) {
    // the array's address belongs to the current device; the stream must too
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace vdit
