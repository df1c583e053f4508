// Static device scratch of mla_attend_noalloc: the attention workspace of
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array lives in the library's code object, so every GPU the library runs
// on holds its own copy (at its own address) until the process ends.  In host
// code the array's name is only a stand-in for the device symbol: its address
// on the current device is looked up once per device with hipGetSymbolAddress
// and that pointer, never the name, is what kernels and copies receive.  No
// part of the attention needs the scratch to start zeroed (every byte a
// kernel reads was written earlier in the same call), and every call on one
// GPU shares the array: calls that overlap in time on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mla_launch.h"

static __device__ __align__(256) unsigned char scratch[mla::kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

namespace mla {

hipError_t scratch_for_current_device(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
