// Device scratch for the entry point that allocates nothing
// (gemm_bf16_splitk_noalloc): the K split's fp32 partial sums live in a
// file-scope device array instead of a caller's workspace.  Each GPU the
// library runs on holds its own copy of the array until the process ends;
// calls on one GPU share it, so calls that overlap on one GPU race.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "tgemm_internal.hpp"

namespace tgemm {
namespace {

// Host code must not pass `scratch` itself to a kernel or a copy: on the
// host the name stands for a host-side shadow, not the device memory.  Use
// the address scratch_init() fetched for the device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::once_flag g_once[kMaxScratchDevices];
hipError_t g_status[kMaxScratchDevices];
void *g_ptr[kMaxScratchDevices];

}  // namespace

hipError_t scratch_init(int dev) {
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  return g_status[dev];
}

void *scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxScratchDevices) return nullptr;
  return g_ptr[dev];
}

}  // namespace tgemm
