// Shader-clock probe for measurements (not on the GEMM path).
//
// The pages time their kernel and turn the latency into TFLOPS = 2 M N K / t
// (TileLang SM100 README, "Compilation and Usage").  On MI355X the time of a
// dense GEMM also depends on the shader clock, which the board's power limit
// moves with the data and with how long the chip has been busy.  The probe
// has one single-wave workgroup per CU read that CU's shader-clock counter
// (s_memtime) and the constant-rate counter (s_memrealtime), and records
// which CU it ran on.  Each CU keeps a counter of its own (they differ by
// millions of ticks within one XCD), so a probe before and one after a timed
// region give the clock each CU delivered over it only when their records
// are paired by CU: (difference of the shader-clock counts) / (difference of
// the constant-rate counts) times the constant rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm_internal.hpp"

namespace tgemm {
namespace {

// One wave per workgroup; workgroup w writes record w: {XCC id << 32 |
// HW_ID (bits 8-15: CU, shader array and shader engine), shader-clock count,
// constant-rate count, 0}.  kProbeGroups workgroups, as many as the CUs; the
// records say where each ran.
__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t *out) {
  if (threadIdx.x == 0) {
    const uint32_t hw = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));    // HW_REG_HW_ID, all 32 bits
    const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11));  // HW_REG_XCC_ID, bits 0-15
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    uint64_t *o = out + 4 * blockIdx.x;
    o[0] = ((uint64_t)(xcc & 15u) << 32) | hw;
    o[1] = t;
    o[2] = r;
    o[3] = 0;
  }
}

}  // namespace

hipError_t launch_clock_probe(void *out, hipStream_t stream) {
  uint64_t *o = static_cast<uint64_t *>(out);
  void *args[] = {&o};
  return hipLaunchKernel(reinterpret_cast<const void *>(&clock_probe_kernel), dim3(kProbeGroups), dim3(64), args, 0,
                         stream);
}

}  // namespace tgemm
