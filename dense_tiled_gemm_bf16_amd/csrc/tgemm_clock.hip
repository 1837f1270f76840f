// Shader-clock probe for measurements (not on the GEMM path).
//
// The pages time their kernel and turn the latency into TFLOPS = 2 M N K / t
// (TileLang SM100 README, "Compilation and Usage").  On MI355X the time of a
// dense GEMM also depends on the shader clock, which the board's power limit
// moves with the data and with how long the chip has been busy.  The probe
// reads, on each XCD, the shader-clock counter (s_memtime) and the
// constant-rate counter (s_memrealtime), then spins for a fixed number of
// constant-rate ticks and reads both again: the ratio of the two differences
// over that spin, times the constant rate, is the XCD's clock at that moment
// (measured within one kernel; differences of the shader-clock counter taken
// across kernels are not reliable while the clock is changing).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm_internal.hpp"

namespace tgemm {
namespace {

// One wave per workgroup; workgroup w writes record w: {XCC id, shader-clock
// count, constant-rate count, (constant-rate ticks of the spin) << 32 |
// (shader-clock ticks of the spin)}, the counts read at the start of the
// spin.  Consecutive workgroups go to the XCDs in turn, so kProbeGroups of
// them sample every XCD; each record says which.  The spin ends after
// `ticks` constant-rate ticks, or after a bounded number of reads.
__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t *out, uint32_t ticks) {
  if (threadIdx.x == 0) {
    const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11));  // HW_REG_XCC_ID, bits 0-15
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    uint64_t r1 = r0;
    for (int i = 0; i < (1 << 20) && r1 - r0 < ticks; ++i) r1 = __builtin_amdgcn_s_memrealtime();
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    uint64_t *o = out + 4 * blockIdx.x;
    o[0] = xcc & 15u;
    o[1] = t0;
    o[2] = r0;
    o[3] = ((r1 - r0) << 32) | ((t1 - t0) & 0xffffffffull);
  }
}

}  // namespace

hipError_t launch_clock_probe(void *out, uint32_t ticks, hipStream_t stream) {
  uint64_t *o = static_cast<uint64_t *>(out);
  void *args[] = {&o, &ticks};
  return hipLaunchKernel(reinterpret_cast<const void *>(&clock_probe_kernel), dim3(kProbeGroups), dim3(64), args, 0,
                         stream);
}

}  // namespace tgemm
