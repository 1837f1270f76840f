// Block-scale quantiser for gfx950: binary32 rows -> OCP e4m3fn elements and
// one e8m0 scale per row per 128 K elements, the operand format of the
// block-scaled GEMM (scale granularity 128 along K: Blackwell TCGEN05 GEMM
// tutorial, section "进阶" (Advanced)).
//
// Per block the scale 2^e is the smallest power of two with
// absmax <= 448 * 2^e (448 = largest e4m3fn), e clamped to [-127, 127] and
// -127 for an all-zero block, stored as the byte e + 127; each element is
// x * 2^-e rounded once to e4m3fn, ties to even.
//
// The work is a streaming pass (4 bytes read and 1 written per element), so
// the layout is chosen for coalescing, not arithmetic: lane l of a wave
// takes 8 consecutive elements (two 16-byte loads), 16 lanes cover one
// 128-element block, a wave covers 4 blocks (2 KiB of one row, read as one
// contiguous span), and a workgroup 4 such segments.  The block maximum is a
// 16-lane butterfly; the exponent comes from frexp of that maximum, the
// scaling is an exact ldexp, and the conversion is the hardware's
// round-to-nearest fp32 -> fp8 pair conversion.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tgemm_internal.hpp"

namespace tgemm {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kQThreads = 256;
constexpr int kSegElems = 512;  // elements per wave: 4 blocks of 128
constexpr int kSegsPerWg = kQThreads / 64;

struct QArgs {
  const float *x;
  uint8_t *q;
  uint8_t *s;
  int64_t M, K;
  int64_t kb;      // scale blocks per row
  int64_t segs_per_row;
  int64_t segs;    // M * segs_per_row
};

__global__ __launch_bounds__(kQThreads) void quantize_mxfp8_kernel(const QArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t seg = (int64_t)blockIdx.x * kSegsPerWg + (threadIdx.x >> 6);
  if (seg >= a.segs) return;  // whole wave: seg is uniform across it
  const int64_t row = seg / a.segs_per_row;
  const int64_t k0 = (seg - row * a.segs_per_row) * kSegElems + lane * 8;
  const bool valid = k0 < a.K;  // K % 8 == 0: a lane's 8 elements are all in or all out

  float v[8];
  if (valid) {
    const f32x4 *p = (const f32x4 *)(a.x + row * a.K + k0);
    const f32x4 lo = p[0], hi = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = lo[i];
      v[4 + i] = hi[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }

  // Block maximum of |x| over the 16 lanes of this lane's block.
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 16));

  // Smallest e with m <= 448 * 2^e: m = f * 2^e2 with f in [0.5, 1), and
  // m / 2^(e2 - 9) = 512 f lies in [256, 512), within 448 iff f <= 0.875.
  int e;
  if (m == 0.0f) {
    e = -127;
  } else {
    int e2;
    const float f = frexpf(m, &e2);
    e = e2 - 9 + (f > 0.875f ? 1 : 0);
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }

  if (valid) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int pk = 0;
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * h + 0], -e), ldexpf(v[4 * h + 1], -e), pk, false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[4 * h + 2], -e), ldexpf(v[4 * h + 3], -e), pk, true);
      w[h] = (uint32_t)pk;
    }
    *(u32x2 *)(a.q + row * a.K + k0) = u32x2{w[0], w[1]};
    if ((lane & 15) == 0) a.s[row * a.kb + k0 / 128] = (uint8_t)(e + 127);
  }
}

}  // namespace

hipError_t launch_quantize(const QuantProblem &p) {
  QArgs a;
  a.x = static_cast<const float *>(p.x);
  a.q = static_cast<uint8_t *>(p.q);
  a.s = static_cast<uint8_t *>(p.scales);
  a.M = p.M;
  a.K = p.K;
  a.kb = (p.K + 127) / 128;
  a.segs_per_row = (p.K + kSegElems - 1) / kSegElems;
  a.segs = p.M * a.segs_per_row;
  const int64_t wgs = (a.segs + kSegsPerWg - 1) / kSegsPerWg;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  void *args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void *>(&quantize_mxfp8_kernel), dim3((unsigned)wgs),
                         dim3(kQThreads), args, 0, p.stream);
}

}  // namespace tgemm
