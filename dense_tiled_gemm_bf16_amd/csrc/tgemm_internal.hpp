// Internal interface between the C-ABI front end (tgemm_abi.cpp) and the
// gfx950 kernels (tgemm_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tgemm {

// Element type of A and B (C is bf16, or fp16 for fp16 inputs).
enum class Dt : int { kBf16 = 0, kF16 = 1, kMxfp8 = 2, kMxfp4 = 3, kMxfp6E2M3 = 4, kMxfp6E3M2 = 5 };

// A validated problem, C = op(A) op(B): sizes are non-negative and fit the
// kernels' limits, pointers and row strides are aligned, M > 0 and N > 0.
struct Problem {
  Dt dt;
  bool trans_a;  // A is stored K x M (op(A) = A^T); else M x K
  bool trans_b;  // B is stored N x K (op(B) = B^T); else K x N
  int64_t M, N, K;
  const void *A;
  int64_t lda;  // row stride of A as stored, in elements
  const void *B;
  int64_t ldb;
  const void *scale_A, *scale_B;  // mxfp8 only
  void *C;
  int64_t ldc;
  hipStream_t stream;
  int cus;             // compute units of the device
  int tile_m, tile_n;  // forced output tile, or 0, 0 to choose by shape
  // K split (16-bit kinds): 1 = none; 0 = the library chooses (at most what
  // ws_bytes holds); >= 2 = that many (at most one per 64-element K slice).
  // ws: fp32 workspace of ws_bytes bytes (16-byte aligned) for the partial
  // sums, splits planes of M x N.
  int splits;
  void *ws;
  uint64_t ws_bytes;
};

// Most K splits of one call, and of an automatic choice.
constexpr int kMaxSplits = 16;
constexpr int kAutoMaxSplits = 4;

// Largest output tile of one workgroup (rows of C x columns of C).
constexpr int kTileM = 256;
constexpr int kTileN = 256;

// Enqueues the kernel for `p` on p.stream.  Returns the launch status
// (hipErrorInvalidValue for a forced tile the kind does not have).
hipError_t launch(const Problem &p);

// Whether p's element type and layout have a kernel for tile_m x tile_n tiles.
bool shape_supported(const Problem &p, int tile_m, int tile_n);

// A validated block-scale quantisation: M, K > 0, K % 16 == 0, x and q
// 16-byte aligned.
struct QuantProblem {
  int64_t M, K;
  const void *x;  // M x K binary32
  void *q;        // M x K e4m3fn bytes
  void *scales;   // M x ceil(K/128) e8m0 bytes
  hipStream_t stream;
};

// Enqueues the quantiser for `p` on p.stream.  Returns the launch status.
hipError_t launch_quantize(const QuantProblem &p);

// Device scratch of the no-allocation K split (tgemm_scratch.hip): bytes
// per device, and the devices it is set up for.
constexpr uint64_t kScratchBytes = 8ull << 20;
constexpr int kMaxScratchDevices = 64;

// With `dev` current: fetch the device address of dev's copy of the scratch
// array (once per device; later calls return the first status).
hipError_t scratch_init(int dev);

// That address (nullptr until scratch_init(dev) has succeeded).
void *scratch_ptr(int dev);

// Workgroups of the clock probe: one per CU of an MI355X (8 XCDs x 32).
constexpr int kProbeGroups = 256;

// Enqueues the clock probe on `stream`: writes kProbeGroups records of four
// uint64 {XCC id << 32 | HW_ID, s_memtime, s_memrealtime, 0} to the device
// buffer `out`.
hipError_t launch_clock_probe(void *out, hipStream_t stream);

}  // namespace tgemm
