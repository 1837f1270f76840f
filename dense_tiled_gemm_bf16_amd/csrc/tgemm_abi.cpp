// C-ABI front end of libtgemm.so: argument validation, per-device set-up,
// error reporting and dispatch to the gfx950 kernels.
//
// The convention follows the host wrapper printed on the velog "tilelang"
// page (1.3 Code Generation & Runtime): an init step, a call that takes raw
// device pointers and a stream and returns 0 or a negative status, and a
// get-last-error string.  The argument checks mirror that page's Host
// IRModule (non-NULL data pointers, packed row-major strides, vectorised
// dimensions divisible by 8), but the sizes are runtime arguments here.
#include <hip/hip_runtime_api.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/tgemm.h"
#include "tgemm_internal.hpp"

namespace {

thread_local char g_err[1024];

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_dev_status[kMaxDevices];  // 0 ok, else TGEMM_EHIP
int g_dev_cus[kMaxDevices];     // compute units
char g_dev_msg[kMaxDevices][256];

// Tile override of this host thread (tgemm_set_tile); 0, 0 = automatic.
thread_local int g_tile_m = 0, g_tile_n = 0;

void init_device(int dev) {
  hipDeviceProp_t prop;
  hipError_t e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    g_dev_status[dev] = TGEMM_EHIP;
    snprintf(g_dev_msg[dev], sizeof g_dev_msg[dev], "hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
    return;
  }
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    g_dev_status[dev] = TGEMM_EHIP;
    snprintf(g_dev_msg[dev], sizeof g_dev_msg[dev], "device %d is %s; this library runs on gfx950 (MI355X) only",
             dev, prop.gcnArchName);
    return;
  }
  g_dev_cus[dev] = prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 256;
  // The no-allocation entry point's scratch: its device address on this
  // device (the device is current here).
  e = tgemm::scratch_init(dev);
  if (e != hipSuccess) {
    g_dev_status[dev] = TGEMM_EHIP;
    snprintf(g_dev_msg[dev], sizeof g_dev_msg[dev], "device %d: address of the scratch array: %s", dev,
             hipGetErrorString(e));
    return;
  }
  g_dev_status[dev] = TGEMM_OK;
}

// Current device, set up once.  Returns TGEMM_OK or TGEMM_EHIP (message set).
int ensure_device(int *cus = nullptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TGEMM_EHIP, "no usable HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TGEMM_EHIP, "device index %d out of range", dev);
  std::call_once(g_once[dev], init_device, dev);
  if (g_dev_status[dev] != TGEMM_OK) return fail(g_dev_status[dev], "%s", g_dev_msg[dev]);
  if (cus) *cus = g_dev_cus[dev];
  return TGEMM_OK;
}

bool overlaps(const void *p, uint64_t pn, const void *q, uint64_t qn) {
  if (!p || !q || pn == 0 || qn == 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + qn && b < a + pn;
}

bool misaligned(const void *p) { return ((uintptr_t)p & 15u) != 0; }

constexpr uint64_t kOffsetLimit = 0x7fffffffull;  // the kernels use 31-bit buffer offsets

// Bytes spanned by the K rows of a K-major 16-bit operand with row stride ld,
// K rounded up to whole slices of 64 rows.
uint64_t k_rows_bytes(int64_t K, int64_t ld) { return (uint64_t)(K + 63) / 64 * 64 * (uint64_t)ld * 2; }

struct Operand {
  const char *name;
  const void *ptr;
  uint64_t bytes;
  bool aligned16;  // must be 16-byte aligned
};

int check_common(const char *fn, int64_t M, int64_t N, int64_t K, int k_multiple, const Operand *ops, int nops,
                 const void *C, uint64_t c_bytes) {
  if (M < 0 || N < 0 || K < 0)
    return fail(TGEMM_EINVAL, "%s: negative size (M=%lld, N=%lld, K=%lld)", fn, (long long)M, (long long)N,
                (long long)K);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
    return fail(TGEMM_ETOOBIG, "%s: sizes must be below 2^31 (M=%lld, N=%lld, K=%lld)", fn, (long long)M,
                (long long)N, (long long)K);
  if (M == 0 || N == 0) return TGEMM_OK;
  if (K % k_multiple != 0)
    return fail(TGEMM_EALIGN, "%s: K=%lld must be a multiple of %d", fn, (long long)K, k_multiple);
  if (N % 8 != 0) return fail(TGEMM_EALIGN, "%s: N=%lld must be a multiple of 8", fn, (long long)N);
  if (!C) return fail(TGEMM_EINVAL, "%s: C is NULL", fn);
  if (misaligned(C)) return fail(TGEMM_EALIGN, "%s: C is not 16-byte aligned", fn);
  for (int i = 0; i < nops; ++i) {
    if (ops[i].bytes == 0) continue;  // an empty operand (K == 0) is never read
    if (!ops[i].ptr) return fail(TGEMM_EINVAL, "%s: %s is NULL", fn, ops[i].name);
    if (ops[i].aligned16 && misaligned(ops[i].ptr))
      return fail(TGEMM_EALIGN, "%s: %s is not 16-byte aligned", fn, ops[i].name);
    if (overlaps(C, c_bytes, ops[i].ptr, ops[i].bytes))
      return fail(TGEMM_EINVAL, "%s: C overlaps %s", fn, ops[i].name);
  }
  return TGEMM_OK;
}

int dispatch(const char *fn, tgemm::Problem p) {
  int rc = ensure_device(&p.cus);
  if (rc != TGEMM_OK) return rc;
  p.tile_m = g_tile_m;
  p.tile_n = g_tile_n;
  if (p.tile_m != 0 && !tgemm::shape_supported(p, p.tile_m, p.tile_n))
    return fail(TGEMM_EINVAL, "%s: no %dx%d tile for this entry point (set by tgemm_set_tile)", fn, p.tile_m,
                p.tile_n);
  hipError_t e = tgemm::launch(p);
  if (e == hipErrorInvalidConfiguration)
    return fail(TGEMM_ETOOBIG, "%s: a %lld x %lld output takes more tiles than one dispatch holds (2^24 workgroups)",
                fn, (long long)p.M, (long long)p.N);
  if (e != hipSuccess) return fail(TGEMM_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return TGEMM_OK;
}

// C = op(A) op(B) for 16-bit inputs with any operand storage and row
// strides (gemm_bf16 / gemm_f16).
int gemm_general(const char *fn, tgemm::Dt dt, int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                 const void *A, int64_t lda, const void *B, int64_t ldb, void *C, int64_t ldc, int splits, void *ws,
                 uint64_t ws_bytes, hipStream_t stream) {
  g_err[0] = '\0';
  if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1))
    return fail(TGEMM_EINVAL, "%s: trans_a and trans_b must be 0 or 1 (got %d, %d)", fn, trans_a, trans_b);
  if (M < 0 || N < 0 || K < 0)
    return fail(TGEMM_EINVAL, "%s: negative size (M=%lld, N=%lld, K=%lld)", fn, (long long)M, (long long)N,
                (long long)K);
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX || lda > INT32_MAX || ldb > INT32_MAX || ldc > INT32_MAX)
    return fail(TGEMM_ETOOBIG, "%s: sizes and strides must be below 2^31", fn);
  if (M == 0 || N == 0) return TGEMM_OK;
  // As stored: A is a_rows x a_cols, B is b_rows x b_cols.
  const int64_t a_rows = trans_a ? K : M, a_cols = trans_a ? M : K;
  const int64_t b_rows = trans_b ? N : K, b_cols = trans_b ? K : N;
  if (lda < a_cols)
    return fail(TGEMM_EINVAL, "%s: lda=%lld is below the stored row length of A (%lld)", fn, (long long)lda,
                (long long)a_cols);
  if (ldb < b_cols)
    return fail(TGEMM_EINVAL, "%s: ldb=%lld is below the stored row length of B (%lld)", fn, (long long)ldb,
                (long long)b_cols);
  if (ldc < N)
    return fail(TGEMM_EINVAL, "%s: ldc=%lld is below N=%lld", fn, (long long)ldc, (long long)N);
  if (a_cols % 8 != 0)
    return fail(TGEMM_EALIGN, "%s: %s=%lld (the contiguous dimension of A) must be a multiple of 8", fn,
                trans_a ? "M" : "K", (long long)a_cols);
  if (b_cols % 8 != 0)
    return fail(TGEMM_EALIGN, "%s: %s=%lld (the contiguous dimension of B) must be a multiple of 8", fn,
                trans_b ? "K" : "N", (long long)b_cols);
  if (N % 8 != 0) return fail(TGEMM_EALIGN, "%s: N=%lld must be a multiple of 8", fn, (long long)N);
  if (lda % 8 != 0 || ldb % 8 != 0 || ldc % 8 != 0)
    return fail(TGEMM_EALIGN, "%s: lda, ldb and ldc must be multiples of 8 (got %lld, %lld, %lld)", fn,
                (long long)lda, (long long)ldb, (long long)ldc);
  if (!C) return fail(TGEMM_EINVAL, "%s: C is NULL", fn);
  if (misaligned(C)) return fail(TGEMM_EALIGN, "%s: C is not 16-byte aligned", fn);
  // Bytes each operand spans (nothing is read when K == 0).
  const uint64_t a_bytes = K == 0 ? 0 : ((uint64_t)(a_rows - 1) * lda + a_cols) * 2;
  const uint64_t b_bytes = K == 0 ? 0 : ((uint64_t)(b_rows - 1) * ldb + b_cols) * 2;
  const uint64_t c_bytes = ((uint64_t)(M - 1) * ldc + N) * 2;
  const Operand ops[] = {{"A", A, a_bytes, true}, {"B", B, b_bytes, true}};
  for (const Operand &o : ops) {
    if (o.bytes == 0) continue;
    if (!o.ptr) return fail(TGEMM_EINVAL, "%s: %s is NULL", fn, o.name);
    if (misaligned(o.ptr)) return fail(TGEMM_EALIGN, "%s: %s is not 16-byte aligned", fn, o.name);
    if (overlaps(C, c_bytes, o.ptr, o.bytes)) return fail(TGEMM_EINVAL, "%s: C overlaps %s", fn, o.name);
  }
  // 31-bit buffer offsets: a K-contiguous operand is addressed per panel of
  // 256 rows, an M/N-contiguous one as a whole, in whole slices of 64 K rows
  // (the ragged last slice reads its rows past K as out of range).
  const uint64_t a_span = trans_a ? k_rows_bytes(K, lda) : (uint64_t)tgemm::kTileM * lda * 2;
  const uint64_t b_span = trans_b ? (uint64_t)tgemm::kTileN * ldb * 2 : k_rows_bytes(K, ldb);
  if (a_span > kOffsetLimit) return fail(TGEMM_ETOOBIG, "%s: A too large for 31-bit offsets", fn);
  if (b_span > kOffsetLimit) return fail(TGEMM_ETOOBIG, "%s: B too large for 31-bit offsets", fn);
  if (splits < 0 || splits > tgemm::kMaxSplits)
    return fail(TGEMM_EINVAL, "%s: splits=%d must be 0 (automatic) or 1 .. %d", fn, splits, tgemm::kMaxSplits);
  if (splits != 1) {
    // The workspace: fp32 partial sums, one M x N plane per split.
    const uint64_t plane = (uint64_t)M * (uint64_t)N * 4u;
    if (!ws && ws_bytes > 0) return fail(TGEMM_EINVAL, "%s: workspace is NULL", fn);
    if (ws && misaligned(ws)) return fail(TGEMM_EALIGN, "%s: workspace is not 16-byte aligned", fn);
    if (splits >= 2 && ws_bytes < (uint64_t)splits * plane)
      return fail(TGEMM_EINVAL, "%s: %d splits of a %lld x %lld output need %llu workspace bytes, got %llu", fn,
                  splits, (long long)M, (long long)N, (unsigned long long)((uint64_t)splits * plane),
                  (unsigned long long)ws_bytes);
    // The part of the workspace a call may write: what its splits need.
    const uint64_t most = (uint64_t)(splits == 0 ? tgemm::kAutoMaxSplits : splits) * plane;
    const uint64_t used = ws_bytes < most ? ws_bytes : most;
    for (const Operand &o : ops)
      if (overlaps(ws, used, o.ptr, o.bytes)) return fail(TGEMM_EINVAL, "%s: workspace overlaps %s", fn, o.name);
    if (overlaps(ws, used, C, c_bytes)) return fail(TGEMM_EINVAL, "%s: workspace overlaps C", fn);
  }
  tgemm::Problem p{dt, trans_a == 1, trans_b == 1, M, N, K, A, lda, B, ldb, nullptr, nullptr, C, ldc, stream,
                   0, 0, 0, splits, splits == 1 ? nullptr : ws, splits == 1 ? 0 : ws_bytes};
  return dispatch(fn, p);
}

}  // namespace

extern "C" {

int tgemm_init(void) {
  g_err[0] = '\0';
  return ensure_device();
}

const char *tgemm_last_error(void) { return g_err; }

int gemm_mxfp4_nt(int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *scale_A,
                  const void *scale_B, void *C, hipStream_t stream) {
  static const char fn[] = "gemm_mxfp4_nt";
  g_err[0] = '\0';
  const uint64_t m = M > 0 ? (uint64_t)M : 0, n = N > 0 ? (uint64_t)N : 0, k = K > 0 ? (uint64_t)K : 0;
  const uint64_t kb = (k + 31) / 32;
  const Operand ops[] = {{"A", A, m * k / 2, true},
                         {"B", B, n * k / 2, true},
                         {"scale_A", scale_A, m * kb, false},
                         {"scale_B", scale_B, n * kb, false}};
  int rc = check_common(fn, M, N, K, 32, ops, 4, C, m * n * 2);
  if (rc != TGEMM_OK || M == 0 || N == 0) return rc;
  if ((uint64_t)tgemm::kTileM * k / 2 > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: K=%lld too large (256 * K / 2 bytes must stay below 2^31)", fn, (long long)K);
  if (m * kb > kOffsetLimit || n * kb > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: scale arrays too large", fn);
  tgemm::Problem p{tgemm::Dt::kMxfp4, false, true, M, N, K, A, K / 2, B, K / 2, scale_A, scale_B, C, N, stream,
                   0, 0, 0, 1, nullptr, 0};
  return dispatch(fn, p);
}

int gemm_mxfp6_nt(int fmt, int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *scale_A,
                  const void *scale_B, void *C, hipStream_t stream) {
  static const char fn[] = "gemm_mxfp6_nt";
  g_err[0] = '\0';
  if (fmt != TGEMM_FP6_E2M3 && fmt != TGEMM_FP6_E3M2)
    return fail(TGEMM_EINVAL, "%s: fmt=%d must be TGEMM_FP6_E2M3 (0) or TGEMM_FP6_E3M2 (1)", fn, fmt);
  const uint64_t m = M > 0 ? (uint64_t)M : 0, n = N > 0 ? (uint64_t)N : 0, k = K > 0 ? (uint64_t)K : 0;
  const uint64_t kb = (k + 31) / 32, row = k / 4 * 3;
  const Operand ops[] = {{"A", A, m * row, true},
                         {"B", B, n * row, true},
                         {"scale_A", scale_A, m * kb, false},
                         {"scale_B", scale_B, n * kb, false}};
  int rc = check_common(fn, M, N, K, 64, ops, 4, C, m * n * 2);
  if (rc != TGEMM_OK || M == 0 || N == 0) return rc;
  if ((uint64_t)tgemm::kTileM * row > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: K=%lld too large (256 * 3K/4 bytes must stay below 2^31)", fn, (long long)K);
  if (m * kb > kOffsetLimit || n * kb > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: scale arrays too large", fn);
  const tgemm::Dt dt = fmt == TGEMM_FP6_E2M3 ? tgemm::Dt::kMxfp6E2M3 : tgemm::Dt::kMxfp6E3M2;
  tgemm::Problem p{dt, false, true, M, N, K, A, K / 4 * 3, B, K / 4 * 3, scale_A, scale_B, C, N, stream, 0, 0, 0, 1, nullptr, 0};
  return dispatch(fn, p);
}

int gemm_bf16(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
              const void *B, int64_t ldb, void *C, int64_t ldc, hipStream_t stream) {
  return gemm_general("gemm_bf16", tgemm::Dt::kBf16, trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, 1, nullptr,
                      0, stream);
}

int gemm_f16(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
             const void *B, int64_t ldb, void *C, int64_t ldc, hipStream_t stream) {
  return gemm_general("gemm_f16", tgemm::Dt::kF16, trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, 1, nullptr, 0,
                      stream);
}

int gemm_bf16_splitk(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                     const void *B, int64_t ldb, void *C, int64_t ldc, int splits, void *workspace,
                     uint64_t workspace_bytes, hipStream_t stream) {
  return gemm_general("gemm_bf16_splitk", tgemm::Dt::kBf16, trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc,
                      splits, workspace, workspace_bytes, stream);
}

int gemm_f16_splitk(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                    const void *B, int64_t ldb, void *C, int64_t ldc, int splits, void *workspace,
                    uint64_t workspace_bytes, hipStream_t stream) {
  return gemm_general("gemm_f16_splitk", tgemm::Dt::kF16, trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, splits,
                      workspace, workspace_bytes, stream);
}

int gemm_bf16_splitk_noalloc(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                             const void *B, int64_t ldb, void *C, int64_t ldc, int splits, hipStream_t stream) {
  static const char fn[] = "gemm_bf16_splitk_noalloc";
  g_err[0] = '\0';
  if (splits >= 2 && M > 0 && N > 0 &&
      (uint64_t)splits * (uint64_t)M * (uint64_t)N * 4u > tgemm::kScratchBytes)
    return fail(TGEMM_ETOOBIG, "%s: %d splits of a %lld x %lld output need %llu bytes of scratch; it holds %llu", fn,
                splits, (long long)M, (long long)N,
                (unsigned long long)((uint64_t)splits * (uint64_t)M * (uint64_t)N * 4u),
                (unsigned long long)tgemm::kScratchBytes);
  int dev = -1;
  void *ws = nullptr;
  if (splits != 1 && M > 0 && N > 0) {
    // Set up the device first (scratch_init runs there), then take its
    // copy's address; never the array's host-side name.
    int rc = ensure_device();
    if (rc != TGEMM_OK) return rc;
    if (hipGetDevice(&dev) != hipSuccess || !(ws = tgemm::scratch_ptr(dev)))
      return fail(TGEMM_EHIP, "%s: no scratch address for the current device", fn);
  }
  return gemm_general(fn, tgemm::Dt::kBf16, trans_a, trans_b, M, N, K, A, lda, B, ldb, C, ldc, splits, ws,
                      ws ? tgemm::kScratchBytes : 0, stream);
}

uint64_t tgemm_splitk_workspace_bytes(int64_t M, int64_t N, int splits) {
  if (M <= 0 || N <= 0 || splits < 0 || splits > tgemm::kMaxSplits) return 0;
  const int s = splits == 0 ? tgemm::kAutoMaxSplits : splits == 1 ? 0 : splits;
  return (uint64_t)s * (uint64_t)M * (uint64_t)N * 4u;
}

int quantize_mxfp8(int64_t M, int64_t K, const float *x, void *q, void *scales, hipStream_t stream) {
  static const char fn[] = "quantize_mxfp8";
  g_err[0] = '\0';
  if (M < 0 || K < 0)
    return fail(TGEMM_EINVAL, "%s: negative size (M=%lld, K=%lld)", fn, (long long)M, (long long)K);
  if (M > INT32_MAX || K > INT32_MAX)
    return fail(TGEMM_ETOOBIG, "%s: sizes must be below 2^31 (M=%lld, K=%lld)", fn, (long long)M, (long long)K);
  if (M == 0 || K == 0) return TGEMM_OK;
  if (K % 16 != 0) return fail(TGEMM_EALIGN, "%s: K=%lld must be a multiple of 16", fn, (long long)K);
  const uint64_t n = (uint64_t)M * (uint64_t)K, kb = ((uint64_t)K + 127) / 128;
  if (!x) return fail(TGEMM_EINVAL, "%s: x is NULL", fn);
  if (!q) return fail(TGEMM_EINVAL, "%s: q is NULL", fn);
  if (!scales) return fail(TGEMM_EINVAL, "%s: scales is NULL", fn);
  if (misaligned(x)) return fail(TGEMM_EALIGN, "%s: x is not 16-byte aligned", fn);
  if (misaligned(q)) return fail(TGEMM_EALIGN, "%s: q is not 16-byte aligned", fn);
  if (overlaps(q, n, x, n * 4)) return fail(TGEMM_EINVAL, "%s: q overlaps x", fn);
  if (overlaps(scales, (uint64_t)M * kb, x, n * 4)) return fail(TGEMM_EINVAL, "%s: scales overlaps x", fn);
  if (overlaps(scales, (uint64_t)M * kb, q, n)) return fail(TGEMM_EINVAL, "%s: scales overlaps q", fn);
  int rc = ensure_device();
  if (rc != TGEMM_OK) return rc;
  tgemm::QuantProblem p{M, K, x, q, scales, stream};
  hipError_t e = tgemm::launch_quantize(p);
  if (e != hipSuccess) return fail(TGEMM_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return TGEMM_OK;
}

int tgemm_clock_probe(void *out, int *wallclock_khz, hipStream_t stream) {
  static const char fn[] = "tgemm_clock_probe";
  g_err[0] = '\0';
  if (!out) return fail(TGEMM_EINVAL, "%s: out is NULL", fn);
  if (misaligned(out)) return fail(TGEMM_EALIGN, "%s: out is not 16-byte aligned", fn);
  int rc = ensure_device();
  if (rc != TGEMM_OK) return rc;
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return fail(TGEMM_EHIP, "%s: wall-clock rate: %s", fn, hipGetErrorString(e));
  if (khz <= 0) return fail(TGEMM_EHIP, "%s: the device reports no constant-rate counter", fn);
  if (wallclock_khz) *wallclock_khz = khz;
  e = tgemm::launch_clock_probe(out, stream);
  if (e != hipSuccess) return fail(TGEMM_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return TGEMM_OK;
}

int tgemm_set_tile(int tile_m, int tile_n) {
  g_err[0] = '\0';
  const bool known = (tile_m == 0 && tile_n == 0) || (tile_m == 256 && tile_n == 256) ||
                     (tile_m == 256 && tile_n == 192) || (tile_m == 128 && tile_n == 128) ||
                     (tile_m == 64 && tile_n == 64);
  if (!known) return fail(TGEMM_EINVAL, "tgemm_set_tile: no %dx%d tile (256x256, 256x192, 128x128, 64x64 or 0x0)", tile_m, tile_n);
  g_tile_m = tile_m;
  g_tile_n = tile_n;
  return TGEMM_OK;
}

int gemm_bf16_nt(int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C, hipStream_t stream) {
  static const char fn[] = "gemm_bf16_nt";
  g_err[0] = '\0';
  const uint64_t m = M > 0 ? (uint64_t)M : 0, n = N > 0 ? (uint64_t)N : 0, k = K > 0 ? (uint64_t)K : 0;
  const Operand ops[] = {{"A", A, m * k * 2, true}, {"B", B, n * k * 2, true}};
  int rc = check_common(fn, M, N, K, 8, ops, 2, C, m * n * 2);
  if (rc != TGEMM_OK || M == 0 || N == 0) return rc;
  if ((uint64_t)tgemm::kTileM * k * 2 > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: K=%lld too large (256 * K * 2 bytes must stay below 2^31)", fn, (long long)K);
  tgemm::Problem p{tgemm::Dt::kBf16, false, true, M, N, K, A, K, B, K, nullptr, nullptr, C, N, stream, 0, 0, 0, 1, nullptr, 0};
  return dispatch(fn, p);
}

int gemm_f16_nn(int64_t M, int64_t N, int64_t K, const void *A, const void *B, void *C, hipStream_t stream) {
  static const char fn[] = "gemm_f16_nn";
  g_err[0] = '\0';
  const uint64_t m = M > 0 ? (uint64_t)M : 0, n = N > 0 ? (uint64_t)N : 0, k = K > 0 ? (uint64_t)K : 0;
  const Operand ops[] = {{"A", A, m * k * 2, true}, {"B", B, k * n * 2, true}};
  int rc = check_common(fn, M, N, K, 8, ops, 2, C, m * n * 2);
  if (rc != TGEMM_OK || M == 0 || N == 0) return rc;
  if ((uint64_t)tgemm::kTileM * k * 2 > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: K=%lld too large (256 * K * 2 bytes must stay below 2^31)", fn, (long long)K);
  if (k_rows_bytes(K, N) > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: B too large (K * N * 2 bytes, K rounded up to 64, must stay below 2^31)", fn);
  tgemm::Problem p{tgemm::Dt::kF16, false, false, M, N, K, A, K, B, N, nullptr, nullptr, C, N, stream, 0, 0, 0, 1, nullptr, 0};
  return dispatch(fn, p);
}

int gemm_mxfp8_nt(int64_t M, int64_t N, int64_t K, const void *A, const void *B, const void *scale_A,
                  const void *scale_B, void *C, hipStream_t stream) {
  static const char fn[] = "gemm_mxfp8_nt";
  g_err[0] = '\0';
  const uint64_t m = M > 0 ? (uint64_t)M : 0, n = N > 0 ? (uint64_t)N : 0, k = K > 0 ? (uint64_t)K : 0;
  const uint64_t kb = (k + 127) / 128;
  const Operand ops[] = {{"A", A, m * k, true},
                         {"B", B, n * k, true},
                         {"scale_A", scale_A, m * kb, false},
                         {"scale_B", scale_B, n * kb, false}};
  int rc = check_common(fn, M, N, K, 16, ops, 4, C, m * n * 2);
  if (rc != TGEMM_OK || M == 0 || N == 0) return rc;
  if ((uint64_t)tgemm::kTileM * k > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: K=%lld too large (256 * K bytes must stay below 2^31)", fn, (long long)K);
  if (m * kb > kOffsetLimit || n * kb > kOffsetLimit)
    return fail(TGEMM_ETOOBIG, "%s: scale arrays too large", fn);
  tgemm::Problem p{tgemm::Dt::kMxfp8, false, true, M, N, K, A, K, B, K, scale_A, scale_B, C, N, stream, 0, 0, 0, 1, nullptr, 0};
  return dispatch(fn, p);
}

}  // extern "C"
