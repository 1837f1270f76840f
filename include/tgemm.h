/*
 * tgemm -- tiled dense GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the library libtgemm.so.  Every entry point takes the problem
 * sizes, plain device pointers and a HIP stream; none takes a framework
 * type.  All matrices are row-major and packed (leading dimension = number
 * of columns), as in the lowered kernel of the velog "tilelang" page
 * (1.2 Pass Pipeline, Host IRModule: strides (K, 1) with byte offset 0).
 *
 * Ownership: the caller owns and allocates every buffer.  The library keeps
 * no per-call state, allocates no device memory and never synchronises: an
 * entry point validates its arguments, enqueues one kernel on `stream`
 * (NULL = the null stream) and returns.  Errors that happen on the device
 * after the enqueue surface at the caller's next synchronisation.
 *
 * Return values (shared by all entry points):
 *   TGEMM_OK          0   success (or nothing to do: M == 0 or N == 0)
 *   TGEMM_EINVAL     -1   negative size, NULL pointer for a non-empty
 *                         operand, or C overlapping an input buffer
 *   TGEMM_EALIGN     -2   a pointer not 16-byte aligned, or a size that
 *                         breaks the vector width (see each entry point)
 *   TGEMM_ETOOBIG    -3   an operand larger than the kernels' 32-bit
 *                         buffer offsets can address (see each entry point),
 *                         or an output of more tiles than one dispatch
 *                         holds (2^24 workgroups of 256 work-items)
 *   TGEMM_EHIP       -4   no usable gfx950 device, or a HIP error at
 *                         initialisation or launch
 * After a non-zero return, tgemm_last_error() describes the failure.
 *
 * Thread safety: entry points may be called from several host threads; the
 * error message is kept per thread.  Calls on one stream run in order.
 */
#ifndef TGEMM_H
#define TGEMM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define TGEMM_API __attribute__((visibility("default")))
#else
#define TGEMM_API
#endif

#define TGEMM_OK 0
#define TGEMM_EINVAL (-1)
#define TGEMM_EALIGN (-2)
#define TGEMM_ETOOBIG (-3)
#define TGEMM_EHIP (-4)

/*
 * C = A . B^T  ("NT"), bfloat16 in, fp32 accumulation, bfloat16 out.
 *
 * Defined by the TileLang SM100 README, "Code Example": A is (M, K), B is
 * (N, K), the product uses trans_B = True, the accumulator is "float" and C
 * is (M, N) bfloat16.
 *
 *   A  device pointer, M x K bf16, row-major (row stride K elements)
 *   B  device pointer, N x K bf16, row-major
 *   C  device pointer, M x N bf16, row-major; written, never read
 *
 * Each output is the fp32 sum over k of A[m][k] * B[n][k] (summation order
 * unspecified), rounded to nearest-even bf16.  K == 0 writes zeros.
 * Requirements: K % 8 == 0 and N % 8 == 0 (vector width, as in the lowered
 * kernel's "divisible by 8" checks on the velog "tilelang" page, Host
 * IRModule); A, B and C 16-byte aligned; 256 * K * 2 < 2^31.
 * A and B may be NULL when K == 0.
 */
TGEMM_API int gemm_bf16_nt(int64_t M, int64_t N, int64_t K,
                 const void *A, const void *B, void *C, hipStream_t stream);

/*
 * C = A . B  ("NN"), fp16 in, fp32 accumulation, fp16 out.
 *
 * Defined by the velog "tilelang" page, 1.1 Front-End DSL: A is (M, K),
 * B is (K, N), the accumulator type is "float" and C is (M, N) float16.
 *
 *   A  device pointer, M x K fp16, row-major
 *   B  device pointer, K x N fp16, row-major (row stride N elements)
 *   C  device pointer, M x N fp16, row-major; written, never read
 *
 * Each output is the fp32 sum over k of A[m][k] * B[k][n], rounded to
 * nearest-even fp16 (overflow gives +-inf).  K == 0 writes zeros.
 * Requirements: K % 8 == 0, N % 8 == 0, 16-byte aligned pointers,
 * 256 * K * 2 < 2^31 and K' * N * 2 < 2^31, where K' is K rounded up to a
 * multiple of 64 (B is read in whole slices of 64 rows).
 */
TGEMM_API int gemm_f16_nn(int64_t M, int64_t N, int64_t K,
                const void *A, const void *B, void *C, hipStream_t stream);

/*
 * Block-scaled FP8 ("MXFP8") C = (sA * A) . (sB * B)^T, bf16 out.
 *
 * The Blackwell TCGEN05 GEMM tutorial, section "进阶" (Advanced), names a
 * block-scaled GEMM with one scale factor per 128 K elements for A and for
 * B.  Elements are OCP FP8 E4M3 ("e4m3fn", bias 7, max 448, no infinities);
 * scales are OCP E8M0 bytes E meaning 2^(E - 127).
 *
 *   A        device pointer, M x K e4m3fn bytes, row-major
 *   B        device pointer, N x K e4m3fn bytes, row-major
 *   scale_A  device pointer, M x ceil(K/128) e8m0 bytes, row-major:
 *            scale_A[m][j] scales A[m][128 j .. 128 j + 127]
 *   scale_B  device pointer, N x ceil(K/128) e8m0 bytes, row-major
 *   C        device pointer, M x N bf16, row-major; written, never read
 *
 * C[m][n] is the fp32 sum over k of
 *   A[m][k] * 2^(scale_A[m][k/128] - 127) * B[n][k] * 2^(scale_B[n][k/128] - 127),
 * rounded to nearest-even bf16.  K == 0 writes zeros.
 * Requirements: K % 16 == 0, N % 8 == 0, A, B and C 16-byte aligned (the
 * scale arrays need no alignment), 256 * K < 2^31.
 */
TGEMM_API int gemm_mxfp8_nt(int64_t M, int64_t N, int64_t K,
                  const void *A, const void *B,
                  const void *scale_A, const void *scale_B,
                  void *C, hipStream_t stream);

/*
 * Block-scaled FP4 ("MXFP4") C = (sA * A) . (sB * B)^T, bf16 out.
 *
 * The Blackwell TCGEN05 GEMM tutorial, section "进阶" (Advanced), names
 * MXFP8 "and other" block-scaled formats.  The pages fix no layout for
 * them; this follows the OCP MX format: OCP FP4 E2M1 elements (values 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit) packed two per byte, element 2i
 * in the low nibble of byte i, and one OCP E8M0 scale per 32 consecutive
 * K elements.
 *
 *   A        device pointer, M x K/2 bytes, row-major (row m holds A[m][0..K-1])
 *   B        device pointer, N x K/2 bytes, row-major
 *   scale_A  device pointer, M x K/32 e8m0 bytes: scale_A[m][j] scales
 *            A[m][32 j .. 32 j + 31]
 *   scale_B  device pointer, N x K/32 e8m0 bytes
 *   C        device pointer, M x N bf16, row-major; written, never read
 *
 * C[m][n] is the fp32 sum over k of
 *   A[m][k] * 2^(scale_A[m][k/32] - 127) * B[n][k] * 2^(scale_B[n][k/32] - 127),
 * rounded to nearest-even bf16.  K == 0 writes zeros.
 * Requirements: K % 32 == 0, N % 8 == 0, A, B and C 16-byte aligned (the
 * scale arrays need no alignment), 256 * K / 2 < 2^31.
 */
TGEMM_API int gemm_mxfp4_nt(int64_t M, int64_t N, int64_t K,
                  const void *A, const void *B,
                  const void *scale_A, const void *scale_B,
                  void *C, hipStream_t stream);

/*
 * Block-scaled FP6 ("MXFP6") C = (sA * A) . (sB * B)^T, bf16 out.
 *
 * Another of the block-scaled formats the Blackwell TCGEN05 GEMM tutorial,
 * section "进阶" (Advanced), groups with MXFP8; as for MXFP4 the pages fix
 * no layout, and this follows the OCP MX format: both operands of one OCP
 * FP6 element type, `fmt`, and one OCP E8M0 scale per 32 consecutive K
 * elements.  The elements are packed densely: a row of K elements is 3K/4
 * bytes, element k at bits 6k .. 6k+5 of the row read as a little-endian
 * bit string (four elements in three bytes).
 *
 *   fmt      TGEMM_FP6_E2M3 (0): sign, 2 exponent bits (bias 1), 3 mantissa
 *            bits, largest value 7.5; TGEMM_FP6_E3M2 (1): sign, 3 exponent
 *            bits (bias 3), 2 mantissa bits, largest value 28.  No
 *            infinities or NaN.
 *   A        device pointer, M x 3K/4 bytes, row-major
 *   B        device pointer, N x 3K/4 bytes, row-major
 *   scale_A  device pointer, M x K/32 e8m0 bytes: scale_A[m][j] scales
 *            A[m][32 j .. 32 j + 31]
 *   scale_B  device pointer, N x K/32 e8m0 bytes
 *   C        device pointer, M x N bf16, row-major; written, never read
 *
 * C[m][n] is the fp32 sum over k of
 *   A[m][k] * 2^(scale_A[m][k/32] - 127) * B[n][k] * 2^(scale_B[n][k/32] - 127),
 * rounded to nearest-even bf16.  K == 0 writes zeros.
 * Requirements: K % 64 == 0 (whole 16-byte pieces of a row), N % 8 == 0,
 * A, B and C 16-byte aligned (the scale arrays need no alignment),
 * 256 * 3K/4 < 2^31.  A fmt other than 0 or 1 returns TGEMM_EINVAL.
 */
#define TGEMM_FP6_E2M3 0
#define TGEMM_FP6_E3M2 1
TGEMM_API int gemm_mxfp6_nt(int fmt, int64_t M, int64_t N, int64_t K,
                  const void *A, const void *B,
                  const void *scale_A, const void *scale_B,
                  void *C, hipStream_t stream);

/*
 * C = op(A) . op(B) for 16-bit inputs with any operand storage and row
 * strides: bfloat16 in and out (gemm_bf16), fp16 in and out (gemm_f16);
 * fp32 accumulation.
 *
 * The pages' GEMM takes transpose flags for its operands (TileLang SM100
 * README, "Code Example": T.gemm(..., trans_B=True); the tutorial notes
 * trans_A as well) and addresses its tensors through row strides (velog
 * "tilelang", 1.2 Pass Pipeline, Host IRModule).
 *
 *   trans_a  0: A is stored M x K (op(A) = A);   1: A is stored K x M (op(A) = A^T)
 *   trans_b  0: B is stored K x N (op(B) = B);   1: B is stored N x K (op(B) = B^T)
 *   A, B     device pointers, row-major as stored, rows lda / ldb elements apart
 *   C        device pointer, M x N row-major, rows ldc elements apart;
 *            written (only its M x N elements), never read
 *
 * Each output is the fp32 sum over k of op(A)[m][k] * op(B)[k][n], rounded
 * to nearest-even bf16 (fp16 for gemm_f16, overflow to +-inf).  K == 0
 * writes zeros.  gemm_bf16(0, 1, ...) with packed strides is gemm_bf16_nt;
 * gemm_f16(0, 0, ...) with packed strides is gemm_f16_nn.
 * Requirements: trans_a, trans_b in {0, 1}; lda, ldb, ldc at least the
 * stored row lengths and multiples of 8; the contiguous dimension of each
 * stored operand (K or M for A, N or K for B) and N multiples of 8; A, B
 * and C 16-byte aligned and C not overlapping A or B; a K-contiguous
 * operand's 256 rows, and an M/N-contiguous operand's K rows rounded up to
 * a multiple of 64 (times its row stride), below 2^31 bytes.
 */
TGEMM_API int gemm_bf16(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t lda, const void *B, int64_t ldb,
                        void *C, int64_t ldc, hipStream_t stream);
TGEMM_API int gemm_f16(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, const void *B, int64_t ldb,
                       void *C, int64_t ldc, hipStream_t stream);

/*
 * C = op(A) . op(B) as gemm_bf16 / gemm_f16, with the K range split over
 * several workgroups per output tile, for problems with too few output tiles
 * to fill the GPU's compute units (M x N small, K deep).
 *
 * The pages give each output tile one thread block for all of K (TileLang
 * SM100 README, "Code Example": T.Kernel over ceil-div tiles of N and M,
 * T.Pipelined over all of K) and point to a persistent, warp-specialised
 * GEMM for scheduling work onto the machine (Blackwell TCGEN05 GEMM
 * tutorial, section "进阶" (Advanced)).  Here, when the tiles are fewer than
 * the CUs, each tile's K slices are divided into `splits` contiguous ranges
 * computed by different workgroups: each writes its fp32 sums to one plane
 * of the workspace, and a second kernel on the same stream adds the planes
 * in order (plane 0 first) and rounds once to the output type.  No device-
 * scope synchronisation is used: the kernel boundary orders the two passes.
 *
 * Arguments and requirements as for gemm_bf16 / gemm_f16, plus:
 *   splits           0: the library chooses (no split unless the plain grid
 *                    leaves at least half the CUs idle and K >= 3072; then
 *                    64 x 64 tiles and at most 4 splits of at least 1024 K
 *                    elements each, no more than the workspace holds);
 *                    1: no split (the workspace is not used); 2 .. 16: that
 *                    many (at most one per 64 K elements: more are clipped)
 *   workspace        device pointer, 16-byte aligned, owned by the caller,
 *                    not overlapping A, B or C; may be NULL when splits == 1
 *   workspace_bytes  its size; at least splits * M * N * 4 for splits >= 2
 *                    (tgemm_splitk_workspace_bytes); its contents on entry
 *                    do not matter and are left undefined
 * Sums are fp32; the order differs from gemm_bf16's only in that the split
 * ranges' sums are added at the end, in range order, so the result is
 * deterministic.  A forced tile (tgemm_set_tile) must be 128 x 128 or
 * 64 x 64 for splits >= 2 (TGEMM_EINVAL otherwise); other forced tiles run
 * without a split when splits == 0.  Returns TGEMM_EINVAL for splits outside
 * 0 .. 16, a NULL or too small workspace, or a workspace overlapping an
 * operand, TGEMM_EALIGN for a misaligned workspace.
 */
TGEMM_API int gemm_bf16_splitk(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                               const void *A, int64_t lda, const void *B, int64_t ldb,
                               void *C, int64_t ldc, int splits, void *workspace,
                               uint64_t workspace_bytes, hipStream_t stream);
TGEMM_API int gemm_f16_splitk(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                              const void *A, int64_t lda, const void *B, int64_t ldb,
                              void *C, int64_t ldc, int splits, void *workspace,
                              uint64_t workspace_bytes, hipStream_t stream);

/*
 * gemm_bf16_splitk for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation and arguments, without the workspace:
 * the partial sums go to a scratch array of 8 MiB that the library holds on
 * each GPU it runs on until the process ends (set up with the device, no
 * allocation per call).  This entry point calls no hipMalloc, hipFree or
 * other allocating routine.
 *
 * Limits: splits * M * N * 4 <= 8 MiB for splits >= 2, else TGEMM_ETOOBIG;
 * splits == 0 chooses within the scratch (no split when even two planes do
 * not fit).  Every call on one GPU uses that GPU's one scratch array, so
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race and may corrupt each other's results; calls on one stream run in
 * order and are safe.  Nothing in the scratch needs clearing: every element
 * a call reads it has written first.
 */
TGEMM_API int gemm_bf16_splitk_noalloc(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                                       const void *A, int64_t lda, const void *B, int64_t ldb,
                                       void *C, int64_t ldc, int splits, hipStream_t stream);

/*
 * Workspace bytes gemm_bf16_splitk / gemm_f16_splitk use for an M x N output
 * with `splits` splits: splits * M * N * 4; for splits == 0 the most the
 * automatic choice can use (4 * M * N * 4); 0 for splits == 1 or invalid
 * arguments.
 */
TGEMM_API uint64_t tgemm_splitk_workspace_bytes(int64_t M, int64_t N, int splits);

/*
 * Block-scale quantiser: binary32 rows to the operand format of
 * gemm_mxfp8_nt (the step before the block-scaled GEMM; one scale per 128 K
 * elements as in the Blackwell TCGEN05 GEMM tutorial, section "进阶"
 * (Advanced)).
 *
 *   x       device pointer, M x K binary32, row-major (finite values)
 *   q       device pointer, M x K e4m3fn bytes, row-major; written
 *   scales  device pointer, M x ceil(K/128) e8m0 bytes, row-major; written
 *
 * For each row and each block of 128 K elements (the last may be shorter),
 * the scale is the smallest power of two 2^e with max |x| <= 448 * 2^e
 * (448 = largest e4m3fn), e clamped to [-127, 127] and e = -127 for an
 * all-zero block, stored as the byte e + 127; each element is x * 2^-e
 * rounded to the nearest e4m3fn value, ties to even.  The pages fix the
 * granularity and format but no rule for the scale: this rule is the
 * library's.
 * Requirements: K % 16 == 0; x and q 16-byte aligned (scales need no
 * alignment); no overlap between the three arrays.  M == 0 or K == 0
 * writes nothing.
 */
TGEMM_API int quantize_mxfp8(int64_t M, int64_t K, const float *x, void *q, void *scales,
                             hipStream_t stream);

/*
 * Optional, idempotent set-up for the current device: checks that it is a
 * gfx950 GPU.  Returns TGEMM_OK or TGEMM_EHIP.  Entry points call it
 * themselves on first use of a device (the host wrapper's init() on the
 * velog "tilelang" page, 1.3 Code Generation & Runtime, plays this role).
 */
TGEMM_API int tgemm_init(void);

/*
 * Message for the last failing call on this host thread; "" after a
 * successful call.  The pointer stays valid until the thread's next call.
 * This is the get_last_error() of the host wrapper on the velog "tilelang"
 * page (1.3 Code Generation & Runtime), which keeps the message of the last
 * failure in a static buffer; here the buffer is per host thread (1024
 * bytes, the page's size) and is cleared by every call.
 */
TGEMM_API const char *tgemm_last_error(void);

/*
 * Shader-clock probe, a measurement helper off the GEMM path.  The pages
 * time a kernel and report TFLOPS = 2 M N K / t (TileLang SM100 README,
 * "Compilation and Usage"); on MI355X that time also depends on the shader
 * clock the board's power limit allows.  The probe runs one single-wave
 * workgroup per CU (256), each reading its CU's shader-clock counter
 * (s_memtime) and the constant-rate counter (s_memrealtime).  Every CU has
 * a shader-clock counter of its own, so two probes give a CU's average
 * clock between them from records of the same CU only:
 * (difference of the shader-clock counts) / (difference of the constant-rate
 * counts) * the constant rate.
 *
 *   out            device pointer to 1024 uint64 (8 KiB), 16-byte aligned,
 *                  owned by the caller; written on `stream` with 256
 *                  records of four uint64, one per workgroup:
 *                  {XCC id << 32 | HW_ID (bits 8-11 CU, bit 12 shader
 *                  array, bits 13-15 shader engine), shader-clock count,
 *                  constant-rate count, 0}
 *   wallclock_khz  host pointer, may be NULL; receives the constant-rate
 *                  counter's frequency in kHz (written before returning)
 *
 * Returns TGEMM_OK, TGEMM_EINVAL (out NULL), TGEMM_EALIGN (out misaligned)
 * or TGEMM_EHIP.
 */
TGEMM_API int tgemm_clock_probe(void *out, int *wallclock_khz, hipStream_t stream);

/*
 * Output tile override for the calling host thread's later calls, for
 * tuning and tests.  Each workgroup computes a tile_m x tile_n block of C;
 * by default (0, 0) the library picks, per call, the shape that needs the
 * fewest waves of workgroups for the least work (the pages' kernels take
 * their block sizes as parameters: SM100 README, "Code Example",
 * block_M / block_N; velog "tilelang", 1.1 Front-End DSL).
 *   B stored N x K (gemm_bf16_nt, trans_b = 1): 256x256, 256x192, 128x128, 64x64
 *   B stored K x N (gemm_f16_nn, trans_b = 0):  256x256, 128x128, 64x64
 *   gemm_mxfp8_nt, gemm_mxfp4_nt, gemm_mxfp6_nt: 256x256
 * Returns TGEMM_OK, or TGEMM_EINVAL for a shape no entry point has; an
 * entry point called with a shape it does not have returns TGEMM_EINVAL.
 * The result does not depend on the tile shape beyond the order of the
 * fp32 summation.
 */
TGEMM_API int tgemm_set_tile(int tile_m, int tile_n);

#ifdef __cplusplus
}
#endif

#endif /* TGEMM_H */
