// Tiled dense GEMM kernels for gfx950 (MI355X, CDNA4).
//
// One workgroup of 256 threads (4 wave64s in a 2 x 2 grid) computes a
// TM x TN tile of C -- 256 x 256, or 256 x 192, 128 x 128 and 64 x 64 where
// that fills the chip better -- and each wave a TM/2 x TN/2 sub-tile of fp32
// accumulators (in AGPRs; 256 per lane for 256 x 256).  The K loop walks
// slices of the A and B panels (128 bytes of a row: 64 bf16/fp16, 128 fp8
// or 256 fp4 elements) through a ring of LDS slots per operand; fp6 runs
// 64-element K steps (48 bytes) over whole 128-byte lines of its rows (the
// fp6 section below).
//
// Where this follows the pages and where it departs:
//  * tile grid: ceil-div over N and M as in the TileLang SM100 README
//    ("Code Example", T.Kernel(T.ceildiv(N, block_N), T.ceildiv(M, block_M)));
//    workgroup ids are remapped so each XCD's workgroups cover a compact
//    block of tiles (the pages only name a threadblock-swizzle header,
//    velog "tilelang", 1.3 Code Generation & Runtime).
//  * accumulator init: the first K slice's MFMAs start from zero (T.clear /
//    clear_accum).
//  * global -> LDS staging: the pages use TMA boxes with a hardware
//    swizzle (velog "tilelang", 1.2 Host IRModule).  Here every lane moves
//    16 bytes with a buffer load that writes LDS directly, a whole 128-byte
//    line per row and slice; the 16-byte chunks of each row are
//    XOR-permuted so the MFMA operand reads hit distinct LDS banks.
//    Out-of-range rows take an out-of-range buffer offset and arrive as
//    zeros (the pages' TMA zero OOB fill).  The ragged last K slice of a
//    K-contiguous operand is zeroed in LDS past column K once it has landed
//    (MXFP8 and MXFP4 with a ragged K check columns in their loads instead;
//    MXFP6 never reads past a row's last K step); a K-major operand's rows
//    past K read as zeros.
//  * pipelined K loop: the pages use a 3-slot ring with producer and
//    consumer warpgroups and mbarrier parity waits (velog "tilelang",
//    Device IRModule).  Here every wave both loads and computes, with a
//    ring of NS slots (two for 256-row tiles, four for 128 x 128 and
//    64 x 64): partway through slice kt's MFMAs (halfway, or three quarters
//    for fp8) a wait and a barrier free slot kt % NS; the loads of slice
//    kt + NS into it then go out spread over the next half slice of MFMAs
//    (three quarters for fp4).  The next slice's first operand reads follow
//    the barrier, overlapping the current slice's remaining MFMAs.  fp6:
//    two slots of line stages, four barriers per 8 K steps.
//  * wave-tile MMA: v_mfma_f32_16x16x32_{bf16,f16} (8 x 8 blocks per wave)
//    and, for the block-scaled kinds, the scaled f8f6f4 MFMA with the e8m0
//    block scales as operands (TCGEN05 tutorial, "进阶" (Advanced)):
//    32 x 32 x 64 (4 x 4 blocks) on fp8 and fp6 elements, 16 x 16 x 128
//    (8 x 8 blocks) on fp4.
//  * operand layouts (trans_A / trans_B of the SM100 README's T.gemm): an
//    operand stored K-contiguous (A as M x K, B as N x K) is staged row by
//    row as above; one stored M- or N-contiguous (A as K x M, B as K x N)
//    stays K-major in LDS and is read with the LDS transpose read
//    (ds_read_b64_tr_b16), which hands each lane four K values of one
//    column.  Rows of every operand and of C are ld elements apart.
//  * epilogue: fp32 -> bf16/fp16 with round-to-nearest-even, masked stores.
//    The MFMA is fed B rows as its first operand and A rows as its second,
//    so each lane's accumulators hold consecutive columns of one row of C;
//    lane swaps regroup them so each lane leaves 16 bytes per store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "tgemm_internal.hpp"

namespace tgemm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(6))) int i32x6;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;                  // bytes of one tile row per K slice
constexpr uint32_t kOOB = 0x80000000u;          // voffset that is always out of range

struct Args {
  const uint8_t *A;
  const uint8_t *B;
  const uint8_t *SA;
  const uint8_t *SB;
  uint8_t *C;
  int M, N, K;
  int lda, ldb, ldc;  // row strides of A, B and C as stored, in elements
  int tiles_m, tiles_n;
  int ksteps;  // ceil(K / elements per slice)
  int kb;      // scale blocks per row (mxfp8)
  // K split (16-bit kinds): workgroup w computes the tile w % tiles over
  // slices [kq s, kq s + kq) with s = w / tiles, and writes its fp32 sums to
  // plane s of ws (splits planes of M x N, rows N apart).
  float *ws;
  int splits, kq;
};

// Element type of A and B, and the storage of each: AK, A is M x K
// (K-contiguous; else K x M); BK, B is N x K (K-contiguous; else K x N).
// fp4 operands are handled as rows of bytes (two E2M1 elements each):
// kElem = 1 and K counts bytes inside the kernel.
// fp6 (E2M3 or E3M2) likewise: rows of densely packed 6-bit elements, K
// counted in bytes; its K loop runs 64-element steps over 128-byte line
// stages (the kernel's fp6 section).
enum : int { kBf16 = 0, kF16 = 1, kFp8 = 2, kFp4 = 3, kFp6E2M3 = 4, kFp6E3M2 = 5 };
template <int DT, bool AK, bool BK, bool WHOLE = false>
struct Traits {
  static constexpr int kDt = DT;
  // MXFP8 and MXFP4 with K a positive multiple of the slice: no slice is
  // ragged, so their loads check no columns (otherwise they do, as MXFP6's
  // always do; the other kinds never do, and zero the ragged slice's tail in
  // LDS instead).  For MXFP4 it also means dword-aligned scale rows (both
  // scale arrays dword-aligned; K a multiple of 256 makes every row's 8 K/256
  // scale bytes a whole number of dwords).
  static constexpr bool kWholeK = WHOLE;
  static constexpr bool kScaled = DT >= kFp8;
  static constexpr bool kFp6 = DT == kFp6E2M3 || DT == kFp6E3M2;
  static constexpr int kElem = kScaled ? 1 : 2;
  static constexpr int kSliceBytes = 128;                  // global bytes of a row per K slice (fp6: line stage)
  static constexpr int kPitch = kSliceBytes;               // LDS bytes of a slot row
  static constexpr bool kAK = AK, kBK = BK;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  // dword3 0x00020000: raw (untyped) 32-bit data format, no swizzle.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

// s_waitcnt immediate for vmcnt(vm) expcnt(7) lgkmcnt(0) (gfx9 encoding:
// vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14).
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(VM >= 0 && VM < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
}

// Wait states between the last MFMAs and VALU code that reads their
// accumulators.  The 16-bit MFMAs are inline asm, which the compiler's hazard
// tracking does not see as MFMAs, so the required states are written out.
// The CDNA3/CDNA4 rule for an XDL MFMA writing a register that a later VALU
// instruction reads is a number of wait states that grows with the MFMA's
// passes; for gfx950 the compiler's own hazard recognizer places, for the
// builtins of the forms used here, 8 wait states after
// v_mfma_f32_16x16x32_bf16/_f16 (4 passes), 12 after the scaled 32 x 32 x 64
// form on fp6 (8 passes) and 12 after the scaled 16 x 16 x 128 form on fp8
// (8 passes) before a dependent v_mul_f32 (checked on this build's own
// assembly); the scaled 16 x 16 x 128 form on fp4 (4 passes) needs no more.
// Three s_nop 7 give 24.  Between MFMAs no states are needed: consecutive
// MFMAs write different accumulators, an accumulator is read again as SrcC
// only by the same form 64 (16 x 16 blocks) or 16 (32 x 32) MFMAs later,
// the fragment registers an MFMA reads (SrcA/B, read in its first pass)
// are rewritten only by LDS reads issued after it, whose data returns tens
// of cycles later, the fp4 scale registers are rewritten at least a slice
// after their last MFMA, and the fp8 ones after their last MFMA of a group
// (the one write-after-read hazard of an MFMA is on SrcC) and at least two
// MFMAs before the next MFMA that reads them (the two wait states a VALU
// write needs before an MFMA reads the register).
__device__ __forceinline__ void mfma_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Store of 16 bytes of C, written through the L2 at system scope (sc0 sc1):
// the L2 keeps none of the output dirty, so the kernel's end has none of it
// to write back.  Measured on the launch-to-launch time at 4096^3: MXFP8
// -2.7%, MXFP4 -4.9%, bf16 4096 x 4096 x 8192 unchanged (non-temporal stores
// gave nothing).  No builtin sets these bits on a global store, so it is
// inline asm; the s_nop 1 in the same statement gives the two wait states
// gfx950 needs before a VALU instruction may overwrite the data registers of
// a 128-bit store (the compiler places the same s_nop after its own such
// stores, but does not see this one as a store).  The store has no output
// register, and the kernel issues no memory operation after its C stores
// whose wait would have to count them.
__device__ __forceinline__ void store_c(uint8_t *p, const u32x4 &v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

// Workgroup barrier that orders LDS traffic for the compiler but leaves the
// hardware waits to the caller (no fence, so no implicit vmcnt(0)).
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk permutation inside a 128-byte tile row: row r keeps logical 16-byte
// chunk c at physical chunk c ^ swz(r).  Chosen by measurement
// (SQ_LDS_BANK_CONFLICT on gfx950): with it neither the 16 x 16 x 32 operand
// reads (lanes 0-15 read 16 rows at one chunk, lanes 16-31 the same rows at
// the next chunk, ...) nor the 32 x 32 x 64 ones conflict, whereas e.g.
// (r & 7) ^ ((r >> 3) & 1) conflicts 2-way on the 16 x 16 pattern.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// K-major slot of W columns: 64 K rows of 2 W bytes.  Row k keeps logical
// chunk c at physical chunk c ^ swz_nn<W>(k).  For W = 256 and 128 the
// permutation was measured conflict-free for the transpose reads, which take
// four consecutive K rows at a time.  A 128-byte row (W = 64) has only 8
// chunks; there the reads' 32-byte column segments move by whole segments,
// so that the 8 K rows a half-wave reads (8 g + 4 t + e, g < 2, e < 4) fall
// on 8 different 32-byte bank groups.
template <int W>
__device__ __forceinline__ int swz_nn(int k) {
  if constexpr (W == 64)
    return (((k >> 1) & 1) | (((k >> 3) & 1) << 1)) << 1;
  else
    return ((k & 3) << 2) ^ ((k >> 2) & 3);
}

// Workgroup id -> output tile.  Consecutive workgroup ids are placed on the
// 8 XCDs in turn; renumber so that the ids sharing an XCD are consecutive,
// then walk tiles in groups of kGroupM tile-rows (column by column inside a
// group) so an XCD's workgroups share A and B panels in its L2.
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_of(int wg, int nwg, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int xcd = wg & 7, local = wg >> 3;
  const int base = nwg >> 3, rem = nwg & 7;
  const int v = xcd * base + (xcd < rem ? xcd : rem) + local;
  const int group = v / (kGroupM * tiles_n);
  const int first_m = group * kGroupM;
  const int gm = (tiles_m - first_m) < kGroupM ? (tiles_m - first_m) : kGroupM;
  const int in = v - group * kGroupM * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

// ---------------------------------------------------------------------------
// Staging of one K slice of a K-contiguous panel (A of every kind, B of the
// NT kinds) of 32 NI rows into a slot of 32 NI rows x 128 bytes.  Wave w
// moves rows [8 NI w, 8 NI (w + 1)) with NI direct-to-LDS instructions of 8
// rows each; lane l of instruction i writes LDS bytes [16 l, 16 l + 16) of
// its 1 KiB row group, i.e. row 8 NI w + 8 i + l / 8, physical chunk l % 8,
// and therefore fetches logical chunk (l % 8) ^ swz(row) of that row.
// swz(row) = (4 NI w + 4 i + l / 16) & 7 = (4 i + l / 16) & 7 for even NI:
// it depends on i only through its parity.
// ---------------------------------------------------------------------------
template <int NI>
struct PanelLoader {
  static_assert(NI % 2 == 0, "the swizzle phase of a wave's first row must not depend on the wave");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[NI];  // per instruction: byte offset of this lane's chunk at slice 0
  int kcol[2];       // element column of this lane's chunk inside a slice (even / odd i)
  uint32_t slice_bytes;

  // slice_k: elements of a row per slice (the 128 bytes of a slot row).
  __device__ __forceinline__ void init(const uint8_t *panel, int rows_valid, int K, int ld, int elem, int slice_k,
                                       int wave, int lane) {
    slice_bytes = (uint32_t)(slice_k * elem);
    rsrc = make_rsrc(panel, ((uint32_t)(rows_valid - 1) * (uint32_t)ld + (uint32_t)K) * (uint32_t)elem);
#pragma unroll
    for (int p = 0; p < 2; ++p) kcol[p] = ((lane & 7) ^ swz(8 * p + (lane >> 3))) * (16 / elem);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = wave * 8 * NI + i * 8 + (lane >> 3);
      off[i] = r < rows_valid ? (uint32_t)r * (uint32_t)ld * (uint32_t)elem + (uint32_t)kcol[i & 1] * elem : kOOB;
    }
  }

  // Instruction i of slice kt.  Columns are not checked: in the ragged last
  // slice a chunk at or past column K reads the start of the next row (past
  // the panel's last row, zeros from the range check), and zero_tail()
  // clears it once it has landed; slices past the last one land in slots
  // that are never read.  (A per-load select right before each load stalled
  // the MFMA stream: 8% more cycles per workgroup.)
  __device__ __forceinline__ void issue(LDS_AS uint8_t *slot, int wave, int kt, int i) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(slot + (wave * NI + i) * 1024), 16, off[i],
                                             (uint32_t)kt * slice_bytes, 0, 0);
  }

  // The same with the column check: a chunk at or past column K takes an
  // out-of-range offset (MXFP8 with a ragged last slice, whose kernel a
  // zeroing branch inside its slice would push into spilling registers).
  __device__ __forceinline__ void issue_masked(LDS_AS uint8_t *slot, int wave, int kt, int K, int slice_k,
                                               int i) const {
    const bool ok = kt * slice_k + kcol[i & 1] < K;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(slot + (wave * NI + i) * 1024), 16,
                                             ok ? off[i] : kOOB, (uint32_t)kt * slice_bytes, 0, 0);
  }

  // Zero the chunks this lane loaded for slice kt (in `slot`) that lie at or
  // past column K.
  __device__ __forceinline__ void zero_tail(LDS_AS uint8_t *slot, int wave, int lane, int kt, int K,
                                            int slice_k) const {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      if (kt * slice_k + kcol[i & 1] >= K) *(LDS_AS u32x4 *)(slot + (wave * NI + i) * 1024 + 16 * lane) = u32x4{};
  }
};

// ---------------------------------------------------------------------------
// Staging of one K slice of an M- or N-contiguous 16-bit operand (A stored
// K x M, B stored K x N, rows ld elements apart) for a tile of W columns
// (W = 256 or 128) into a slot of 64 K rows x 2 W bytes.  Wave w moves K
// rows [16 w, 16 w + 16) with NI = W / 32 instructions of RPI = 512 / W
// rows each; lane l of instruction i writes row 16 w + RPI i + l / LPR
// (LPR = W / 8 lanes per row), physical chunk l % LPR, fetching logical
// chunk (l % LPR) ^ swz_nn(row), i.e. columns c0 + 8 chunk .. + 8.
// ---------------------------------------------------------------------------
template <int W>
struct MNLoader {
  static_assert(W == 256 || W == 128 || W == 64, "an instruction covers whole K rows of the slot");
  static constexpr int NI = W / 32, RPI = 512 / W, LPR = W / 8;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[NI];  // per instruction: byte offset at slice 0 (kOOB past the last column)
  int krow0;         // K row of instruction 0 inside the slice
  uint32_t slice_bytes;

  // X: the whole operand; ext: its columns (M or N); c0: the tile's first.
  __device__ __forceinline__ void init(const uint8_t *X, int K, int ext, int c0, int ld, int wave, int lane) {
    rsrc = make_rsrc(X, K > 0 ? ((uint32_t)(K - 1) * (uint32_t)ld + (uint32_t)ext) * 2u : 0u);
    const uint32_t row_bytes = (uint32_t)ld * 2u;
    slice_bytes = 64u * row_bytes;
    krow0 = wave * 16 + lane / LPR;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int kr = krow0 + RPI * i;
      const int c = c0 + ((lane % LPR) ^ swz_nn<W>(kr)) * 8;
      off[i] = c < ext ? (uint32_t)kr * row_bytes + (uint32_t)c * 2u : kOOB;
    }
  }

  // Instruction i of slice kt.  K rows are not checked: the rows of the
  // ragged last slice at or past K lie past the end of the resource, so the
  // range check returns zeros for them (the host keeps whole slices of rows
  // inside 31-bit offsets, so no offset wraps).  A slice past the last one
  // re-reads the last (its slot is never read).
  __device__ __forceinline__ void issue(LDS_AS uint8_t *slot, int wave, int kt, int nk, int i) const {
    const int ks = kt < nk ? kt : (nk > 0 ? nk - 1 : 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(slot + (wave * NI + i) * 1024), 16, off[i],
                                             (uint32_t)ks * slice_bytes, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
// LDS slots of the K-slice ring.  The 256-row tiles fill the LDS with two
// (2 x 64 KiB).  A 128 x 128 tile's slice holds a quarter of the MFMA work
// of a 256 x 256 one, too little to cover the latency of the next slice's
// loads with one slice in flight, so its ring has four slots (4 x 32 KiB):
// the loads of slice kt + 4 go out in slice kt, three slices ahead of use.
template <class T, int TM, int TN>
constexpr int kSlots = (!T::kScaled && TM * TN <= 128 * 128) ? 4 : 2;

struct Slots {
  LDS_AS uint8_t *a[4];
  LDS_AS uint8_t *b[4];
  LDS_AS uint8_t *junk;      // 256 bytes per wave: landing area of the L2 prefetches
  LDS_AS uint8_t *stage;     // fp4, fp6: staged 16-byte scale chunks of the 512 rows
};


// fp8 K loop (the scaled 16 x 16 x 128 MFMA, one K step per slice, 8 x 8
// blocks of 16 x 16 per wave): the order of a slice's 64 MFMAs and the
// positions of the fragment reads.  A slice runs four quadrants of 4 x 4
// blocks (x blocks 0-3 or 4-7 against y blocks 0-3 or 4-7), x block by x
// block with the y blocks snaking, each quadrant's x blocks in the reverse
// order of the one before, so that every MFMA shares an operand with the
// one before it.  Slices of phase 0 (even) take the quadrants (x lo, y lo),
// (x lo, y hi), (x hi, y hi), (x hi, y lo); slices of phase 1 (x lo, y hi),
// (x lo, y lo), (x hi, y lo), (x hi, y hi).  Either way each group of
// fragments is free (its last MFMA issued) 16 MFMAs or more before the next
// slice first takes it, so the reads of the next slice's fragments spread
// over the second half of a slice and the first of the next.
namespace f8 {
constexpr int kNB = 8;         // blocks per wave and dimension
constexpr int kM = kNB * kNB;  // MFMAs per slice
struct IJ {
  int i, j;  // x block, y block
};
constexpr IJ order(int p, int q) {
  const int k = q / 16, r = q % 16;
  const int xh = k >= 2 ? 1 : 0;
  const int yh = p ? (k == 0 || k == 3 ? 1 : 0) : (k == 1 || k == 2 ? 1 : 0);
  const int xi = (k & 1) ? 3 - r / 4 : r / 4;
  const int yi = ((r / 4) & 1) ? 3 - r % 4 : r % 4;
  return IJ{4 * xh + xi, 4 * yh + yi};
}
// Fragment F: x block F (F < 8) or y block F - 8.
constexpr bool uses(int p, int q, int F) { return F < kNB ? order(p, q).i == F : order(p, q).j == F - kNB; }
constexpr int last_use(int p, int F) {
  int l = -1;
  for (int q = 0; q < kM; ++q)
    if (uses(p, q, F)) l = q;
  return l;
}
constexpr int first_use(int p, int F) {
  for (int q = 0; q < kM; ++q)
    if (uses(p, q, F)) return q;
  return kM;
}
// Read positions for the next slice's fragments during a slice of phase p
// (before MFMA pos of this slice; kM and on: of the next slice): each
// fragment once its registers are free (after its last MFMA here) and the
// barrier before MFMA `bar` has published the next slice, in order of
// availability, at least kGap MFMAs apart (a fragment is two 16-byte LDS
// reads per lane; the LDS also takes the loads of the slice after).
struct Sched {
  int pos[2 * kNB];
};
constexpr int kGap = 2;
constexpr Sched schedule(int p, int bar) {
  Sched s{};
  bool done[2 * kNB] = {};
  int ready[2 * kNB] = {};
  for (int F = 0; F < 2 * kNB; ++F) {
    const int r = last_use(p, F) + 1;
    ready[F] = r < bar ? bar : r;
  }
  int next = 0;
  for (int n = 0; n < 2 * kNB; ++n) {
    int best = -1, best_r = 0;
    for (int F = 0; F < 2 * kNB; ++F)
      if (!done[F] && (best < 0 || ready[F] < best_r)) {
        best = F;
        best_r = ready[F];
      }
    done[best] = true;
    next = best_r > next ? best_r : next;
    s.pos[best] = next;
    next += kGap;
  }
  return s;
}
// Every read lands before the next slice's barrier and at least four
// MFMAs before its first use there.
constexpr bool schedule_ok(int bar) {
  for (int p = 0; p < 2; ++p) {
    const Sched s = schedule(p, bar);
    for (int F = 0; F < 2 * kNB; ++F)
      if (s.pos[F] >= kM + bar || s.pos[F] + 4 > kM + first_use(p ^ 1, F)) return false;
  }
  return true;
}
// A conversion at position pos of a slice of phase 1 (kM and on: of the
// next slice, phase 0) writes the scale registers of blocks 4 J .. 4 J + 3
// (x blocks for J < 2, y blocks after): after their last MFMA in the one
// and at least two MFMAs before their first in the other.
constexpr bool convert_ok(int pos, int J) {
  for (int c = 0; c < 4; ++c) {
    const int F = 4 * J + c;
    if (pos <= last_use(1, F) || pos + 2 > kM + first_use(0, F)) return false;
  }
  return true;
}
}  // namespace f8

template <class T, int TM, int TN, bool SPLIT = false>
struct Kernel {
  static_assert(!SPLIT || !T::kScaled, "the K split is for the 16-bit kinds");
  static constexpr int kNS = kSlots<T, TM, TN>;
  static constexpr int kElem = T::kElem;
  static constexpr int kWM = TM / 2, kWN = TN / 2;   // wave tile (2 x 2 waves)
  static constexpr int kSlotA = TM * T::kPitch;      // one slot of A, of B (K-major: 64 K rows x 2 TM / 2 TN bytes)
  static constexpr int kSlotB = TN * T::kPitch;
  static constexpr int kSliceK = T::kSliceBytes / kElem;  // K elements (packed kinds: bytes) per slice
  // MFMA shape.  16-bit inputs: v_mfma_f32_16x16x32 (it reads and writes 4
  // accumulators per 16 K flops, half the accumulator traffic per flop of
  // the 32 x 32 x 16 form; under full load the chip is power-capped, and the
  // lower-energy form runs at a higher clock).  fp4: the scaled 16 x 16 x 128
  // form for the same reason (in a register-only stream of random operands
  // under the power limit it delivered 13% more flops per second than the
  // 32 x 32 x 64 form); its 16-byte fragments are laid out like the 16-bit
  // kinds'.  Their slices are two K substeps.  fp8: the scaled 16 x 16 x 128
  // form too (9% more flops per second than 32 x 32 x 64 in the same
  // stream), one K step per slice, in a K loop of its own (below).  fp6:
  // the scaled 32 x 32 x 64 form, in its own K loop.
  static constexpr bool kW = T::kFp6;  // 32 x 32 blocks
  static constexpr int kBlk = kW ? 32 : 16;
  static constexpr int kNBm = kWM / kBlk;       // blocks per wave along M (y blocks)
  static constexpr int kNBn = kWN / kBlk;       // blocks per wave along N (x blocks)
  static constexpr int kNR = kNBm + kNBn;       // fragment reads per substep
  static constexpr int kPerSub = kNBm * kNBn;   // MFMAs per substep
  static constexpr int kMfma = 2 * kPerSub;     // MFMAs per slice
  // Load instructions per wave per slice: 8 rows of 128 bytes each (fp6 has
  // its own K loop, below).
  static constexpr int kLA = TM / 32, kLB = TN / 32;
  static constexpr int kLoads = kLA + kLB;
  static_assert(!T::kScaled || (TM == 256 && TN == 256 && T::kAK && T::kBK),
                "the block-scaled kernel uses 256 x 256 tiles of K-contiguous operands");
  static_assert(kWM % kBlk == 0 && kWN % kBlk == 0, "wave tile");
  // Schedule, in MFMAs of a slice: the wait + barrier go before MFMA
  // kBarrierAt; the loads of slice kt + kNS go out evenly over the kWindow
  // MFMAs from there on (running into slice kt + 1), which leaves
  // kMfma - kWindow MFMAs for the last of them to land.  Loads spread over
  // too short a window overrun the texture unit (about 64 bytes per clock
  // per CU) and stall the MFMA stream behind a full queue.  The barrier
  // positions are the measured best (fewest cycles per workgroup): halfway
  // for the 128-MFMA 16-bit slice; halfway with loads spread over three
  // quarters of a slice for fp4 (about 3% fewer cycles than three quarters
  // and a half).  (fp8 and fp6 have K loops of their own.)
  static constexpr bool kFp46 = T::kDt == kFp4 || T::kFp6;
  static constexpr int kBarrierAt = kMfma / 2;
  static constexpr int kFreeAt = kBarrierAt;
  static constexpr int kWindow = kFp46 ? kMfma * 3 / 4 : kMfma / 2;
  static_assert(kFreeAt >= kNR && kFreeAt <= kBarrierAt, "slot-free barrier after this slice's reads");
  static_assert(kBarrierAt + kNR <= kMfma, "next-slice fragment reads must fit after the barrier");
  static_assert(kNR <= kBarrierAt, "this slice's second-substep reads come before the barrier");
  static_assert(kWindow <= kMfma && kWindow >= kLoads, "load window");

  // L2 prefetch (fp8, and fp4 whose scale rows are not dword-aligned; the
  // aligned fp4 kernel needs the LDS area for its scales and measured no
  // slower without it).  A slice's lines are first touched by its loads
  // into LDS, which have about one slice to land.  One dword of every
  // 128-byte line of slice kt + kPfDist is loaded early (into a scratch LDS
  // area, no registers), right after the last LDS load that the next
  // barrier waits for: that barrier waits with vmcnt(1), and the prefetch
  // has until the barrier after it to complete -- before the LDS loads of
  // slice kt + kPfDist are issued.  The workgroups of an XCD that share a
  // panel split its lines between them.  Measured: 7% fewer cycles for fp8
  // on the scaled 32 x 32 x 64 form, 1.5% on its 16 x 16 x 128 K loop
  // (which places the prefetch itself); none for the 16-bit kinds, which
  // do not use it.  (kPfAt: its place in the slices of run_slices.)
  static constexpr int kLastLoad = kFreeAt + (kLoads - 1) * kWindow / kLoads;
  static constexpr bool kPfHead = kLastLoad >= kMfma;  // last load in the next slice's head
  static constexpr int kPfAt = kPfHead ? kLastLoad - kMfma + 1 : kLastLoad + 1;
  // (Not for fp6, which has its own K loop.)
  static constexpr int kPfDist = T::kScaled && !T::kFp6 && !(T::kDt == kFp4 && T::kWholeK) ? 3 : 0;
  static_assert(kPfDist == 0 || !kPfHead || kPfAt < kBarrierAt, "prefetch goes before the barrier it may pass");
  static_assert(kPfDist == 0 || kPfHead || kPfAt < kMfma, "prefetch position");
  static_assert(kPfDist == 0 || kFreeAt == kBarrierAt, "the prefetch placement assumes one barrier per slice");

  // Loads of a slice issued in the tail of the slice kNS before it, before
  // MFMA `end` of that slice.
  static constexpr int tail_loads(int end = kMfma) {
    int n = 0;
    for (int i = 0; i < kLoads; ++i) n += kFreeAt + i * kWindow / kLoads < end;
    return n;
  }

  // Which load (0 .. kLoads - 1) of slice kt + kNS (TAIL, positions >=
  // kFreeAt of slice kt) or of slice kt + kNS - 1 (positions < kFreeAt of
  // slice kt, the continuation of the window opened in slice kt - 1) goes
  // out at MFMA Q; -1 for none.
  static constexpr int load_at(int Q, bool tail) {
    for (int i = 0; i < kLoads; ++i) {
      const int pos = kFreeAt + i * kWindow / kLoads;
      if (tail && pos == Q) return i;
      if (!tail && pos - kMfma == Q) return i;
    }
    return -1;
  }

  // fp8 fragments are 32 bytes, fp6 24 (six registers).
  using Frag = typename std::conditional<
      T::kFp6, i32x6, typename std::conditional<T::kDt == kFp8, i32x8, u32x4>::type>::type;
  using Acc = typename std::conditional<kW, f32x16, f32x4>::type;
  struct Frags {
    Frag x[kNBn], y[kNBm];
  };

  const Args &a;
  Slots slots;
  int tid, lane, wave, wave_m, wave_n, lane_sw;
  int m0, n0;
  int nk;
  int kK;     // K of this workgroup's range (all of K unless split)
  int split;  // K split: this workgroup's range
  int zt;  // the ragged last slice (or the only, all-zero one when K = 0); -1 if none
  typename std::conditional<T::kAK, PanelLoader<kLA>, MNLoader<TM>>::type la;
  typename std::conditional<T::kBK, PanelLoader<kLB>, MNLoader<TN>>::type lb;
  __amdgpu_buffer_rsrc_t pf_rsrc;
  uint32_t pf_off;
  // Block scales.  Each lane takes the scale bytes of one row per
  // "instruction" j (the wave's B rows 64 j .. + 63 for j < 2, its A rows
  // 64 (j - 2) .. + 63 after), addressed from the dword holding the row's
  // first scale byte.  Any 4 consecutive bytes of the row can be shifted
  // out of the two dwords from the one holding the first of them.  The
  // resource ends at the dword holding the tile's last scale byte; the
  // hardware checks each dword of a load against it (soffset included), so
  // dwords past it read 0.
  //  * fp8: group g (slices 4 g .. 4 g + 3) is one shifted dword, handed
  //    to the lanes that feed that row to the MFMA; the MFMA's byte select
  //    then picks the slice.  Each lane loads the group's dword pair itself
  //    (8 bytes, one load per instruction and group).
  //  * fp4 and fp6 stage the bytes of every row of the tile in LDS first
  //    (below).
  // Bytes past the row's last scale block (the next row's, in a padded
  // slice) are zeroed: the slices they would scale hold zeros, and a NaN
  // scale (0xff) would turn those zeros into NaN.
  __amdgpu_buffer_rsrc_t rss[2];  // B scales, A scales; based at the tile's first row, dword aligned
  uint32_t sc_off[4];             // per instruction: aligned byte offset of this lane's row, or kOOB
  uint32_t sc_sh[4];              // per instruction: byte shift of the row inside a dword pair
  u32x4 sc_ck[4], sc_ckn[4];      // fp6: chunks 2 p and 2 p + 1 of round p per instruction
  // fp4, fp6: the scale chunks of every row of the tile are loaded into LDS
  // once per workgroup (waves 0-1 the B rows, waves 2-3 the A rows), and
  // each wave then reads the rows its MFMAs take (every row feeds two
  // waves).
  //  * fp6: two consecutive chunks of a row at a time (a "group": chunks
  //    2 g and 2 g + 1).  A load instruction takes 32 rows, lanes l and
  //    l + 32 the two chunks of row l, so it touches 32 cache lines for
  //    1 KiB.  (Loading each wave's rows itself took 64 rows per
  //    instruction, one line per lane, and every row twice.)  st_off: this
  //    lane's row and chunk in the wave's first load instruction (aligned
  //    byte offset, or kOOB); the other three are 32, 64 and 96 rows
  //    further, by soffset.  Instruction i of wave w fills 1 KiB block
  //    4 w + i: chunk q of row 32 i + r of the wave's 128 at bytes 512 q +
  //    16 r.
  //  * fp4 with dword-aligned scale rows: groups as for fp6, in two 16 KiB
  //    slots (group g in slot g % 2), written from registers (sv4) rather
  //    than loaded into LDS directly; pair u of slices takes chunk u % 2 of
  //    group u / 2.
  //  * other fp4: one chunk at a time into a ring of three 8 KiB slots (chunk c
  //    in slot c % 3), row R of the tile (B rows 0-255, then A rows) at
  //    bytes 16 R of its slot; wave w's two load instructions take rows
  //    128 w + 64 i + l.  A pair of slices reads chunks u and u + 1 (a
  //    row's 16 scale bytes of the pair start inside chunk u when the row
  //    does not start on a dword).  st_off: this lane's row in the first
  //    instruction (aligned byte offset, or kOOB).
  static constexpr bool kStaged = T::kDt == kFp4 || T::kFp6;
  // fp4 with dword-aligned scale rows: two slots of groups, pair u in chunk
  // u % 2 of group u / 2.  (The L2 prefetch area goes to make room: 128 +
  // 32 KiB fill the LDS.)
  static constexpr bool kA4 = T::kDt == kFp4 && T::kWholeK;
  static constexpr int kStageBytes = kA4 ? 2 * 512 * 32 : T::kDt == kFp4 ? 3 * 512 * 16 : 512 * 32;
  static constexpr int kChunkStride = 16;  // row bytes between consecutive chunks
  uint32_t st_off;
  // fp4 (rows not dword-aligned): lane l = 16 g + r converts row r of
  // blocks 4 g .. 4 g + 3 (x blocks 0-7, then y blocks 0-7): sh4, the byte
  // shift of those rows inside a dword (16 rows apart, so the same for all
  // four); rd4, the offset of the first in a chunk slot; the current pair's
  // slot offsets (chunks u and u + 1) and the mask of the lane's bytes that
  // hold scale blocks of the row.  Aligned rows: rd4, the offset of the
  // first row in a group slot; sb4, the slot.
  uint32_t sh4, rd4;
  uint32_t keep4, cs4[2];
  u32x4 t4[4];
  uint32_t t4n[4];
  uint32_t w4[4], e4[4];  // one row's realigned dwords and their byte pairs
  u32x4 sv4[4];    // aligned rows: a group on its way from the L2 to its slot
  const LDS_AS uint8_t *sb4;  // aligned rows: the slot of the pair being converted
  // Per block (x blocks, then y blocks): fp8, the bytes of a group of 4
  // slices, converted into sc_cur block by block between the block's last
  // MFMA of one group and its first of the next.  fp4 and fp6 convert their
  // scales into the set their MFMAs read next (fp4: set (kt / 2) % 2 for a
  // pair of slices; fp6: set (k / 2) % 2 for K step k).
  int sc_cur[kNR];
  int sc_set[2][kNR];
  Acc acc[kNBn][kNBm];

  __device__ __forceinline__ Kernel(const Args &args, const Slots &s) : a(args), slots(s) {}

  // Fragment of one block of kBlk rows (B rows = C columns for x, A rows for
  // y), K substep `sub`, from a K-contiguous slot.
  __device__ __forceinline__ Frag read_rows(const LDS_AS uint8_t *slot, int row0, int sub) const {
    if constexpr (T::kDt == kFp8) {
      // 16 x 16 x 128 on fp8 (one K step per slice): lane l holds row l % 16
      // and K block l / 16 of the slice, 32 bytes: logical chunks 2 (l / 16)
      // and the one after, which the fp8 slots keep at chunks l / 16 and
      // l / 16 + 4 (before the row's permutation; chunk8_of), so that each
      // read has the 16-bit kinds' conflict-free pattern.
      const int g = lane >> 4;
      const LDS_AS uint8_t *p = slot + (row0 + (lane & 15)) * kRowBytes;
      u32x4 u = *(const LDS_AS u32x4 *)(p + ((g ^ lane_sw) << 4));
      u32x4 v = *(const LDS_AS u32x4 *)(p + (((g + 4) ^ lane_sw) << 4));
      i32x8 r;
      r[0] = u[0]; r[1] = u[1]; r[2] = u[2]; r[3] = u[3];
      r[4] = v[0]; r[5] = v[1]; r[6] = v[2]; r[7] = v[3];
      return r;
    } else {
      // 16 x 16 x 32: lane l holds row l % 16 and 8 elements of K: logical
      // chunk 4 sub + l / 16.  (fp4, 16 x 16 x 128: 32 elements, one K
      // block of 16 bytes, the same chunk.)
      const LDS_AS uint8_t *p = slot + (row0 + (lane & 15)) * kRowBytes;
      return *(const LDS_AS u32x4 *)(p + (((4 * sub + (lane >> 4)) ^ lane_sw) << 4));
    }
  }

  // Fragment of 16 columns col0 + l % 16 of a K-major slot W columns wide
  // (the [k][n] B slot, or the [k][m] A slot), K values 32 sub + 8 (l / 16)
  // + 0..7: the same lane layout as read_rows gives.  Each transpose read
  // gives a lane 4 K values of one column: in a 16-lane group, source lane
  // 4 e + q points at K row base + e, columns col0 + 4 q .. + 3, and lane i
  // receives column col0 + i.
  template <int W>
  __device__ __forceinline__ Frag read_cols(const LDS_AS uint8_t *slot, int col0, int sub) const {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int n = col0 + 4 * q;
    u32x4 r;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kr = 32 * sub + 8 * g + 4 * t + e;
      // (Masked to the slot so the compiler can see the read stays inside it
      // and needs no wait for loads into the other slot.)
      const int off = (kr * (2 * W) + (((n >> 3) ^ swz_nn<W>(kr)) << 4) + (n & 7) * 2) & (W * kRowBytes - 1);
      const LDS_AS uint8_t *p = slot + off;
      s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)p);
      u32x2 w = __builtin_bit_cast(u32x2, v);
      r[2 * t] = w[0];
      r[2 * t + 1] = w[1];
    }
    return r;
  }
  // Half t of the same fragment (K values 4 t .. 4 t + 3 of each lane's
  // eight): one transpose read into registers 2 t and 2 t + 1 of r.  (The
  // both-K-major kernels read whole fragments through read_cols: written
  // as two calls of this, that made their register allocation spill.)
  template <int W>
  __device__ __forceinline__ void read_cols_half(const LDS_AS uint8_t *slot, int col0, int sub, int t, Frag &r) const {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int n = col0 + 4 * q;
    const int kr = 32 * sub + 8 * g + 4 * t + e;
    // (Masked to the slot so the compiler can see the read stays inside it
    // and needs no wait for loads into the other slot.)
    const int off = (kr * (2 * W) + (((n >> 3) ^ swz_nn<W>(kr)) << 4) + (n & 7) * 2) & (W * kRowBytes - 1);
    const LDS_AS uint8_t *p = slot + off;
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)p);
    u32x2 w = __builtin_bit_cast(u32x2, v);
    r[2 * t] = w[0];
    r[2 * t + 1] = w[1];
  }

  // FIRST: the first K substep, whose MFMAs start from an accumulator of 0
  // (an inline constant), so the accumulators are never written by VALU code.
  // SEL: byte of the scale registers to use.
  template <bool FIRST, int SEL = 0>
  __device__ static __forceinline__ Acc mma(const Frag &x, const Frag &y, const Acc &c, int sx, int sy) {
    // The 16 x 16 forms are written as inline asm with the accumulator tied
    // in place ("+a"): with the builtin the register allocator rotates the
    // 64 accumulator tuples through spare registers on every loop trip.  The
    // compiler still places the LDS waits for the fragment inputs; the
    // accumulators are never written by VALU code and are read by it only
    // after fence_acc().
    if constexpr (T::kDt == kBf16) {
      Acc d = c;
      if constexpr (FIRST)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(d) : "v"(x), "v"(y));
      else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(x), "v"(y));
      return d;
    } else if constexpr (T::kDt == kF16) {
      Acc d = c;
      if constexpr (FIRST)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(d) : "v"(x), "v"(y));
      else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(d) : "v"(x), "v"(y));
      return d;
    } else if constexpr (T::kFp6) {
      // Format code 2 (OCP FP6 E2M3) or 3 (E3M2): 24 bytes, 32 elements per
      // lane, in the fragment's first six registers; byte SEL of each scale
      // VGPR (the K step).
      constexpr int F = T::kDt == kFp6E2M3 ? 2 : 3;
      const i32x8 x6 = {x[0], x[1], x[2], x[3], x[4], x[5], 0, 0};
      const i32x8 y6 = {y[0], y[1], y[2], y[3], y[4], y[5], 0, 0};
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x6, y6, c, F, F, SEL, sx, SEL, sy);
    } else {
      // The scaled 16 x 16 x 128 form.  fp4: format code 4 (OCP FP4 E2M1)
      // for both operands (cbsz, blgp), 16 bytes, 32 elements per lane.
      // fp8: format code 0 (OCP FP8 E4M3, the default), 32 bytes, 32
      // elements per lane.  Byte SEL of each scale VGPR: op_sel bit 0 and
      // op_sel_hi bit 1, the same for both.  Inline asm with the accumulator
      // tied in place, as for the 16-bit forms.
#define TGEMM_MFMA_S(SRC_C, OPS) \
  "v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, " SRC_C ", %3, %4 " OPS
      constexpr bool k4 = T::kDt == kFp4;
      Acc d = c;
      if constexpr (FIRST) {
        if constexpr (SEL == 0 && k4)
          asm volatile(TGEMM_MFMA_S("0", "op_sel:[0,0,0] op_sel_hi:[0,0,0] cbsz:4 blgp:4") : "=a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 1 && k4)
          asm volatile(TGEMM_MFMA_S("0", "op_sel:[1,1,0] op_sel_hi:[0,0,0] cbsz:4 blgp:4") : "=a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 2 && k4)
          asm volatile(TGEMM_MFMA_S("0", "op_sel:[0,0,0] op_sel_hi:[1,1,0] cbsz:4 blgp:4") : "=a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (k4)
          asm volatile(TGEMM_MFMA_S("0", "op_sel:[1,1,0] op_sel_hi:[1,1,0] cbsz:4 blgp:4") : "=a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 0)
          asm volatile(TGEMM_MFMA_S("0", "op_sel:[0,0,0] op_sel_hi:[0,0,0]") : "=a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 1)
          asm volatile(TGEMM_MFMA_S("0", "op_sel:[1,1,0] op_sel_hi:[0,0,0]") : "=a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 2)
          asm volatile(TGEMM_MFMA_S("0", "op_sel:[0,0,0] op_sel_hi:[1,1,0]") : "=a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else
          asm volatile(TGEMM_MFMA_S("0", "op_sel:[1,1,0] op_sel_hi:[1,1,0]") : "=a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
      } else {
        if constexpr (SEL == 0 && k4)
          asm volatile(TGEMM_MFMA_S("%0", "op_sel:[0,0,0] op_sel_hi:[0,0,0] cbsz:4 blgp:4") : "+a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 1 && k4)
          asm volatile(TGEMM_MFMA_S("%0", "op_sel:[1,1,0] op_sel_hi:[0,0,0] cbsz:4 blgp:4") : "+a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 2 && k4)
          asm volatile(TGEMM_MFMA_S("%0", "op_sel:[0,0,0] op_sel_hi:[1,1,0] cbsz:4 blgp:4") : "+a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (k4)
          asm volatile(TGEMM_MFMA_S("%0", "op_sel:[1,1,0] op_sel_hi:[1,1,0] cbsz:4 blgp:4") : "+a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 0)
          asm volatile(TGEMM_MFMA_S("%0", "op_sel:[0,0,0] op_sel_hi:[0,0,0]") : "+a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 1)
          asm volatile(TGEMM_MFMA_S("%0", "op_sel:[1,1,0] op_sel_hi:[0,0,0]") : "+a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else if constexpr (SEL == 2)
          asm volatile(TGEMM_MFMA_S("%0", "op_sel:[0,0,0] op_sel_hi:[1,1,0]") : "+a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
        else
          asm volatile(TGEMM_MFMA_S("%0", "op_sel:[1,1,0] op_sel_hi:[1,1,0]") : "+a"(d) : "v"(x), "v"(y), "v"(sx), "v"(sy));
      }
#undef TGEMM_MFMA_S
      return d;
    }
  }

  // Wait states after the last MFMA before VALU code reads the
  // accumulators.  The empty asm statements redefine every accumulator after
  // the s_nops, so no accumulator read can be scheduled above them.
  __device__ __forceinline__ void fence_acc() {
    mfma_fence();
#pragma unroll
    for (int i = 0; i < kNBn; ++i)
#pragma unroll
      for (int j = 0; j < kNBm; ++j) asm volatile("" : "+a"(acc[i][j]));
  }

  // Fragment read R (0 .. kNR - 1) of substep `sub` of slot S: x blocks,
  // then y blocks.
  template <int S, int R>
  __device__ __forceinline__ void read_one(Frags &f, int sub) const {
    if constexpr (R < kNBn) {
      if constexpr (T::kBK)
        f.x[R] = read_rows(slots.b[S], wave_n * kWN + R * kBlk, sub);
      else
        f.x[R] = read_cols<TN>(slots.b[S], wave_n * kWN + R * kBlk, sub);
    } else {
      if constexpr (T::kAK)
        f.y[R - kNBn] = read_rows(slots.a[S], wave_m * kWM + (R - kNBn) * kBlk, sub);
      else
        f.y[R - kNBn] = read_cols<TM>(slots.a[S], wave_m * kWM + (R - kNBn) * kBlk, sub);
    }
  }

  // Read pieces.  With exactly one K-major operand its fragments are read
  // as two pieces (the two transpose reads), each at an MFMA of its own, so
  // the reads of a substep spread over twice as many MFMAs: 3-4% fewer
  // cycles at 4096 x 4096 x 8192 (0.3-0.9% of the time under the power
  // cap).  With both operands K-major the split made the kernel spill, and
  // it stays off there.
  static constexpr int kPx = T::kBK ? 1 : 2, kPy = T::kAK ? 1 : 2;
  static constexpr int kPieces = kNBn * kPx + kNBm * kPy;
  static constexpr bool kSplit =
      !T::kScaled && (kPx == 2) != (kPy == 2) && kPieces <= kBarrierAt && kBarrierAt + kPieces <= kMfma;
  static constexpr int kNRead = kSplit ? kPieces : kNR;  // read positions per substep

  // Read piece P of substep `sub` of slot S (read R = P when not split).
  template <int S, int P>
  __device__ __forceinline__ void read_piece(Frags &f, int sub) const {
    if constexpr (!kSplit) {
      read_one<S, P>(f, sub);
    } else if constexpr (P < kNBn * kPx) {
      constexpr int R = P / kPx, t = P % kPx;
      if constexpr (kPx == 1)
        f.x[R] = read_rows(slots.b[S], wave_n * kWN + R * kBlk, sub);
      else
        read_cols_half<TN>(slots.b[S], wave_n * kWN + R * kBlk, sub, t, f.x[R]);
    } else {
      constexpr int R = (P - kNBn * kPx) / kPy, t = (P - kNBn * kPx) % kPy;
      if constexpr (kPy == 1)
        f.y[R] = read_rows(slots.a[S], wave_m * kWM + R * kBlk, sub);
      else
        read_cols_half<TM>(slots.a[S], wave_m * kWM + R * kBlk, sub, t, f.y[R]);
    }
  }

  template <int S, int... R>
  __device__ __forceinline__ void read_all(std::integer_sequence<int, R...>, Frags &f, int sub) const {
    (read_one<S, R>(f, sub), ...);
  }

  // Every load of slices 0 .. kNS - 2, slice s into slot s (the prologue).
  template <int... SL>
  __device__ __forceinline__ void load_slices(std::integer_sequence<int, SL...>) {
    (load_slice<SL>(), ...);
  }
  template <int SL>
  __device__ __forceinline__ void load_slice() {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_one<SL>(SL, i);
  }

  // Load instruction i (0 .. kLoads - 1) of slice kt into slot S: A panel,
  // then B.
  template <int S>
  __device__ __forceinline__ void load_one(int kt, int i) {
    if (i < kLA) {
      if constexpr (T::kScaled && !T::kWholeK)
        la.issue_masked(slots.a[S], wave, kt, kK, kSliceK, i);
      else if constexpr (T::kAK)
        la.issue(slots.a[S], wave, kt, i);
      else
        la.issue(slots.a[S], wave, kt, nk, i);
    } else {
      if constexpr (T::kScaled && !T::kWholeK)
        lb.issue_masked(slots.b[S], wave, kt, kK, kSliceK, i - kLA);
      else if constexpr (T::kBK)
        lb.issue(slots.b[S], wave, kt, i - kLA);
      else
        lb.issue(slots.b[S], wave, kt, nk, i - kLA);
    }
  }

  // Zero the chunks of the ragged last slice kt (in slot S) past column K,
  // after this wave's loads of it have landed and before the barrier that
  // lets the workgroup read it.  (K-major operands need nothing: their rows
  // past K read as zeros.  MXFP8 and MXFP4 with a ragged K check columns in
  // their loads; MXFP6 reads no byte past a row's last K step.)
  static constexpr bool kZeroTail = !T::kScaled && (T::kAK || T::kBK);
  template <int S>
  __device__ __forceinline__ void zero_tail(int kt) {
    if constexpr (T::kAK) la.zero_tail(slots.a[S], wave, lane, kt, kK, kSliceK);
    if constexpr (T::kBK) lb.zero_tail(slots.b[S], wave, lane, kt, kK, kSliceK);
    wait_vm_lgkm0<63>();
  }

  // One dword of each 128-byte line of slice kt of this workgroup's share of
  // the A and B panels; out-of-range rows and slices past K load nothing.
  __device__ __forceinline__ void prefetch(int kt) {
    const bool ok = kt * kSliceK < kK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(pf_rsrc, (LDS_AS void *)(slots.junk + wave * 256), 4,
                                             ok ? pf_off : kOOB, (uint32_t)kt * T::kSliceBytes, 0, 0);
  }

  // fp4, fp6: group g (chunks 2 g and 2 g + 1) of this wave's 128 rows into
  // the staging buffer.
  __device__ __forceinline__ void stage_group(int g, int slot = 0) {
    LDS_AS uint8_t *dst = slots.stage + slot * (512 * 32) + wave * 4 * 1024;
    // (A select on the wave-uniform operand, not rss[wave >> 1]: a dynamic
    // index into the member array would move the kernel's state to memory.)
    const __amdgpu_buffer_rsrc_t r = (wave >> 1) ? rss[1] : rss[0];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void *)(dst + i * 1024), 16, st_off,
                                               (uint32_t)(2 * kChunkStride * g + 32 * i * a.kb), 0, 0);
  }
  // Chunk Q of the staged group for every instruction's row into dst: 64
  // consecutive rows, two 512-byte runs (conflict-free 16-byte reads).
  template <int Q>
  __device__ __forceinline__ void fetch_chunk(u32x4 (&dst)[4]) {
    const int lp = (lane >> 5) * 1024 + (lane & 31) * 16 + Q * 512;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int blk = j < 2 ? wave_n * 4 + 2 * j : 8 + wave_m * 4 + 2 * (j - 2);
      dst[j] = *(const LDS_AS u32x4 *)(slots.stage + blk * 1024 + lp);
    }
  }

  // Mask keeping the bytes of a dword that holds scale blocks b .. b + 3 of
  // a row with kb blocks (nv = kb - b of them valid).
  __device__ static __forceinline__ uint32_t keep_mask(int nv) {
    return nv >= 4 ? ~0u : nv <= 0 ? 0u : (1u << (8 * nv)) - 1u;
  }

  // fp4 scales.  Inside a slice (8 K blocks of 32 elements, 16 bytes of a
  // row each), K step s of lane group g (lanes 16 g .. 16 g + 15) takes K
  // block 4 s + g; over a pair of slices (u: slices 2 u, 2 u + 1) K step
  // s = 2 (t % 2) + sub of slice t takes block 16 u + 4 s + g of the row,
  // byte s of the lane's scale dword for its block: bytes g, g + 4, g + 8,
  // g + 12 of the row's 16 for the pair, a column of the 4 x 4 byte matrix
  // they form.  Each lane converts four rows (all four columns of each) and
  // the lane groups then exchange the columns (exchange4).  (The order with
  // each lane group's two blocks of a slice side by side, 2 g + s, needed
  // no transpose but made the fragment reads conflict in LDS banks, half of
  // their cycles.)
  //
  // Rows whose scales start on a dword (kA4): groups of two chunks staged
  // through registers.  Group g + 1 is loaded in slice 4 g - 1, written to
  // its slot after the next barrier and published by the one after.
  __device__ __forceinline__ void load_group4(int g) {
    const __amdgpu_buffer_rsrc_t r = (wave >> 1) ? rss[1] : rss[0];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sv4[i] = __builtin_amdgcn_raw_buffer_load_b128(r, st_off, (uint32_t)(2 * kChunkStride * g + 32 * i * a.kb), 0);
  }
  __device__ __forceinline__ void store_group4(int g) {
    // The bytes stage_group would have written: chunk q of row 32 i + r of
    // the wave's 128 at block 4 w + i, bytes 512 q + 16 r.
    LDS_AS uint8_t *dst = slots.stage + (g & 1) * (512 * 32) + wave * 4096 + 16 * lane;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(LDS_AS u32x4 *)(dst + i * 1024) = sv4[i];
  }
  // Pair u (slices 2 u, 2 u + 1) is converted like the other rows' below
  // (each lane reads four rows and the lane groups exchange their dwords),
  // without the realignment: the slot of group u / 2.  (Chosen between two
  // pointers into the buffer rather than as an offset added to it: with an
  // offset the compiler lost track of which LDS array the reads address,
  // and made each wait for all the panel loads in flight.)
  __device__ __forceinline__ void begin_pair4a(int u) {
    sb4 = ((u >> 1) & 1) ? slots.stage + 512 * 32 : slots.stage;
  }
  // Row K (16 K + r of the lane's four 16-row blocks, in 32-row blocks of
  // the slot) of chunk Q (= u % 2) of the group.
  template <int K, int Q>
  __device__ __forceinline__ void read_row4a() {
    t4[K] = *(const LDS_AS u32x4 *)(sb4 + rd4 + Q * 512 + (K >> 1) * 1024 + (K & 1) * 256);
  }

  // Other rows (a dword may start inside a row's scales, or K not a
  // multiple of the slice): chunk c of this wave's 128 rows into slot c % 3
  // of a ring; a pair's 16 bytes of a row start inside chunk u.
  __device__ __forceinline__ void stage_chunk4(int c) {
    LDS_AS uint8_t *dst = slots.stage + (c % 3) * 8192 + wave * 2048;
    const __amdgpu_buffer_rsrc_t r = (wave >> 1) ? rss[1] : rss[0];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS_AS void *)(dst + i * 1024), 16, st_off,
                                               (uint32_t)(kChunkStride * c + 64 * i * a.kb), 0, 0);
  }
  // Pair u: the slot offsets of chunks u and u + 1, and the mask of the
  // bytes of this lane's dwords that hold scale blocks of the row (byte s:
  // block 16 u + 4 s + g below kb).
  __device__ __forceinline__ void begin_pair4(int u) {
    cs4[0] = (uint32_t)((u % 3) * 8192);
    cs4[1] = (uint32_t)(((u + 1) % 3) * 8192);
    const int left = a.kb - 16 * u - (lane >> 4);
    keep4 = keep_mask(left <= 0 ? 0 : (left + 3) >> 2);
  }
  // This lane's four rows (row r of blocks 4 g' .. 4 g' + 3 for lane group
  // g'): chunk u and the first dword of chunk u + 1.  The reads are written
  // out, with their wait, in one asm statement: as ordinary loads the
  // compiler cannot tell them from the staging loads into the same buffer
  // still in flight, and made them wait for every outstanding global load
  // (about 10% of the K loop).  Every staging load they depend on was
  // waited for by an earlier barrier.
  __device__ __forceinline__ void read_scales4() {
    const uint32_t p0 = (uint32_t)(uintptr_t)slots.stage + rd4 + cs4[0];
    const uint32_t p1 = (uint32_t)(uintptr_t)slots.stage + rd4 + cs4[1];
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:256\n\t"
        "ds_read_b128 %2, %8 offset:512\n\t"
        "ds_read_b128 %3, %8 offset:768\n\t"
        "ds_read_b32 %4, %9\n\t"
        "ds_read_b32 %5, %9 offset:256\n\t"
        "ds_read_b32 %6, %9 offset:512\n\t"
        "ds_read_b32 %7, %9 offset:768\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(t4[0]), "=&v"(t4[1]), "=&v"(t4[2]), "=&v"(t4[3]), "=&v"(t4n[0]), "=&v"(t4n[1]), "=&v"(t4n[2]),
          "=&v"(t4n[3])
        : "v"(p0), "v"(p1)
        : "memory");
  }
  // Piece P (0-3) of row K: the dword of lane group j, bytes j, j + 4,
  // j + 8, j + 12 of the row's 16 for the pair, into slot j of the row's
  // block (sc_set[SET][4 j + K]) until exchange4 hands it to lane group j.
  template <int SET, int K, int P>
  __device__ __forceinline__ void convert_scale4() {
    const u32x4 &c = t4[K];
    // w0 .. w3: the row's 16 bytes of the pair (realigned to its first
    // block unless aligned); e0 .. e3 pair up the bytes of w0, w1 and of
    // w2, w3; column j = (w0.j, w1.j, w2.j, w3.j).  At most three VALU
    // instructions per piece, so that each fits beside one MFMA.
    if constexpr (kA4) {
      if constexpr (P == 0) {
        e4[0] = __builtin_amdgcn_perm(c[1], c[0], 0x05010400u);  // w0.0 w1.0 w0.1 w1.1
        e4[1] = __builtin_amdgcn_perm(c[1], c[0], 0x07030602u);  // w0.2 w1.2 w0.3 w1.3
      } else if constexpr (P == 1) {
        e4[2] = __builtin_amdgcn_perm(c[3], c[2], 0x05010400u);
        e4[3] = __builtin_amdgcn_perm(c[3], c[2], 0x07030602u);
      }
    } else if constexpr (P == 0) {
      w4[0] = __builtin_amdgcn_alignbyte(c[1], c[0], sh4);
      w4[1] = __builtin_amdgcn_alignbyte(c[2], c[1], sh4);
      w4[2] = __builtin_amdgcn_alignbyte(c[3], c[2], sh4);
    } else if constexpr (P == 1) {
      w4[3] = __builtin_amdgcn_alignbyte(t4n[K], c[3], sh4);
      e4[0] = __builtin_amdgcn_perm(w4[1], w4[0], 0x05010400u);
      e4[1] = __builtin_amdgcn_perm(w4[1], w4[0], 0x07030602u);
    }
    if constexpr (!kA4 && P == 2) {
      e4[2] = __builtin_amdgcn_perm(w4[3], w4[2], 0x05010400u);
      e4[3] = __builtin_amdgcn_perm(w4[3], w4[2], 0x07030602u);
      sc_set[SET][K] = (int)__builtin_amdgcn_perm(e4[2], e4[0], 0x05040100u);
    } else if constexpr (kA4 && P == 2) {
      sc_set[SET][K] = (int)__builtin_amdgcn_perm(e4[2], e4[0], 0x05040100u);
      sc_set[SET][4 + K] = (int)__builtin_amdgcn_perm(e4[2], e4[0], 0x07060302u);
    }
    if constexpr (P == 3) {
      if constexpr (!kA4) sc_set[SET][4 + K] = (int)__builtin_amdgcn_perm(e4[2], e4[0], 0x07060302u);
      sc_set[SET][8 + K] = (int)__builtin_amdgcn_perm(e4[3], e4[1], 0x05040100u);
      sc_set[SET][12 + K] = (int)__builtin_amdgcn_perm(e4[3], e4[1], 0x07060302u);
    }
  }
  // Lane group g holds in slot j the dwords of lane group j for its blocks
  // 4 g .. + 3; lane group j needs them in slot g.  A transpose of (lane
  // group, slot) in two stages: the halves of the wave exchange slots 2-3
  // against 0-1, then odd and even 16-lane rows exchange odd slots against
  // even ones; after both, slot g of lane l holds its dwords for blocks
  // 4 g .. 4 g + 3.  Swaps 2 Q and 2 Q + 1 of stage P.
  template <int SET, int P, int Q>
  __device__ __forceinline__ void exchange4() {
#pragma unroll
    for (int n = 2 * Q; n < 2 * Q + 2; ++n) {
      const int h = n / 4, k = n % 4;
      const int d = P == 0 ? 4 * h + k : 8 * h + k, e = P == 0 ? d + 8 : d + 4;
      if constexpr (P == 0) {
        const auto r = __builtin_amdgcn_permlane32_swap(sc_set[SET][d], sc_set[SET][e], false, false);
        sc_set[SET][d] = (int)r[0];
        sc_set[SET][e] = (int)r[1];
      } else {
        const auto r = __builtin_amdgcn_permlane16_swap(sc_set[SET][d], sc_set[SET][e], false, false);
        sc_set[SET][d] = (int)r[0];
        sc_set[SET][e] = (int)r[1];
      }
    }
  }
  // Dwords 2 Q and 2 Q + 1 masked to the scale blocks of the row.
  template <int SET, int Q>
  __device__ __forceinline__ void mask4() {
    sc_set[SET][2 * Q] &= (int)keep4;
    sc_set[SET][2 * Q + 1] &= (int)keep4;
  }
  // Step N of a pair's conversion, one per MFMA: the four rows' reads (0),
  // their conversion (4 + 4 K + P), the exchange (20-27) and the masks
  // (28-35).
  template <int SET, int N, int Q = 0>
  __device__ __forceinline__ void pair4_step() {
    if constexpr (kA4) {
      // Aligned rows: reads (0-3), their conversion four MFMAs later (8-23),
      // the exchange (24-31); whole blocks of the row, nothing to mask.
      if constexpr (N < 4) read_row4a<N, Q>();
      else if constexpr (N >= 8 && N < 24) convert_scale4<SET, (N - 8) / 4, (N - 8) % 4>();
      else if constexpr (N >= 24 && N < 32) exchange4<SET, (N - 24) / 4, (N - 24) % 4>();
    } else if constexpr (N == 0) read_scales4();
    else if constexpr (N >= 4 && N < 20) convert_scale4<SET, (N - 4) / 4, (N - 4) % 4>();
    else if constexpr (N >= 20 && N < 28) exchange4<SET, (N - 20) / 4, (N - 20) % 4>();
    else if constexpr (N >= 28 && N < 36) mask4<SET, N - 28>();
  }
  static constexpr int kPair4Steps = 36;

  // Every step at once (the prologue: pair 0 into set 0).
  template <int... N>
  __device__ __forceinline__ void convert_pair4(std::integer_sequence<int, N...>) {
    (pair4_step<0, N, 0>(), ...);
  }

  // fp8: the scale bytes of group g (slices 4 g .. 4 g + 3) of each
  // instruction's row, as the two dwords from the one holding the row's
  // byte 4 g (one 8-byte load per instruction and group, two slices ahead
  // of their use; past the resource's end they read 0), shifted out and
  // handed to the scale registers of the instruction's four blocks.
  // Instruction J's lane l holds row 64 (J % 2) + l of the wave's x rows (J
  // < 2) or y rows (rows 64 apart share their shift, as 64 kb is a multiple
  // of 4); block 4 (J % 2) + c is rows 16 c .. 16 c + 15 of them, which
  // lane l (every 16-lane row) takes from lane 16 c + l % 16: a swap of the
  // wave halves (lane l then holds rows 32 h + l % 32 for h = 0, 1), then
  // of odd and even 16-lane rows of each (rows 32 h + 16 c' + l % 16).
  u32x2 sc_pr[4];
  __device__ __forceinline__ void load_pairs8(int g) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sc_pr[j] = __builtin_amdgcn_raw_buffer_load_b64(rss[j >> 1], sc_off[j], (uint32_t)(4 * g), 0);
  }
  template <int J>
  __device__ __forceinline__ void convert8(int g) {
    const uint32_t keep = keep_mask(a.kb - 4 * g);
    const uint32_t d = __builtin_amdgcn_alignbyte(sc_pr[J][1], sc_pr[J][0], sc_sh[J & 2]) & keep;
    const auto h = __builtin_amdgcn_permlane32_swap(d, d, false, false);
    const auto lo = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
    sc_cur[4 * J] = (int)lo[0];
    sc_cur[4 * J + 1] = (int)lo[1];
    sc_cur[4 * J + 2] = (int)hi[0];
    sc_cur[4 * J + 3] = (int)hi[1];
  }

  // MFMA Q (0 .. kMfma - 1) of slice kt held in slot S.  Substep Q / kPerSub;
  // inside it x block q / kNBm times y block q % kNBm (in reverse order
  // under odd x blocks).  Interleaved with it:
  //  * Q < kNRead: read piece Q of substep 1 of this slot into f1;
  //  * before Q = kBarrierAt: wait for this wave's loads of slice kt + 1 and
  //    synchronise the workgroup (slot kt % kNS is then free);
  //  * from kBarrierAt: reads of substep 0 of slice kt + 1 into f0;
  //  * the loads of slice kt + kNS into this slot, and the end of those of
  //    slice kt + kNS - 1 into the slot before, as load_at places them.
  template <int S, int JB, bool FIRST, int Q>
  __device__ __forceinline__ void mfma_one(int kt, Frags &f0, Frags &f1) {
    constexpr int SUB = Q / kPerSub, q = Q % kPerSub;
    // The y blocks snake (forward under even x blocks, backward under odd
    // ones), so the two MFMAs at each turn share their y operand: less
    // operand switching, 0.4% faster under the power cap at 4096 x 4096 x
    // 8192 bf16, 0.2-0.9% for the block-scaled kinds.
    constexpr int I = q / kNBm, J0 = q % kNBm;
    constexpr int J = (I & 1) ? kNBm - 1 - J0 : J0;
    constexpr int kHead = load_at(Q, false), kTail = load_at(Q, true);
    if constexpr (kFreeAt < kBarrierAt && Q == kFreeAt) {
      // Every wave's reads of this slot are done: its loads may start.
      wait_vm_lgkm0<63>();
      barrier();
    }
    if constexpr (Q == kBarrierAt) {
      // The prefetch issued after the last needed load may be outstanding
      // (none precedes the first slice's barrier in the tail placement).
      // The loads of slices kt + 2 .. kt + kNS - 1 may be outstanding too,
      // and those of slice kt + kNS issued since kFreeAt (the newest).
      constexpr int kPfOut = kPfDist > 0 && (kPfHead || !FIRST) ? 1 : 0;
      wait_vm_lgkm0<(kNS - 2) * kLoads + kPfOut + tail_loads(kBarrierAt)>();
      if constexpr (kZeroTail)
        if (kt + 1 == zt) zero_tail<(S + 1) % kNS>(kt + 1);
      barrier();
      // fp4 (JB = kt % 4), rows not dword-aligned: in an even slice, every
      // wave's reads of chunk kt / 2 - 1 lie behind this barrier, and chunk
      // kt / 2 + 3 goes into its slot; the next barrier waits for it.
      //    Aligned rows: at kt = 4 g - 1, group g + 1 is loaded into
      //    registers; at kt = 4 g (this barrier waited for it) it goes into
      //    the slot of group g - 1, whose last reads (pair 2 g - 1) were in
      //    slice 4 g - 4; the barrier of slice 4 g + 1 publishes it for pair
      //    2 g + 2, converted in slice 4 g + 2.
      if constexpr (kA4) {
        if constexpr (JB == 3) load_group4(((kt + 1) >> 2) + 1);
        if constexpr (JB == 0) store_group4((kt >> 2) + 1);
      } else if constexpr (T::kDt == kFp4) {
        if constexpr ((JB & 1) == 0) stage_chunk4((kt >> 1) + 3);
      }
    }
    if constexpr (T::kDt == kFp4 && (JB & 1) == 0) {
      // An even slice kt converts the scales of the pair after the current
      // one (u = kt / 2 + 1) into the set the previous pair used: chunks u
      // and u + 1, staged and published by the barriers of slices kt - 2 and
      // kt - 1 or earlier.  One step per MFMA, ending at the barrier; the
      // reads (whose wait takes every LDS read in flight) go out several
      // MFMAs after this slice's substep-1 fragment reads.
      constexpr int N = Q - (kBarrierAt - kPair4Steps), SET = ((JB >> 1) + 1) & 1;
      static_assert(kNRead + 1 + kPair4Steps <= kBarrierAt, "a pair's conversion fits before the barrier");
      if constexpr (N == -1) {
        if constexpr (kA4)
          begin_pair4a((kt >> 1) + 1);
        else
          begin_pair4((kt >> 1) + 1);
      }
      // (Aligned rows: u = kt / 2 + 1 is odd for kt % 4 = 0, chunk 1 of its group.)
      if constexpr (N >= 0 && N < kPair4Steps) pair4_step<SET, N, JB == 0 ? 1 : 0>();
    }
    if constexpr (Q < kNRead) read_piece<S, Q>(f1, 1);
    if constexpr (Q >= kBarrierAt && Q - kBarrierAt < kNRead) read_piece<(S + 1) % kNS, Q - kBarrierAt>(f0, 0);
    if constexpr (kHead >= 0) load_one<(S + kNS - 1) % kNS>(kt + kNS - 1, kHead);
    if constexpr (kTail >= 0) load_one<S>(kt + kNS, kTail);
    if constexpr (kPfDist > 0 && Q == kPfAt) prefetch(kt + kPfDist);
    const Frags &f = SUB == 0 ? f0 : f1;
    if constexpr (T::kDt == kFp4) {
      // A set per pair of slices (kt / 2 % 2), byte 2 (kt % 2) + SUB.
      constexpr int SET4 = (JB >> 1) & 1, SEL4 = 2 * (JB & 1) + SUB;
      acc[I][J] = mma<FIRST && SUB == 0, SEL4>(f.x[I], f.y[J], acc[I][J], sc_set[SET4][I], sc_set[SET4][kNBn + J]);
    }
    else
      acc[I][J] = mma<FIRST && SUB == 0>(f.x[I], f.y[J], acc[I][J], 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  template <int S, int JB, bool FIRST, int... Q>
  __device__ __forceinline__ void slice_seq(std::integer_sequence<int, Q...>, int kt, Frags &f0, Frags &f1) {
    (mfma_one<S, JB, FIRST, Q>(kt, f0, f1), ...);
  }

  // One K slice kt from slot S (its substep-0 fragments already in f0); JB
  // = kt % 4 for fp4.
  template <int S, int JB, bool FIRST = false>
  __device__ __forceinline__ void step(int kt, Frags &f0, Frags &f1) {
    slice_seq<S, JB, FIRST>(std::make_integer_sequence<int, kMfma>(), kt, f0, f1);
  }

  __device__ __forceinline__ void run() {
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    wave_m = wave >> 1;
    wave_n = wave & 1;
    lane_sw = swz(lane & 15);  // fragment blocks start at multiples of 16 rows

    int tm, tn;
    const int tiles = a.tiles_m * a.tiles_n;
    const int wg = (int)blockIdx.x;
    split = SPLIT ? wg / tiles : 0;
    tile_of(SPLIT ? wg - split * tiles : wg, tiles, a.tiles_m, a.tiles_n, tm, tn);
    m0 = tm * TM;
    n0 = tn * TN;
    // This workgroup's K range: all of K, or (split) slices [kq s, kq s + kq)
    // clipped to K, i.e. the K elements from k0 on.  The loaders are based at
    // column (K-contiguous) or row (K-major) k0 and see a K of kK.
    int k0 = 0;
    kK = a.K;
    nk = a.ksteps;
    if constexpr (SPLIT) {
      const int s0 = split * a.kq;
      nk = min(a.kq, a.ksteps - s0);
      k0 = s0 * kSliceK;
      kK = min(a.K - k0, nk * kSliceK);
    }
    const int K = kK;
    zt = K % kSliceK != 0 || nk == 0 ? (nk > 0 ? nk - 1 : 0) : -1;

    if constexpr (T::kFp6)
      ;  // fp6 sets up its own loads (run6)
    else if constexpr (T::kAK)
      la.init(a.A + ((size_t)m0 * a.lda + k0) * kElem, min(a.M - m0, TM), K, a.lda, kElem, kSliceK, wave, lane);
    else
      la.init(a.A + (size_t)k0 * a.lda * kElem, K, a.M, m0, a.lda, wave, lane);
    if constexpr (T::kFp6)
      ;
    else if constexpr (T::kBK)
      lb.init(a.B + ((size_t)n0 * a.ldb + k0) * kElem, min(a.N - n0, TN), K, a.ldb, kElem, kSliceK, wave, lane);
    else
      lb.init(a.B + (size_t)k0 * a.ldb * kElem, K, a.N, n0, a.ldb, wave, lane);
    if constexpr (kPfDist > 0) {
      // Waves 0-1 take 32 rows of the A panel (its share among the 8 tile
      // columns of an XCD's block), waves 2-3 take 64 rows of the B panel
      // (its share among the 4 tile rows).
      const bool is_a = wave < 2;
      pf_rsrc = is_a ? la.rsrc : lb.rsrc;
      const int rows_valid = is_a ? min(a.M - m0, TM) : min(a.N - n0, TN);
      const int r = is_a ? 32 * (tn & 7) + 16 * wave + (lane & 15) : 64 * (tm & 3) + 32 * (wave - 2) + (lane & 31);
      const bool active = is_a ? lane < 16 : lane < 32;
      pf_off = active && r < rows_valid ? (uint32_t)r * (uint32_t)(is_a ? a.lda : a.ldb) * (uint32_t)kElem : kOOB;
    }
    if constexpr (T::kScaled) {
      // Each operand's scale rows of this tile through a resource based at
      // the dword holding its first byte; its size is rounded up to whole
      // dwords (the extra bytes lie in the same dword as the last scale
      // byte, so in the same page).
#pragma unroll
      for (int op = 0; op < 2; ++op) {
        const uintptr_t start = (uintptr_t)(op ? a.SA + (size_t)m0 * a.kb : a.SB + (size_t)n0 * a.kb);
        const uint32_t mis = (uint32_t)(start & 3);
        const int rows_valid = op ? min(a.M - m0, TM) : min(a.N - n0, TN);
        rss[op] = make_rsrc((const void *)(start - mis), (mis + (uint32_t)rows_valid * (uint32_t)a.kb + 3) & ~3u);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 2 * op + h;
          const int r = (op ? wave_m : wave_n) * 128 + 64 * h + lane;
          const uint32_t pos = mis + (uint32_t)r * (uint32_t)a.kb;
          sc_off[j] = r < rows_valid ? (pos & ~3u) : kOOB;
          sc_sh[j] = pos & 3;
        }
        if constexpr (kA4) {
          if (op == (wave >> 1)) {
            // As fp6: rows r + 32, r + 64, r + 96 are 32 kb bytes apart.
            const int r = (wave & 1) * 128 + (lane & 31);
            const uint32_t pos = (uint32_t)r * (uint32_t)a.kb;
            st_off = r < rows_valid ? pos + (uint32_t)(kChunkStride * (lane >> 5)) : kOOB;
          }
          // Lane 16 g + r reads rows 64 (g % 2) + 16 k + r of the wave's x
          // rows (g < 2) or y rows: 32-row block op 8 + 4 wave + 2 (g % 2)
          // + k / 2 of the slot, row 16 (k % 2) + r.
          if (op == (lane >> 5)) {
            const int blk = op * 8 + (op ? wave_m : wave_n) * 4 + 2 * ((lane >> 4) & 1);
            rd4 = (uint32_t)(1024 * blk + 16 * (lane & 15));
          }
        } else if constexpr (T::kDt == kFp4) {
          if (op == (wave >> 1)) {
            // Row r + 64 is 64 kb bytes further, and so is its aligned
            // offset.  (Past the last row the resource ends: zeros.)
            const int r = (wave & 1) * 128 + lane;
            const uint32_t pos = mis + (uint32_t)r * (uint32_t)a.kb;
            st_off = r < rows_valid ? (pos & ~3u) : kOOB;
          }
          // Lane 16 g + r converts rows 64 (g % 2) + 16 k + r of the wave's
          // x rows (g < 2) or y rows: 16 kb bytes apart, so one shift.
          if (op == (lane >> 5)) {
            const int r = (op ? wave_m : wave_n) * 128 + 64 * ((lane >> 4) & 1) + (lane & 15);
            sh4 = (mis + (uint32_t)r * (uint32_t)a.kb) & 3;
            rd4 = (uint32_t)(16 * ((op ? 256 : 0) + r));
          }
        } else if constexpr (kStaged) {
          if (op == (wave >> 1)) {
            // Rows r + 32, r + 64, r + 96 are 32 kb bytes apart each, and so
            // are their aligned offsets.
            const int r = (wave & 1) * 128 + (lane & 31);
            const uint32_t pos = mis + (uint32_t)r * (uint32_t)a.kb;
            st_off = r < rows_valid ? (pos & ~3u) + (uint32_t)(kChunkStride * (lane >> 5)) : kOOB;
          }
        }
      }
      if constexpr (T::kFp6) {
        // (fp4 and fp8 start their accumulators from the MFMA's constant 0.)
#pragma unroll
        for (int i = 0; i < kNBn; ++i)
#pragma unroll
          for (int j = 0; j < kNBm; ++j) acc[i][j] = Acc{};
      }
    }
    if constexpr (T::kFp6)
      run6();
    else if constexpr (T::kDt == kFp8)
      run8();
    else
      run_slices();
  }

  // The K loop over slices (the 16-bit kinds and fp4), from its prologue to
  // the epilogue.
  __device__ __forceinline__ void run_slices() {

    // Prologue: the first scale chunks, slice 0 into slot 0, the loads of
    // slice 1 that a previous slice's tail would have issued; wait for all
    // but those, and convert slice 0's scales.  (With K = 0 every slice is
    // all zeros.)
    if constexpr (kA4) {
      load_group4(0);
    } else if constexpr (T::kDt == kFp4) {
      stage_chunk4(0);
      stage_chunk4(1);
      stage_chunk4(2);
    }
    load_slices(std::make_integer_sequence<int, kNS - 1>());
    constexpr int kTailLoads = tail_loads();
#pragma unroll
    for (int i = 0; i < kTailLoads; ++i) load_one<kNS - 1>(kNS - 1, i);
    wait_vm_lgkm0<(kNS - 2) * kLoads + kTailLoads>();
    if constexpr (kA4) {
      // Group 0 into its slot (group 1 follows it into registers; slice 0's
      // barrier stores it); every wave's part is in LDS after the barrier;
      // then pair 0's scales into set 0.
      store_group4(0);
      // (The LDS writes may read their registers after a later load has
      // started: wait for them before the registers take group 1.)
      wait_vm_lgkm0<63>();
      load_group4(1);
      barrier();
      begin_pair4a(0);
      convert_pair4(std::make_integer_sequence<int, kPair4Steps>());
    } else if constexpr (T::kDt == kFp4) {
      // Every wave's staged chunks 0-2 are in LDS after this barrier.
      barrier();
      begin_pair4(0);
      convert_pair4(std::make_integer_sequence<int, kPair4Steps>());
    }
    if constexpr (kZeroTail)
      if (zt == 0) zero_tail<0>(0);
    barrier();
    Frags f0, f1;
    read_all<0>(std::make_integer_sequence<int, kNR>(), f0, 0);
    // Slice 0 starts the accumulators; then the slices go round the ring a
    // whole number of slots at a time (fp4: four, for its scale chunks), and
    // the one to three left after the last round run on their own, so no
    // slice past nk is computed.
    step<0, 0, true>(0, f0, f1);
    if constexpr (T::kDt == kFp4) {
      int kt = 1;
      for (; kt + 3 < nk; kt += 4) {
        step<1, 1>(kt, f0, f1);
        step<0, 2>(kt + 1, f0, f1);
        step<1, 3>(kt + 2, f0, f1);
        step<0, 0>(kt + 3, f0, f1);
      }
      if (kt < nk) step<1, 1>(kt, f0, f1);
      if (kt + 1 < nk) step<0, 2>(kt + 1, f0, f1);
      if (kt + 2 < nk) step<1, 3>(kt + 2, f0, f1);
    } else if constexpr (kNS == 4) {
      int kt = 1;
      for (; kt + 3 < nk; kt += 4) {
        step<1, 1>(kt, f0, f1);
        step<2, 2>(kt + 1, f0, f1);
        step<3, 3>(kt + 2, f0, f1);
        step<0, 0>(kt + 3, f0, f1);
      }
      if (kt < nk) step<1, 1>(kt, f0, f1);
      if (kt + 1 < nk) step<2, 2>(kt + 1, f0, f1);
      if (kt + 2 < nk) step<3, 3>(kt + 2, f0, f1);
    } else {
      int kt = 1;
      for (; kt + 1 < nk; kt += 2) {
        step<1, 1>(kt, f0, f1);
        step<0, 2>(kt + 1, f0, f1);
      }
      if (kt < nk) step<1, 1>(kt, f0, f1);
    }
    // Drain the loads still in flight into the slots before the workgroup
    // can finish.
    wait_vm_lgkm0<0>();
    fence_acc();
    if constexpr (SPLIT)
      epilogue_partial(split);
    else
      epilogue();
  }

  // -------------------------------------------------------------------------
  // fp8: the scaled 16 x 16 x 128 MFMA.
  //
  // A slice (128 bytes of every row, one K step of 128) is 64 MFMAs per
  // wave, on one set of fragments (16 of 32 bytes: 128 registers; two sets,
  // as the other kinds keep, do not fit beside the accumulators): each
  // fragment of the next slice is read into the registers of this slice's
  // once their last MFMA has issued (the MFMA reads them as it issues; the
  // LDS data returns later), at the positions f8::schedule gives.  Two
  // slots: the barrier before MFMA kB8 of slice kt waits for this wave's
  // loads of slice kt + 1 and publishes them; every read of slot kt % 2 was
  // issued before it (the last in the head of slice kt), so the loads of
  // slice kt + 2 go into that slot from there on, one every two MFMAs, and
  // the L2 prefetch of slice kt + 3 after the last of them.  The scales of
  // group g (slices 4 g .. 4 g + 3) are loaded in slice 4 g - 3 and
  // converted in slices 4 g - 1 and 4 g (kCv8).  Measured at 4096^3 against
  // the scaled 32 x 32 x 64 form: 2-4% less time (a 6% higher clock under
  // the power limit at 2% more cycles, mostly the form's issue: 32.8
  // cycles per MFMA against 32.1 for half a 32 x 32 x 64 one).  The
  // barrier at 16 or 32, the loads further apart, or the y blocks in x-block
  // pairs rather than quadrants measured no better.
  static constexpr int kB8 = 24;
  static constexpr f8::Sched kSch8[2] = {f8::schedule(0, kB8), f8::schedule(1, kB8)};
  // Position of the conversion of instruction J's scales (blocks 4 J ..
  // 4 J + 3: x blocks for J < 2, y blocks after) in slice 4 g - 1 (phase
  // 1), or in slice 4 g (phase 0) at kM and on.
  static constexpr int kCv8[4] = {33, f8::kM + 5, 56, f8::kM + 3};

  // Load instruction i (A panel for i < kLA, then B) of slice kt into slot
  // S, as PanelLoader::issue / issue_masked, with the lane's offset rebuilt
  // from one of two bases (instructions i and i + 2 are 16 rows apart)
  // rather than held per instruction: 12 registers fewer, which the fp8
  // kernel needs.  A row past the panel's last needs no out-of-range
  // offset: it starts at least ld >= K bytes past the start of the last
  // row, at or past the end of the resource.
  // fp8 slots keep logical chunk 2 g + h of a row at chunk g + 4 h (then
  // permuted by the row like the other kinds'): this is the logical chunk
  // at chunk q.  (With the logical order the fragment reads met 2-way bank
  // conflicts: every read took twice its cycles.)
  __device__ static __forceinline__ int chunk8_of(int q) { return ((q & 3) << 1) | (q >> 2); }
  uint32_t lo8[2][2];  // [B][parity]: this lane's chunk offset at slice 0 in instruction 0 / 1
  int kcol8[2];        // element column of this lane's chunk inside a slice (parity)
  template <int S>
  __device__ __forceinline__ void load8(int kt, int i) {
    const bool isb = i >= kLA;
    const int ii = isb ? i - kLA : i;
    const uint32_t ld = (uint32_t)(isb ? a.ldb : a.lda);
    uint32_t v = lo8[isb][ii & 1] + (uint32_t)(ii >> 1) * 16u * ld;
    if constexpr (!T::kWholeK) v = kt * kSliceK + kcol8[ii & 1] < kK ? v : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(isb ? lb.rsrc : la.rsrc,
                                             (LDS_AS void *)((isb ? slots.b[S] : slots.a[S]) + (wave * kLA + ii) * 1024),
                                             16, v, (uint32_t)kt * T::kSliceBytes, 0, 0);
  }

  // Fragment F (x blocks, then y blocks) of the slice in slot S.
  template <int S, int F>
  __device__ __forceinline__ void read8(Frags &f) const {
    if constexpr (F < kNBn)
      f.x[F] = read_rows(slots.b[S], wave_n * kWN + F * kBlk, 0);
    else
      f.y[F - kNBn] = read_rows(slots.a[S], wave_m * kWM + (F - kNBn) * kBlk, 0);
  }
  // The reads at MFMA Q of a slice of phase P in slot S: the next slice's
  // fragments placed here, and this slice's placed at kM + Q by the
  // previous slice (none in the first slice, whose fragments the prologue
  // reads).
  template <int S, int P, int Q, bool FIRST, int F>
  __device__ __forceinline__ void read8_at(Frags &f) const {
    if constexpr (kSch8[P].pos[F] == Q) read8<S ^ 1, F>(f);
    if constexpr (!FIRST && kSch8[P ^ 1].pos[F] == f8::kM + Q) read8<S, F>(f);
  }
  template <int S, int P, int Q, bool FIRST, int... F>
  __device__ __forceinline__ void reads8(std::integer_sequence<int, F...>, Frags &f) const {
    (read8_at<S, P, Q, FIRST, F>(f), ...);
  }

  // MFMA Q of slice kt (JB = kt % 4; slot and phase kt % 2).
  template <int JB, bool FIRST, int Q>
  __device__ __forceinline__ void mfma8(int kt, Frags &f) {
    constexpr int S = JB & 1;
    if constexpr (Q == kB8) {
      wait_vm_lgkm0<(kPfDist > 0 ? 1 : 0)>();
      barrier();
      // Slice 4 g + 1 loads the scales of group g + 1 (the next barrier
      // waits for them).
      if constexpr (JB == 1) load_pairs8((kt + 3) >> 2);
    }
    // The scales of group g go into the registers of each block once its
    // last MFMA of slice 4 g - 1 has issued, and at least two MFMAs before
    // its first of slice 4 g (the wait states between a VALU write and an
    // MFMA that reads the register, which the compiler does not place for
    // an inline-asm MFMA).
    if constexpr (JB == 3 && Q == kCv8[0]) convert8<0>((kt + 1) >> 2);
    if constexpr (JB == 3 && Q == kCv8[2]) convert8<2>((kt + 1) >> 2);
    if constexpr (JB == 0 && !FIRST && Q == kCv8[1] - f8::kM) convert8<1>(kt >> 2);
    if constexpr (JB == 0 && !FIRST && Q == kCv8[3] - f8::kM) convert8<3>(kt >> 2);
    reads8<S, S, Q, FIRST>(std::make_integer_sequence<int, 2 * f8::kNB>(), f);
    if constexpr (Q >= kB8 && (Q - kB8) % 2 == 0 && (Q - kB8) / 2 < kLoads) load8<S>(kt + 2, (Q - kB8) / 2);
    if constexpr (kPfDist > 0 && Q == f8::kM - 1) prefetch(kt + kPfDist);
    constexpr f8::IJ o = f8::order(S, Q);
    acc[o.i][o.j] = mma<FIRST, JB>(f.x[o.i], f.y[o.j], acc[o.i][o.j], sc_cur[o.i], sc_cur[kNBn + o.j]);
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int JB, bool FIRST, int... Q>
  __device__ __forceinline__ void slice8(std::integer_sequence<int, Q...>, int kt, Frags &f) {
    (mfma8<JB, FIRST, Q>(kt, f), ...);
  }
  template <int JB, bool FIRST = false>
  __device__ __forceinline__ void step8(int kt, Frags &f) {
    // (Without this the compiler computes the 16 load offsets ahead of the
    // loop and holds them in registers, which made it spill.)
    asm volatile("" : "+v"(lo8[0][0]), "+v"(lo8[0][1]), "+v"(lo8[1][0]), "+v"(lo8[1][1]));
    slice8<JB, FIRST>(std::make_integer_sequence<int, f8::kM>(), kt, f);
  }
  template <int... F>
  __device__ __forceinline__ void read8_all(std::integer_sequence<int, F...>, Frags &f) const {
    (read8<0, F>(f), ...);
  }

  __device__ __forceinline__ void run8() {
    static_assert(TM == 256 && TN == 256 && kNBn == f8::kNB && kNBm == f8::kNB && kNS == 2,
                  "fp8: 256 x 256 tiles, 16 x 16 blocks, two slots");
    static_assert(f8::schedule_ok(kB8), "fp8 fragment reads");
    static_assert(f8::convert_ok(kCv8[0], 0) && f8::convert_ok(kCv8[1], 1) && f8::convert_ok(kCv8[2], 2) &&
                      f8::convert_ok(kCv8[3], 3) && kCv8[0] > kB8 && kCv8[2] > kB8,
                  "fp8 scale conversions");
    static_assert(kB8 + 2 * (kLoads - 1) < f8::kM - 1, "fp8 loads: one every two MFMAs from the barrier");
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      kcol8[par] = chunk8_of((lane & 7) ^ swz(8 * par + (lane >> 3))) * 16;
      const uint32_t r = (uint32_t)(wave * 8 * kLA + 8 * par + (lane >> 3));
      lo8[0][par] = r * (uint32_t)a.lda + (uint32_t)kcol8[par];
      lo8[1][par] = r * (uint32_t)a.ldb + (uint32_t)kcol8[par];
    }
    // Prologue: the scales of group 0, slices 0 and 1 into their slots, the
    // L2 prefetch of slice 2; wait for all but slice 1 and the prefetch.
    load_pairs8(0);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load8<0>(0, i);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load8<1>(1, i);
    if constexpr (kPfDist > 0) prefetch(2);
    wait_vm_lgkm0<(kLoads + (kPfDist > 0 ? 1 : 0))>();
    convert8<0>(0);
    convert8<1>(0);
    convert8<2>(0);
    convert8<3>(0);
    barrier();
    Frags f;
    read8_all(std::make_integer_sequence<int, 2 * f8::kNB>(), f);
    // Slice 0 starts the accumulators; then rounds of four slices (a scale
    // group), and the one to three left run on their own.
    step8<0, true>(0, f);
    int kt = 1;
    for (; kt + 3 < nk; kt += 4) {
      step8<1>(kt, f);
      step8<2>(kt + 1, f);
      step8<3>(kt + 2, f);
      step8<0>(kt + 3, f);
    }
    if (kt < nk) step8<1>(kt, f);
    if (kt + 1 < nk) step8<2>(kt + 1, f);
    if (kt + 2 < nk) step8<3>(kt + 2, f);
    wait_vm_lgkm0<0>();
    fence_acc();
    epilogue();
  }

  // -------------------------------------------------------------------------
  // fp6: line stages.
  //
  // A K step (64 elements) is 48 bytes of a row; lane l of the 32 x 32 x 64
  // MFMA takes row l % 32 and the step's bytes 24 (l / 32) .. + 23.  Slices
  // of two steps (96 bytes) would straddle 128-byte cache lines in half the
  // rows, and a row's line fetched twice costs the texture path as much as
  // two lines: 1.5 lines per row per 96 bytes.  Here the loads stage whole
  // lines instead, stage L being row bytes 128 L .. 128 L + 127 of every
  // row of the tile, so every byte crosses from L2 once: three stages per
  // period of 8 K steps (384 bytes).  Two slots hold two stages, in rows of
  // 128 bytes with the 16-byte chunks permuted as in the other kinds' slots
  // (the 32 rows of a fragment read, 8 bytes each at one line byte, meet at
  // most two to a bank pair, the least 8-byte reads of 16-byte aligned rows
  // allow).  A slot row of 144 bytes instead (the line and an unused piece,
  // so that every read address was a per-lane base plus a constant) cost
  // one load lane in nine and measured 4% slower; rows shifted so the reads
  // met no bank conflict loaded 8 bytes of the neighbouring lines and
  // measured 15% slower: these loads, not the LDS, bound this kernel.
  //
  // Inside a period, step J (0..7) takes bytes 48 J .. 48 J + 47 of its
  // period: steps 0, 1 lie in the period's first line (ell 0), 3, 4 in the
  // second, 6, 7 in the third; step 2's upper half-wave needs pieces of
  // lines 0 and 1, step 5's lower half-wave pieces of lines 1 and 2.  The
  // fragments of step k + 1 are read during step k.  For steps 2 and 5 the
  // pieces in the older line are read first (by the half-wave that needs
  // them), the barrier then publishes the newer line and frees the older,
  // and the other half-wave reads its pieces of the newer line.  Barriers,
  // at MFMA kMB of steps 1, 4, 6 and 7:
  //   step 1: line ell 1 has landed; ell 0's slot takes line ell 2;
  //   step 4: ell 2 has landed; ell 1's slot takes ell 3;
  //   step 6: ell 2's reads are done; its slot takes ell 4;
  //   step 7: ell 3 has landed.
  // (ell 3 and ell 4 are the next period's lines 0 and 1.)  Each line's
  // loads go out over about two steps and have three steps from the barrier
  // that frees its slot to the one that publishes it.  Line L sits in slot
  // L % 2; a round of two periods (16 steps, 6 lines) makes every slot and
  // position static.
  //
  // Scales: 16-byte chunks (one per 8 steps), staged two per row per round
  // (group p: chunks 2 p, 2 p + 1); sc_ck holds chunk 2 p (read in step 6 of
  // round p - 1), sc_ckn chunk 2 p + 1 (read in step 14 of round p - 1);
  // group p + 2 is staged in step 15 of round p, after the last read of
  // group p + 1.  Pair u (steps 2 u, 2 u + 1) of a round has its 4 bytes
  // converted in step 2 u - 1 into set u % 2.
  // -------------------------------------------------------------------------
  static constexpr int kL6 = 8;   // load instructions per wave per operand and line
  static constexpr int kMB = 8;   // MFMA of a step at which its barrier goes
  static constexpr int kLS = 2;   // MFMAs between two load instructions of a line
  // Period position (16 J + MFMA) of load instruction i of the lines issued
  // in a period: ell 2 from the barrier in step 1, ell 3 from the one in
  // step 4, ell 4 from one MFMA after the one in step 6 (odd positions, so
  // they never meet ell 3's); ell 4's last six fall in the next period.
  static constexpr int kPos2 = 16 * 1 + kMB, kPos3 = 16 * 4 + kMB, kPos4 = 16 * 6 + kMB + 1;
  static_assert(kPos2 + kLS * (2 * kL6 - 1) < kPos3, "ell 2's loads end before their barrier");
  static_assert(kPos3 + kLS * (2 * kL6 - 1) < 16 * 7 + kMB, "ell 3's loads end before their barrier");
  static_assert(kPos4 + kLS * (2 * kL6 - 1) - 128 < 16 * 1 + kMB, "ell 4's loads end before their barrier");
  // Loads of ell 4 issued between the last of ell 3 and the barrier of step
  // 7 (which waits for ell 3 only).
  static constexpr int vm_at7() {
    const int last3 = kPos3 + kLS * (2 * kL6 - 1);
    int n = 0;
    for (int i = 0; i < 2 * kL6; ++i) n += kPos4 + kLS * i > last3 && kPos4 + kLS * i < 16 * 7 + kMB;
    return n;
  }

  uint32_t l6off[2];                 // this lane's piece in even / odd load instructions (panel byte offset)
  __amdgpu_buffer_rsrc_t rs6[2];     // the A and B panels of the tile
  const LDS_AS uint8_t *rowb[2][2];  // [slot][0: A, 1: B]: this lane's fragment row (block 0)
  uint32_t swz16, a24;               // the row's chunk permutation (x 16); 24 (lane / 32)
  u32x2 t6[8][3];                  // MODE 2 pieces between their read and their merge

  // Load instruction I (A: 0 .. kL6 - 1, B: kL6 ..) of line L into slot S.
  // Past the last row the range check returns zeros; past a row's end the
  // pieces hold the next row's bytes, which no fragment read takes.
  template <int S, int I>
  __device__ __forceinline__ void load6(int L) {
    constexpr int op = I < kL6 ? 0 : 1, i = I % kL6;
    LDS_AS uint8_t *dst = (op ? slots.b[S] : slots.a[S]) + (kL6 * wave + i) * 1024;
    // (Instruction i takes rows 8 i further: by soffset.)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs6[op], (LDS_AS void *)dst, 16, l6off[i & 1],
                                             (uint32_t)(128 * L + 8 * i * a.lda), 0, 0);
  }

  // Piece Q (bytes 8 Q .. 8 Q + 7, registers 2 Q and 2 Q + 1) of fragment R
  // (x blocks 0-3 from B, then y blocks 0-3 from A) from slot S, at byte X
  // of the lower half-wave's line (MODE 0: both half-waves, the upper one 24
  // bytes further; MODE 1: for the lower half-wave) or of the upper
  // half-wave's line (MODE 2: for the upper half-wave).
  template <int S, int R, int Q, int MODE, int X>
  __device__ __forceinline__ void piece6(Frags &f) {
    constexpr int op = R < kNBn ? 1 : 0;
    static_assert(X >= 0 && (R % 4) * 32 * T::kPitch + X < 65536, "constant LDS offset");
    if constexpr (R < kNBn)
      piece6_into<S, op, Q, MODE, X, R>(f.x[R]);
    else
      piece6_into<S, op, Q, MODE, X, R>(f.y[R - kNBn]);
  }
  // (MODE 1 reads for every lane at byte X: the upper half-wave takes bytes
  // of its own row that its MODE 2 read replaces.  A MODE 2 read lands in
  // t6 and is merged into the fragment with a select kMD MFMAs later
  // (merge6): a select right after the read waited for it in the middle of
  // the MFMA stream, and a branch around the read made the compiler spill.)
  template <int S, int OP, int Q, int MODE, int X, int R>
  __device__ __forceinline__ void piece6_into(Frag &fr) {
    // Line byte x of the row at its permuted chunk: x ^ swz16 (x & 15 is 0
    // or 8, so the permutation keeps the 8-byte half).
    const LDS_AS uint8_t *p = rowb[S][OP] + (((uint32_t)X + (MODE == 0 ? a24 : 0u)) ^ swz16) + (R % 4) * 32 * 128;
    const u32x2 v = *(const LDS_AS u32x2 *)p;
    if constexpr (MODE < 2) {
      fr[2 * Q] = (int)v[0];
      fr[2 * Q + 1] = (int)v[1];
    } else {
      t6[R][Q] = v;
    }
  }
  template <int R, int Q>
  __device__ __forceinline__ void merge6(Frags &f) {
    Frag &fr = R < kNBn ? f.x[R % kNBn] : f.y[R % kNBm];
    const bool up = lane >= 32;
    fr[2 * Q] = up ? (int)t6[R][Q][0] : fr[2 * Q];
    fr[2 * Q + 1] = up ? (int)t6[R][Q][1] : fr[2 * Q + 1];
  }

  // The reads of step J's successor, in the order y0, x0, y1, y2, y3, x1,
  // x2, x3 (the order the MFMAs first take them).  Read n of the N in a
  // list goes out at MFMA M0 + n (M1 - M0) / N.
  static constexpr int kFragOrder[8] = {4, 0, 5, 6, 7, 1, 2, 3};
  struct Rd {
    int r, q, mode, ell, x;
  };
  // Read n of the list of step J (period position): part 0 before the
  // barrier, part 1 after it (steps 1 and 4), or the whole list.
  static constexpr int n_reads(int J, int part) {
    return J == 1 ? (part == 0 ? 24 : 16) : J == 4 ? (part == 0 ? 16 : 24) : 24;
  }
  static constexpr Rd read_of(int J, int part, int n) {
    const int Jt = J + 1;  // the step read (8: the next period's step 0)
    if (J == 1 && part == 1) {
      const int f = kFragOrder[n / 2], q = 1 + n % 2;
      return Rd{f, q, 2, 1, 48 * Jt + 24 + 8 * q - 128};
    }
    if (J == 4 && part == 0) {
      const int f = kFragOrder[n / 2], q = n % 2;
      return Rd{f, q, 1, 1, 48 * Jt + 8 * q - 128};
    }
    if (J == 4 && part == 1) {
      const int f = kFragOrder[n / 3], q = n % 3;
      return q < 2 ? Rd{f, q, 2, 2, 48 * Jt + 24 + 8 * q - 256} : Rd{f, 2, 0, 2, 48 * Jt + 16 - 256};
    }
    const int f = kFragOrder[n / 3], q = n % 3;
    const int ell = Jt * 48 / 128;  // the line of the step's first byte
    const int mode = J == 1 && q > 0 ? 1 : 0;
    return Rd{f, q, mode, ell, 48 * Jt + 8 * q - 128 * ell};
  }
  // MFMA range of a list.
  static constexpr int rd_m0(int J, int part) { return (J == 1 || J == 4) ? (part == 0 ? 0 : kMB) : J == 7 ? kMB : 0; }
  static constexpr int rd_m1(int J, int part) {
    return (J == 1 || J == 4) ? (part == 0 ? kMB : 16) : J == 6 ? kMB : 16;
  }
  static constexpr int rd_m(int J, int part, int n) {
    return rd_m0(J, part) + n * (rd_m1(J, part) - rd_m0(J, part)) / n_reads(J, part);
  }

  // Merge of MODE 2 read n of step J (1 or 4): kMD MFMAs after the read,
  // as a position counted from the start of step J (16 and on: the next
  // step, which first takes fragment x i at its MFMA 4 i, y j at MFMA j).
  static constexpr int kMD = 3;
  static constexpr int merge_pos(int J, int n) {
    const Rd d = read_of(J, 1, n);
    const int want = rd_m(J, 1, n) + kMD;
    const int use = 16 + (d.r < 4 ? 4 * d.r : 0);
    return want < use ? want : use;
  }
  template <int J, int POS, int N>
  __device__ __forceinline__ void merge_if(Frags &f) {
    if constexpr (read_of(J, 1, N).mode == 2 && merge_pos(J, N) == POS) merge6<read_of(J, 1, N).r, read_of(J, 1, N).q>(f);
  }
  template <int J, int POS, int... N>
  __device__ __forceinline__ void merges_at(std::integer_sequence<int, N...>, Frags &f) {
    (merge_if<J, POS, N>(f), ...);
  }

  template <int H, int J, int M, int PART, int N>
  __device__ __forceinline__ void read_if(Frags &f) {
    if constexpr (rd_m(J, PART, N) == M) {
      constexpr Rd d = read_of(J, PART, N);
      piece6<(H + d.ell) % 2, d.r, d.q, d.mode, d.x>(f);
    }
  }
  template <int H, int J, int M, int PART, int... N>
  __device__ __forceinline__ void reads_at(std::integer_sequence<int, N...>, Frags &f) {
    (read_if<H, J, M, PART, N>(f), ...);
  }

  // Loads at period position P of half H of round p.
  template <int H, int P, int I>
  __device__ __forceinline__ void load_if(int p) {
    if constexpr (P >= kPos2 && (P - kPos2) % kLS == 0 && (P - kPos2) / kLS == I) load6<H % 2, I>(6 * p + 3 * H + 2);
    if constexpr (P >= kPos3 && (P - kPos3) % kLS == 0 && (P - kPos3) / kLS == I) load6<(H + 1) % 2, I>(6 * p + 3 * H + 3);
    if constexpr (P >= kPos4 && (P - kPos4) % kLS == 0 && (P - kPos4) / kLS == I) load6<H % 2, I>(6 * p + 3 * H + 4);
    // The end of the previous period's ell 4 (this period's ell 1).
    if constexpr (P + 128 >= kPos4 && (P + 128 - kPos4) % kLS == 0 && (P + 128 - kPos4) / kLS == I)
      load6<(H + 1) % 2, I>(6 * p + 3 * H + 1);
  }
  template <int H, int P, int... I>
  __device__ __forceinline__ void loads_at(std::integer_sequence<int, I...>, int p) {
    (load_if<H, P, I>(p), ...);
  }

  // The 4 scale bytes per row of step pair U (0..7) of a round: dwords U and
  // U + 1 of chunk 2 p (sc_ck) and chunk 2 p + 1 (sc_ckn), shifted by the
  // row's byte offset; pair 7 shifts in the first dword of chunk 2 p + 2,
  // which replaced chunk 2 p in sc_ck by then.  The MFMA of step 2 u + s in
  // half-wave w uses group 2 s + w, so lanes 0-31 take groups 0, 2 and
  // lanes 32-63 groups 1, 3, in byte s.  t: the pair's index over all of K.
  template <int U>
  __device__ __forceinline__ void convert6(int t) {
    const uint32_t keep = keep_mask(a.kb - 4 * t);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w0 = U < 4 ? sc_ck[j][U] : sc_ckn[j][U - 4];
      const uint32_t w1 = U == 3 ? sc_ckn[j][0] : U == 7 ? sc_ck[j][0] : U < 4 ? sc_ck[j][U + 1] : sc_ckn[j][U - 3];
      const uint32_t d = __builtin_amdgcn_alignbyte(w1, w0, sc_sh[j]) & keep;
      const uint32_t lo = __builtin_amdgcn_perm(0u, d, 0x0c0c0200u);  // groups 0, 2
      const uint32_t hi = __builtin_amdgcn_perm(0u, d, 0x0c0c0301u);  // groups 1, 3
      const auto sw = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
      sc_set[U & 1][2 * j] = (int)sw[0];
      sc_set[U & 1][2 * j + 1] = (int)sw[1];
    }
  }

  // MFMA M of step JJ (0..15) of round p.
  template <int JJ, int M>
  __device__ __forceinline__ void mstep6(int p, Frags &f0, Frags &f1) {
    constexpr int H = JJ / 8, J = JJ % 8, P = 16 * J + M;
    if constexpr (M == kMB && (J == 1 || J == 4 || J == 6 || J == 7)) {
      if constexpr (J == 1 || J == 4)
        wait_vm_lgkm0<0>();
      else if constexpr (J == 6)
        wait_vm_lgkm0<63>();
      else
        wait_vm_lgkm0<vm_at7()>();
      barrier();
      if constexpr (JJ == 6) fetch_chunk<0>(sc_ck);    // chunk 2 p + 2
      if constexpr (JJ == 14) fetch_chunk<1>(sc_ckn);  // chunk 2 p + 3
      if constexpr (JJ == 15) stage_group(p + 2);
    }
    if constexpr (M == 2 && (JJ & 1)) convert6<((JJ + 1) / 2) % 8>(8 * p + (JJ + 1) / 2);
    Frags &fn = (JJ % 2 == 0) ? f1 : f0;  // the next step's fragments
    Frags &fc = (JJ % 2 == 0) ? f0 : f1;  // this step's
    if constexpr (J == 1 || J == 4) {
      if constexpr (M < kMB)
        reads_at<H, J, M, 0>(std::make_integer_sequence<int, n_reads(J, 0)>(), fn);
      else
        reads_at<H, J, M, 1>(std::make_integer_sequence<int, n_reads(J, 1)>(), fn);
      merges_at<J, M>(std::make_integer_sequence<int, n_reads(J, 1)>(), fn);
    } else {
      reads_at<H, J, M, 0>(std::make_integer_sequence<int, n_reads(J, 0)>(), fn);
    }
    // Merges of the previous step's MODE 2 reads that fall in this step.
    if constexpr (J == 2 || J == 5) merges_at<J - 1, 16 + M>(std::make_integer_sequence<int, n_reads(J - 1, 1)>(), fc);
    loads_at<H, P>(std::make_integer_sequence<int, 2 * kL6>(), p);
    // x blocks in order, y blocks snaking (as in the other kinds).
    constexpr int I = M / 4, J0 = M % 4, Y = (I & 1) ? 3 - J0 : J0;
    const Frags &f = (JJ % 2 == 0) ? f0 : f1;
    acc[I][Y] = mma<false, JJ & 1>(f.x[I], f.y[Y], acc[I][Y], sc_set[(JJ / 2) & 1][I], sc_set[(JJ / 2) & 1][4 + Y]);
    __builtin_amdgcn_sched_barrier(0);
  }
  template <int JJ, int... M>
  __device__ __forceinline__ void kstep6(std::integer_sequence<int, M...>, int p, Frags &f0, Frags &f1) {
    // (The read addresses are per-lane constants; without this the compiler
    // computes them all ahead of the loop and holds them in registers, which
    // made it spill.)
    asm volatile("" : "+v"(swz16), "+v"(a24));
    (mstep6<JJ, M>(p, f0, f1), ...);
  }
  template <int... JJ>
  __device__ __forceinline__ void round6(std::integer_sequence<int, JJ...>, int p, Frags &f0, Frags &f1) {
    (kstep6<JJ>(std::make_integer_sequence<int, 16>(), p, f0, f1), ...);
  }
  // The steps k0 + JJ < nks of a last, partial round.
  template <int... JJ>
  __device__ __forceinline__ void tail6(std::integer_sequence<int, JJ...>, int p, int left, Frags &f0, Frags &f1) {
    ((JJ < left ? kstep6<JJ>(std::make_integer_sequence<int, 16>(), p, f0, f1) : void()), ...);
  }

  __device__ __forceinline__ void run6() {
    static_assert(TM == 256 && TN == 256 && kNBn == 4 && kNBm == 4, "fp6: 256 x 256 tiles, 32 x 32 blocks");
    // Panels: rows a.lda (= a.ldb) bytes apart; the resource ends with the
    // last valid row.
    const int ld = a.lda;
    rs6[0] = make_rsrc(a.A + (size_t)m0 * ld, (uint32_t)min(a.M - m0, TM) * (uint32_t)ld);
    rs6[1] = make_rsrc(a.B + (size_t)n0 * ld, (uint32_t)min(a.N - n0, TN) * (uint32_t)ld);
    // Slot rows of 128 bytes with the 16-byte chunks permuted as in the
    // other kinds' slots: lane l of load instruction i of wave w writes row
    // 64 w + 8 i + l / 8, physical chunk l % 8, holding logical chunk
    // (l % 8) ^ swz(row); swz depends on i only through its parity.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 64 * wave + 8 * i + (lane >> 3), c = (lane & 7) ^ swz(r);
      l6off[i] = (uint32_t)(64 * wave + (lane >> 3)) * (uint32_t)ld + 16u * (uint32_t)c;
    }
    swz16 = (uint32_t)swz(lane & 31) << 4;  // fragment rows start at multiples of 32
    a24 = 24u * (uint32_t)(lane >> 5);
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      rowb[sl][0] = slots.a[sl] + (wave_m * kWM + (lane & 31)) * 128;
      rowb[sl][1] = slots.b[sl] + (wave_n * kWN + (lane & 31)) * 128;
    }
    const int nks = a.ksteps;  // K steps of 64 elements

    // Prologue: group 0 of the scales, line 0 into slot 0, and the loads of
    // line 1 that the K loop's previous period would have issued (the rest
    // go out in steps 0 and 1).
    stage_group(0);
    load_line6_first<0>(0, std::make_integer_sequence<int, 2 * kL6>());
    constexpr int kEarly1 = (128 - kPos4 + kLS - 1) / kLS;  // ell 4 loads issued in its own period
    load_line6_first<1>(1, std::make_integer_sequence<int, kEarly1>());
    wait_vm_lgkm0<kEarly1>();
    barrier();
    fetch_chunk<0>(sc_ck);
    fetch_chunk<1>(sc_ckn);
    convert6<0>(0);
    Frags f0, f1;
    read_first6(std::make_integer_sequence<int, 24>(), f0);
    // Every wave has read group 0 before group 1 replaces it.
    wait_vm_lgkm0<kEarly1>();
    barrier();
    stage_group(1);

    int k = 0, p = 0;
    for (; k + 16 <= nks; k += 16, ++p) round6(std::make_integer_sequence<int, 16>(), p, f0, f1);
    if (k < nks) tail6(std::make_integer_sequence<int, 16>(), p, nks - k, f0, f1);
    wait_vm_lgkm0<0>();
    fence_acc();
    epilogue();
  }
  template <int S, int... I>
  __device__ __forceinline__ void load_line6_first(int L, std::integer_sequence<int, I...>) {
    (load6<S, I>(L), ...);
  }
  // Step 0's fragments (line 0, slot 0).
  template <int... N>
  __device__ __forceinline__ void read_first6(std::integer_sequence<int, N...>, Frags &f) {
    (piece6<0, kFragOrder[N / 3], N % 3, 0, 8 * (N % 3)>(f), ...);
  }

  // K split: the tile's fp32 sums into plane `split` of the workspace (M x N,
  // rows N apart).  16 x 16 blocks: lane l holds row l % 16, columns
  // 4 (l / 16) .. + 3, one 16-byte store each (N % 8 == 0, so a group of four
  // columns is all in or all out of range).
  __device__ __forceinline__ void epilogue_partial(int split) {
    static_assert(kBlk == 16, "16 x 16 blocks");
    float *plane = a.ws + (size_t)split * (size_t)a.M * (size_t)a.N;
    const int q = lane >> 4;
#pragma unroll
    for (int j = 0; j < kNBm; ++j) {
      const int m = m0 + wave_m * kWM + j * kBlk + (lane & 15);
#pragma unroll
      for (int i = 0; i < kNBn; ++i) {
        const int n = n0 + wave_n * kWN + i * kBlk + 4 * q;
        // Written through like C (the reduction reads them from another
        // kernel): 512 x 512 x 4096 split 4 ways, 10.40 -> 9.98 us per call.
        if (m < a.M && n < a.N) store_c((uint8_t *)(plane + (size_t)m * a.N + n), __builtin_bit_cast(u32x4, acc[i][j]));
      }
    }
  }

  // acc[i][j] covers B rows (C columns) n0 + kWN wave_n + kBlk i and A rows
  // (C rows) m0 + kWM wave_m + kBlk j.  32 x 32 blocks: lane l, register r
  // holds C row l % 32 of the block, column 8 (r / 4) + 4 (l / 32) + r % 4.
  // 16 x 16 blocks: lane l, register r holds row l % 16, column
  // 4 (l / 16) + r.
  //
  // Four fp32 -> one 8-byte group of C values (bf16, or fp16 for fp16 inputs).
  __device__ __forceinline__ u32x2 pack4(const Acc &c, int r0) const {
    const f32x2 lo = {c[r0], c[r0 + 1]};
    const f32x2 up = {c[r0 + 2], c[r0 + 3]};
    u32x2 pk;
    if constexpr (T::kDt == kF16) {
      pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, f16x2));
      pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(up, f16x2));
    } else {
      pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
      pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(up, bf16x2));
    }
    return pk;
  }

  __device__ __forceinline__ void epilogue() {
    const int row_l = lane % kBlk;
    if constexpr (kBlk == 32) {
      // 32 x 32 blocks: lanes l and l + 32 hold the same row, columns
      // 8 g .. 8 g + 3 and 8 g + 4 .. 8 g + 7 of group g.  One swap of the
      // wave halves per pair of groups (2 p, 2 p + 1) gives lane l columns
      // 16 p .. 16 p + 7 and lane l + 32 columns 16 p + 8 .. 16 p + 15 (X
      // for p = 0, Y for p = 1).  A swap of odd and even 16-lane rows of X
      // and Y then leaves the 16-lane rows of the wave with (X_0 Y_0 X_2 Y_2)
      // -- the 32 columns of block rows 0-15 -- and (X_1 Y_1 X_3 Y_3), those
      // of rows 16-31: each store instruction writes 64 contiguous bytes of
      // each of 16 rows, four lanes per row.  (Every lane swaps; only the
      // stores are masked.)
      const int r16 = lane & 15;
      const int col = 16 * ((lane >> 4) & 1) + 8 * (lane >> 5);
#pragma unroll
      for (int j = 0; j < kNBm; ++j) {
        const int m = m0 + wave_m * kWM + j * kBlk + r16;
        uint8_t *crow0 = a.C + (size_t)m * a.ldc * 2;
        uint8_t *crow1 = a.C + (size_t)(m + 16) * a.ldc * 2;
#pragma unroll
        for (int i = 0; i < kNBn; ++i) {
          u32x4 xy[2];
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const u32x2 p0 = pack4(acc[i][j], 8 * pr), p1 = pack4(acc[i][j], 8 * pr + 4);
            const auto s0 = __builtin_amdgcn_permlane32_swap(p0[0], p1[0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(p0[1], p1[1], false, false);
            xy[pr] = u32x4{s0[0], s1[0], s0[1], s1[1]};
          }
          u32x4 lo, hi;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const auto r = __builtin_amdgcn_permlane16_swap(xy[0][d], xy[1][d], false, false);
            lo[d] = r[0];
            hi[d] = r[1];
          }
          const int n = n0 + wave_n * kWN + i * kBlk + col;
          if (n < a.N) {
            if (m < a.M) store_c(crow0 + (size_t)n * 2, lo);
            if (m + 16 < a.M) store_c(crow1 + (size_t)n * 2, hi);
          }
        }
      }
    } else {
      // 16 x 16 blocks: lane l holds row l % 16, columns 4 (l / 16) .. + 3.
      // Per pair of blocks (i, i + 1) the 16-lane rows q of the wave hold
      // X_q = columns 4 q .. of block i and Y_q of block i + 1.  A swap of
      // the wave halves, then of odd and even 16-lane rows, leaves row q
      // with columns 8 q .. 8 q + 7 of the 32 (X_0 X_1 | X_2 X_3 | Y_0 Y_1 |
      // Y_2 Y_3), so each lane stores 16 bytes and an instruction writes 64
      // contiguous bytes of each of 16 rows.  (The lanes that trade hold the
      // same row, so a row's lanes are all in or all out of range.)
      static_assert(kNBn % 2 == 0, "blocks pair up along N");
      const int q = lane >> 4;
#pragma unroll
      for (int j = 0; j < kNBm; ++j) {
        const int m = m0 + wave_m * kWM + j * kBlk + row_l;
        uint8_t *crow = a.C + (size_t)m * a.ldc * 2;
#pragma unroll
        for (int i = 0; i < kNBn; i += 2) {
          const u32x2 x = pack4(acc[i][j], 0), y = pack4(acc[i + 1][j], 0);
          uint32_t xo[2], yo[2];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            const auto h = __builtin_amdgcn_permlane32_swap(x[d], y[d], false, false);
            const auto r = __builtin_amdgcn_permlane16_swap(h[0], h[1], false, false);
            xo[d] = r[0];
            yo[d] = r[1];
          }
          const u32x4 out = {xo[0], xo[1], yo[0], yo[1]};
          const int n = n0 + wave_n * kWN + i * kBlk + 8 * q;
          if (m < a.M && n < a.N) store_c(crow + (size_t)n * 2, out);
        }
      }
    }
  }

};

// One workgroup per CU: either shape's ring takes 128 KiB of the 160 KiB
// LDS, and a 256-row tile's accumulators fill a SIMD's registers.
template <class T, int TM, int TN, bool SPLIT = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(const Args a) {
#if defined(__HIP_DEVICE_COMPILE__)  // the body is device code only; the host pass needs the symbol
  // A separate array per slot (not one indexed array) so the compiler can
  // tell the slot being loaded from the slot being read and does not insert
  // a vmcnt wait in front of every LDS read.
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[TM * T::kPitch];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[TM * T::kPitch];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[TN * T::kPitch];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[TN * T::kPitch];
  Slots slots;
  slots.a[0] = (LDS_AS uint8_t *)sA0;
  slots.a[1] = (LDS_AS uint8_t *)sA1;
  slots.b[0] = (LDS_AS uint8_t *)sB0;
  slots.b[1] = (LDS_AS uint8_t *)sB1;
  if constexpr (kSlots<T, TM, TN> == 4) {
    __shared__ __attribute__((aligned(1024))) uint8_t sA2[TM * kRowBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sA3[TM * kRowBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sB2[TN * kRowBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sB3[TN * kRowBytes];
    slots.a[2] = (LDS_AS uint8_t *)sA2;
    slots.a[3] = (LDS_AS uint8_t *)sA3;
    slots.b[2] = (LDS_AS uint8_t *)sB2;
    slots.b[3] = (LDS_AS uint8_t *)sB3;
  }
  slots.junk = nullptr;
  if constexpr (Kernel<T, TM, TN, SPLIT>::kPfDist > 0) {
    __shared__ __attribute__((aligned(256))) uint8_t junk[4 * 256];
    slots.junk = (LDS_AS uint8_t *)junk;
  }
  slots.stage = nullptr;
  if constexpr (Kernel<T, TM, TN, SPLIT>::kStaged) {
    __shared__ __attribute__((aligned(1024))) uint8_t st[Kernel<T, TM, TN, SPLIT>::kStageBytes];
    slots.stage = (LDS_AS uint8_t *)st;
  }
  Kernel<T, TM, TN, SPLIT> k(a, slots);
  k.run();
#endif
}

template <class T, int TM, int TN, bool SPLIT = false>
hipError_t launch_shape(const Problem &p, Args a) {
  a.tiles_m = (int)((p.M + TM - 1) / TM);
  a.tiles_n = (int)((p.N + TN - 1) / TN);
  // A dispatch holds fewer than 2^32 work-items per dimension.
  const int64_t tiles = (int64_t)a.tiles_m * a.tiles_n;
  const int64_t wgs = tiles * (SPLIT ? a.splits : 1);
  if (wgs > (int64_t)(UINT32_MAX / kThreads)) return hipErrorInvalidConfiguration;
  // hipLaunchKernel returns this launch's own status (hipGetLastError could
  // report an earlier, unrelated failure of the calling thread).
  void *args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void *>(&gemm_kernel<T, TM, TN, SPLIT>), dim3((unsigned)wgs),
                         dim3(kThreads), args, 0, p.stream);
}

// K split, second pass: C[m][n] = the sum over s = 0, 1, ... splits - 1, in
// that order, of plane s [m][n], rounded to nearest-even bf16 (DT = kBf16)
// or fp16.  One thread per 8 consecutive columns of a row (N % 8 == 0):
// two 16-byte loads per plane, one 16-byte store.
struct ReduceArgs {
  const float *ws;
  uint8_t *C;
  int splits, M, N, ldc;
};

template <int DT>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const ReduceArgs r) {
  const int per_row = r.N >> 3;
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= (int64_t)r.M * per_row) return;
  const int m = (int)(g / per_row);
  const int n = (int)(g - (int64_t)m * per_row) * 8;
  const size_t plane = (size_t)r.M * (size_t)r.N;
  const float *p = r.ws + (size_t)m * r.N + n;
  f32x4 lo = *(const f32x4 *)p, hi = *(const f32x4 *)(p + 4);
  for (int s = 1; s < r.splits; ++s) {
    lo += *(const f32x4 *)(p + s * plane);
    hi += *(const f32x4 *)(p + s * plane + 4);
  }
  u32x4 out;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x4 &v = h ? hi : lo;
    const f32x2 x = {v[0], v[1]}, y = {v[2], v[3]};
    if constexpr (DT == kF16) {
      out[2 * h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
      out[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, f16x2));
    } else {
      out[2 * h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
      out[2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(y, bf16x2));
    }
  }
  store_c(r.C + ((size_t)m * r.ldc + n) * 2, out);
}

template <int DT>
hipError_t launch_reduce(const Problem &p, const Args &a) {
  ReduceArgs r{a.ws, a.C, a.splits, a.M, a.N, a.ldc};
  const int64_t blocks = ((int64_t)p.M * (p.N / 8) + 255) / 256;
  if (blocks > INT32_MAX) return hipErrorInvalidConfiguration;
  void *args[] = {&r};
  return hipLaunchKernel(reinterpret_cast<const void *>(&splitk_reduce_kernel<DT>), dim3((unsigned)blocks),
                         dim3(256), args, 0, p.stream);
}

// The K-split pair of one layout: partial sums, then the reduction.
template <int DT, bool AK, bool BK>
hipError_t launch_split_layout(const Problem &p, const Args &a, int tm, int tn) {
  using T = Traits<DT, AK, BK>;
  hipError_t e = hipErrorInvalidValue;
  if (tm == 128 && tn == 128) e = launch_shape<T, 128, 128, true>(p, a);
  else if (tm == 64 && tn == 64) e = launch_shape<T, 64, 64, true>(p, a);
  if (e != hipSuccess) return e;
  return launch_reduce<DT>(p, a);
}

template <int DT>
hipError_t launch_split_dt(const Problem &p, const Args &a, int tm, int tn) {
  const bool ak = !p.trans_a, bk = p.trans_b;
  if (ak && bk) return launch_split_layout<DT, true, true>(p, a, tm, tn);
  if (ak) return launch_split_layout<DT, true, false>(p, a, tm, tn);
  if (bk) return launch_split_layout<DT, false, true>(p, a, tm, tn);
  return launch_split_layout<DT, false, false>(p, a, tm, tn);
}

// The 16-bit kernels of one operand layout, by tile shape (256 x 192 only
// where B is K-contiguous: a K-major B slot must be 256 or 128 wide).
template <int DT, bool AK, bool BK>
hipError_t launch_layout(const Problem &p, const Args &a, int tm, int tn) {
  using T = Traits<DT, AK, BK>;
  if (tm == 256 && tn == 256) return launch_shape<T, 256, 256>(p, a);
  if constexpr (BK)
    if (tm == 256 && tn == 192) return launch_shape<T, 256, 192>(p, a);
  if (tm == 128 && tn == 128) return launch_shape<T, 128, 128>(p, a);
  if (tm == 64 && tn == 64) return launch_shape<T, 64, 64>(p, a);
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const Problem &p, const Args &a, int tm, int tn) {
  const bool ak = !p.trans_a, bk = p.trans_b;
  if (ak && bk) return launch_layout<DT, true, true>(p, a, tm, tn);
  if (ak) return launch_layout<DT, true, false>(p, a, tm, tn);
  if (bk) return launch_layout<DT, false, true>(p, a, tm, tn);
  return launch_layout<DT, false, false>(p, a, tm, tn);
}

// Tile shapes per kind, largest first, each with a rate relative to
// 256 x 256 per unit of tile area in a wave of workgroups (one workgroup
// per CU).  The rates are fitted to sustained measurements on MI355X
// (bf16 NT unless noted, us):
//                        256x256  256x192  128x128  64x64
//   4096 x 4096 x 8192     193      --       251      --   (rate 0.77 here)
//   3072 x 3072 x 3072      65      --        74      --
//   4000 x 3000 x 5000     118     117       156      --
//   2048 x 2048 x 4096      78      63        35      --
//   2048 x 1024 x 4096      77      --        27      --
//   512 x 512 x 4096        --      --        25.8    12.2
//   fp16 NN 2048 x 1024^2   --      --        12.0    11.1
//   fp16 NN 1024^3          31      --        11.8     6.2
//   256^3                   --      --         5.9     3.7
// 0.70 for 128 x 128 sits between the first two rows: a partly filled last
// wave runs at a higher clock under the power cap than whole ones.  0.35
// for 64 x 64 fits the rows below it, where a slice's loads and barrier,
// not its 8 MFMAs per wave, set the pace.
struct Shape {
  int tm, tn;
  double rel;
};
constexpr Shape kShapesBK[] = {{256, 256, 1.0}, {256, 192, 0.92}, {128, 128, 0.70}, {64, 64, 0.35}};  // B K-contiguous
constexpr Shape kShapesBN[] = {{256, 256, 1.0}, {128, 128, 0.70}, {64, 64, 0.35}};                     // B N-contiguous

// The shape with the least estimated time: whole waves of tiles over the
// CUs, each wave costing its tile area over the shape's relative rate.
template <size_t NS>
Shape pick_shape(const Shape (&shapes)[NS], int64_t M, int64_t N, int cus) {
  Shape best = shapes[0];
  double best_t = 0;
  for (size_t i = 0; i < NS; ++i) {
    const Shape &s = shapes[i];
    const int64_t tiles = ((M + s.tm - 1) / s.tm) * ((N + s.tn - 1) / s.tn);
    const int64_t slots = cus;  // one workgroup per CU
    const int64_t waves = (tiles + slots - 1) / slots;
    const double t = (double)waves * s.tm * s.tn / s.rel;
    if (i == 0 || t < best_t) {
      best = s;
      best_t = t;
    }
  }
  return best;
}

// Whether to split K, and into how many pieces of which tile shape.  Only
// the 128 x 128 and 64 x 64 tiles have split kernels; with another tile
// forced there is no split (the front end refuses explicit splits then).
// Explicit splits are taken as given (the caller's workspace holds them).
// Automatic ones (p.splits == 0) only where the plain grid leaves at least
// half the CUs idle and K has at least 48 slices (3072 elements): then
// 64 x 64 tiles and at most 4 splits, no more than fill the CUs once, at
// least 16 slices each, and no more than the workspace holds.  Measured
// under graph replay (bf16 NT, us per call, plain -> split): 512 x 512 x 4096
// 10.95 -> 9.68 (3 splits 9.3, 6 splits 12.7), 512 x 512 x 8192 22.5 -> 13.1,
// 256 x 256 x 4096 10.8 -> 7.7; but 768 x 512 x 2048 (32 slices) 6.7 -> 8.4
// with 2 splits: the partial sums' round trip and the second kernel cost
// about 2-3 us, which short K ranges do not repay.  Returns false for no
// split (tm, tn untouched).
bool choose_split(const Problem &p, int ksteps, int &tm, int &tn, int &splits) {
  const bool forced = p.tile_m != 0;
  if (forced && !((p.tile_m == 128 && p.tile_n == 128) || (p.tile_m == 64 && p.tile_n == 64))) return false;
  const uint64_t plane = (uint64_t)p.M * (uint64_t)p.N * 4u;
  const int64_t fit = plane > 0 ? (int64_t)(p.ws_bytes / plane) : 0;
  if (p.splits >= 2) {
    splits = (int)std::min<int64_t>({(int64_t)p.splits, (int64_t)kMaxSplits, (int64_t)ksteps, fit});
    if (splits < 2) return false;
    tm = forced ? p.tile_m : 64;
    tn = forced ? p.tile_n : 64;
    return true;
  }
  const Shape plain = p.trans_b ? pick_shape(kShapesBK, p.M, p.N, p.cus) : pick_shape(kShapesBN, p.M, p.N, p.cus);
  const int64_t plain_tiles = ((p.M + plain.tm - 1) / plain.tm) * ((p.N + plain.tn - 1) / plain.tn);
  if (plain_tiles * 2 > p.cus || ksteps < 48) return false;
  const int stm = forced ? p.tile_m : 64, stn = forced ? p.tile_n : 64;
  const int64_t tiles = ((p.M + stm - 1) / stm) * ((p.N + stn - 1) / stn);
  const int64_t want = std::min<int64_t>({(int64_t)p.cus / tiles, (int64_t)kAutoMaxSplits, (int64_t)ksteps / 16, fit});
  if (want < 2) return false;
  splits = (int)want;
  tm = stm;
  tn = stn;
  return true;
}

}  // namespace

hipError_t launch(const Problem &p) {
  Args a;
  a.A = static_cast<const uint8_t *>(p.A);
  a.B = static_cast<const uint8_t *>(p.B);
  a.SA = static_cast<const uint8_t *>(p.scale_A);
  a.SB = static_cast<const uint8_t *>(p.scale_B);
  a.C = static_cast<uint8_t *>(p.C);
  a.M = (int)p.M;
  a.N = (int)p.N;
  a.K = (int)p.K;
  a.lda = (int)p.lda;
  a.ldb = (int)p.ldb;
  a.ldc = (int)p.ldc;
  a.ws = nullptr;
  a.splits = 1;
  a.kq = 0;
  const int slice = p.dt == Dt::kMxfp8 ? 128 : 64;
  a.ksteps = (int)((p.K + slice - 1) / slice);
  a.kb = (int)((p.K + 127) / 128);
  if (p.dt == Dt::kMxfp4) {
    // Rows of bytes (two elements each), 128-byte slices, a scale per 32.
    a.K = (int)(p.K / 2);
    a.ksteps = (a.K + kRowBytes - 1) / kRowBytes;
    a.kb = (int)((p.K + 31) / 32);
  }
  const bool fp6 = p.dt == Dt::kMxfp6E2M3 || p.dt == Dt::kMxfp6E3M2;
  if (fp6) {
    // Rows of bytes (four elements in three), a scale per 32; the K loop
    // counts 64-element steps (48 bytes; K % 64 == 0).
    a.K = (int)(p.K / 4 * 3);
    a.ksteps = (int)(p.K / 64);
    a.kb = (int)((p.K + 31) / 32);
  }
  const bool scaled = p.dt == Dt::kMxfp8 || p.dt == Dt::kMxfp4 || fp6;
  // MXFP8 with no ragged slice (128 elements each) takes the kernel whose
  // loads check no columns (2% fewer cycles).
  const bool whole = p.K > 0 && p.K % 128 == 0;
  int tm = p.tile_m, tn = p.tile_n;
  if ((p.dt == Dt::kBf16 || p.dt == Dt::kF16) && p.splits != 1 && p.ws != nullptr) {
    int splits = 0;
    if (choose_split(p, a.ksteps, tm, tn, splits)) {
      // Whole slices per split, and no split left empty.
      a.kq = (a.ksteps + splits - 1) / splits;
      a.splits = (a.ksteps + a.kq - 1) / a.kq;
      a.ws = static_cast<float *>(p.ws);
      return p.dt == Dt::kBf16 ? launch_split_dt<kBf16>(p, a, tm, tn) : launch_split_dt<kF16>(p, a, tm, tn);
    }
  }
  if (tm == 0) {
    const Shape s = scaled             ? Shape{256, 256, 1.0}
                    : p.trans_b        ? pick_shape(kShapesBK, p.M, p.N, p.cus)
                                       : pick_shape(kShapesBN, p.M, p.N, p.cus);
    tm = s.tm;
    tn = s.tn;
  }
  switch (p.dt) {
    case Dt::kBf16:
      return launch_dt<kBf16>(p, a, tm, tn);
    case Dt::kF16:
      return launch_dt<kF16>(p, a, tm, tn);
    case Dt::kMxfp8:
      if (tm == 256 && tn == 256 && !p.trans_a && p.trans_b)
        return whole ? launch_shape<Traits<kFp8, true, true, true>, 256, 256>(p, a)
                     : launch_shape<Traits<kFp8, true, true>, 256, 256>(p, a);
      break;
    case Dt::kMxfp4:
      if (tm == 256 && tn == 256 && !p.trans_a && p.trans_b)
        return p.K > 0 && p.K % 256 == 0 && (((uintptr_t)a.SA | (uintptr_t)a.SB) & 3) == 0
                   ? launch_shape<Traits<kFp4, true, true, true>, 256, 256>(p, a)
                   : launch_shape<Traits<kFp4, true, true>, 256, 256>(p, a);
      break;
    case Dt::kMxfp6E2M3:
      if (tm == 256 && tn == 256 && !p.trans_a && p.trans_b)
        return launch_shape<Traits<kFp6E2M3, true, true>, 256, 256>(p, a);
      break;
    case Dt::kMxfp6E3M2:
      if (tm == 256 && tn == 256 && !p.trans_a && p.trans_b)
        return launch_shape<Traits<kFp6E3M2, true, true>, 256, 256>(p, a);
      break;
  }
  return hipErrorInvalidValue;
}

bool shape_supported(const Problem &p, int tile_m, int tile_n) {
  if (p.dt != Dt::kBf16 && p.dt != Dt::kF16) return tile_m == 256 && tile_n == 256;
  if (p.splits >= 2) return (tile_m == 128 && tile_n == 128) || (tile_m == 64 && tile_n == 64);
  return (tile_m == 256 && tile_n == 256) || (tile_m == 128 && tile_n == 128) || (tile_m == 64 && tile_n == 64) ||
         (tile_m == 256 && tile_n == 192 && p.trans_b);
}

}  // namespace tgemm
