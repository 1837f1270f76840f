// Tiled dense GEMM kernels for gfx950 (MI355X, CDNA4).
//
// One workgroup of 256 threads (4 wave64s in a 2 x 2 grid) computes a
// 256 x 256 tile of C; each wave owns a 128 x 128 sub-tile held as 4 x 4
// blocks of 32 x 32 fp32 accumulators (256 per lane, in AGPRs).  The K loop
// walks 64-byte slices of the A and B panels (32 bf16/fp16 or 64 fp8
// elements per row) through a ring of four LDS slots, loading three slices
// ahead of the one being multiplied.
//
// Where this follows the pages and where it departs:
//  * tile grid: ceil-div over N and M as in the TileLang SM100 README
//    ("Code Example", T.Kernel(T.ceildiv(N, block_N), T.ceildiv(M, block_M)));
//    workgroup ids are remapped so each XCD's workgroups cover a compact
//    block of tiles (the pages only name a threadblock-swizzle header,
//    velog "tilelang", 1.3 Code Generation & Runtime).
//  * accumulator init: zero fp32 accumulators (T.clear / clear_accum).
//  * global -> LDS staging: the pages use TMA boxes with a hardware
//    swizzle (velog "tilelang", 1.2 Host IRModule).  Here every lane moves
//    16 bytes with a buffer load that writes LDS directly; the 16-byte
//    chunks of each row are XOR-permuted so the MFMA operand reads hit
//    distinct LDS banks.  Out-of-range rows and the ragged K tail take an
//    out-of-range buffer offset and arrive as zeros (the pages' TMA zero
//    OOB fill).
//  * pipelined K loop: the pages use a 3-slot ring with producer and
//    consumer warpgroups and mbarrier parity waits (velog "tilelang",
//    Device IRModule).  Here every wave both loads and computes: a 4-slot
//    ring, loads issued 3 slices ahead and spread evenly between MFMAs, one
//    s_waitcnt + s_barrier per slice placed so that the first operand reads
//    of the next slice overlap the last MFMAs of the current one.
//  * wave-tile MMA: v_mfma_f32_32x32x16_{bf16,f16} and, for the
//    block-scaled path, v_mfma_scale_f32_32x32x64_f8f6f4 with the e8m0
//    block scales as operands (TCGEN05 tutorial, "进阶" (Advanced)).
//  * NN: B stays K x N in LDS and is read with the LDS transpose read
//    (ds_read_b64_tr_b16), which hands each lane four K values of one column.
//  * epilogue: fp32 -> bf16/fp16 with round-to-nearest-even, masked stores.
//    The MFMA is fed B rows as its first operand and A rows as its second,
//    so each lane's accumulators hold 4 consecutive columns of one row of C
//    and leave as one 8-byte store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "tgemm_internal.hpp"

namespace tgemm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kRowBytes = 64;                   // bytes of one tile row per K slice
constexpr int kSlotBytes = kTileM * kRowBytes;  // one operand, one slot: 16 KiB
constexpr int kAhead = 3;                       // slices loaded ahead of the one multiplied
constexpr uint32_t kOOB = 0x80000000u;          // voffset that is always out of range

static_assert(kTileM == 256 && kTileN == 256, "kernel assumes 256 x 256 tiles");

struct Args {
  const uint8_t *A;
  const uint8_t *B;
  const uint8_t *SA;
  const uint8_t *SB;
  uint8_t *C;
  int M, N, K;
  int tiles_m, tiles_n;
  int ksteps;  // ceil(K / elements per slice)
  int kb;      // scale blocks per row (mxfp8)
};

template <int KIND>
struct Traits;
template <>
struct Traits<0> {  // bf16 NT
  static constexpr int kElem = 2;
  static constexpr bool kNN = false, kScaled = false;
};
template <>
struct Traits<1> {  // fp16 NN
  static constexpr int kElem = 2;
  static constexpr bool kNN = true, kScaled = false;
};
template <>
struct Traits<2> {  // mxfp8 NT
  static constexpr int kElem = 1;
  static constexpr bool kNN = false, kScaled = true;
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

// Wait states between VALU accesses of accumulators and inline-asm MFMAs,
// which the compiler's hazard tracking does not see: 24 idle cycles cover
// the longest MFMA result latency of the forms used here.
__device__ __forceinline__ void mfma_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that orders LDS traffic for the compiler but leaves the
// hardware waits to the caller (no fence, so no implicit vmcnt(0)).
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk permutation inside a 64-byte tile row: row r keeps logical 16-byte
// chunk c at physical chunk c ^ swz(r).  Eight consecutive rows read at one
// logical chunk land on 8 distinct 16-byte bank groups of a 128-byte bank
// period, and sixteen on 16 distinct groups of a 256-byte period.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// NN B slot: 32 K rows of 512 bytes (256 columns).  Row k keeps logical
// chunk c at physical chunk c ^ swz_nn(k), which spreads the four rows read
// together by a transpose read over distinct bank groups.
__device__ __forceinline__ int swz_nn(int k) { return (k & 3) << 1; }

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
// NT kinds) into a slot of 256 rows x 64 bytes.  Wave w moves rows
// [64 w, 64 w + 64) with 4 direct-to-LDS instructions of 16 rows each; lane
// l of instruction i writes LDS bytes [16 l, 16 l + 16) of its 1 KiB row
// group, i.e. row 64 w + 16 i + l / 4, physical chunk l % 4, and therefore
// fetches logical chunk (l % 4) ^ swz(row) of that row.  swz depends on the
// row only through row % 16 = l / 4, so the chunk is the same for all i.
// ---------------------------------------------------------------------------
struct PanelLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[4];  // per instruction: byte offset of this lane's chunk at slice 0
  int kcol;         // element column of this lane's chunk inside a slice

  __device__ __forceinline__ void init(const uint8_t *panel, int rows_valid, int K, int elem, int wave,
                                       int lane) {
    rsrc = make_rsrc(panel, (uint32_t)rows_valid * (uint32_t)K * (uint32_t)elem);
    const int c = (lane & 3) ^ swz(lane >> 2);
    kcol = c * (16 / elem);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wave * 64 + i * 16 + (lane >> 2);
      off[i] = r < rows_valid ? (uint32_t)r * (uint32_t)K * (uint32_t)elem + (uint32_t)c * 16u : kOOB;
    }
  }

  // Instruction i of slice kt.  A chunk at or past column K (the ragged last
  // slice, or a slice past the end) takes an out-of-range offset.
  __device__ __forceinline__ void issue(LDS_AS uint8_t *slot, int wave, int kt, int K, int slice_k, int i) const {
    const bool ok = kt * slice_k + kcol < K;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(slot + wave * 4096 + i * 1024), 16,
                                             ok ? off[i] : kOOB, (uint32_t)kt * kRowBytes, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Staging of one K slice of the NN B operand (K x N, N-contiguous) into a
// slot of 32 K rows x 512 bytes.  Wave w moves K rows [8 w, 8 w + 8) with 4
// instructions of 2 rows each; lane l of instruction i writes row
// 8 w + 2 i + l / 32, physical chunk l % 32, fetching logical chunk
// (l % 32) ^ swz_nn(row), i.e. columns n0 + 8 chunk .. + 8.
// ---------------------------------------------------------------------------
struct NNLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[4];  // per instruction: byte offset at slice 0 (kOOB past N)
  int krow[4];      // K row inside the slice
  uint32_t slice_bytes;

  __device__ __forceinline__ void init(const uint8_t *B, int K, int N, int n0, int wave, int lane) {
    rsrc = make_rsrc(B, (uint32_t)K * (uint32_t)N * 2u);
    slice_bytes = 32u * (uint32_t)N * 2u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = wave * 8 + i * 2 + (lane >> 5);
      const int c = (lane & 31) ^ swz_nn(kr);
      const int n = n0 + c * 8;
      krow[i] = kr;
      off[i] = n < N ? (uint32_t)kr * (uint32_t)N * 2u + (uint32_t)n * 2u : kOOB;
    }
  }

  __device__ __forceinline__ void issue(LDS_AS uint8_t *slot, int wave, int kt, int K, int i) const {
    const bool ok = kt * 32 + krow[i] < K;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(slot + wave * 4096 + i * 1024), 16,
                                             ok ? off[i] : kOOB, (uint32_t)kt * slice_bytes, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
struct Slots {
  LDS_AS uint8_t *a[4];
  LDS_AS uint8_t *b[4];
};

typedef __attribute__((ext_vector_type(4))) float f32x4;

template <int KIND>
struct Kernel {
  using T = Traits<KIND>;
  static constexpr int kElem = T::kElem;
  static constexpr int kSliceK = kRowBytes / kElem;  // K elements per slice
  // MFMA shape.  16-bit inputs: v_mfma_f32_16x16x32 (one per 16 x 16 block per
  // slice; it reads and writes 4 accumulators per 16 K flops, half the
  // accumulator traffic per flop of the 32 x 32 x 16 form, which costs
  // power).  fp8: v_mfma_scale_f32_32x32x64 (one per 32 x 32 block).
  static constexpr int kBlk = T::kScaled ? 32 : 16;
  static constexpr int kNB = 128 / kBlk;       // blocks per wave along M and along N
  static constexpr int kMfma = kNB * kNB;      // MFMAs per slice
  static constexpr int kHalf = kMfma / 2;
  // Load instructions per thread per slice: 4 for the A panel and 4 for B
  // (issued three slices ahead, one per kMfma / 8 MFMAs), plus, for the
  // block-scaled kind, 8 scale bytes (issued one slice ahead, at the start of
  // the slice before).
  static constexpr int kLoads = 8;
  static constexpr int kScaleLoads = T::kScaled ? 8 : 0;
  // The wait in the middle of slice j must cover the panel loads of slice
  // j + 1 (issued during slice j - 2).  Issued after them: the panel loads of
  // slice j + 2, the first half of those of slice j + 3, and the scale loads
  // made at the starts of slices j - 1 and j.
  static constexpr int kWaitVm = kLoads + kLoads / 2 + 2 * kScaleLoads;

  using Frag = typename std::conditional<T::kScaled, i32x8, u32x4>::type;
  using Acc = typename std::conditional<T::kScaled, f32x16, f32x4>::type;
  struct Frags {
    Frag x[kNB], y[kNB];
  };

  const Args &a;
  Slots slots;
  int tid, lane, wave, wave_m, wave_n, lane_sw;
  int m0, n0;
  int nk;
  PanelLoader la, lb;
  NNLoader lnn;
  __amdgpu_buffer_rsrc_t rsa, rsb;
  uint32_t soA[4], soB[4];
  // Scale bytes by slice parity: the B-row scales of the 4 x blocks, then the
  // A-row scales of the 4 y blocks (each in byte 0 of its register).
  int sc[2][8];
  Acc acc[kNB][kNB];

  __device__ __forceinline__ Kernel(const Args &args, const Slots &s) : a(args), slots(s) {}

  // Fragment of one block of kBlk rows (B rows = C columns for x, A rows for
  // y) from a K-contiguous slot.
  __device__ __forceinline__ Frag read_rows(const LDS_AS uint8_t *slot, int row0) const {
    if constexpr (T::kScaled) {
      // 32 x 32 x 64: lane l holds row l % 32, 32 bytes of K: logical chunks
      // 2 (l / 32) and 2 (l / 32) + 1.
      const int hi = lane >> 5;
      const LDS_AS uint8_t *p = slot + (row0 + (lane & 31)) * kRowBytes;
      u32x4 u = *(const LDS_AS u32x4 *)(p + (((2 * hi) ^ lane_sw) << 4));
      u32x4 v = *(const LDS_AS u32x4 *)(p + (((2 * hi + 1) ^ lane_sw) << 4));
      i32x8 r;
      r[0] = u[0]; r[1] = u[1]; r[2] = u[2]; r[3] = u[3];
      r[4] = v[0]; r[5] = v[1]; r[6] = v[2]; r[7] = v[3];
      return r;
    } else {
      // 16 x 16 x 32: lane l holds row l % 16, 8 elements of K: logical
      // chunk l / 16.
      const LDS_AS uint8_t *p = slot + (row0 + (lane & 15)) * kRowBytes;
      return *(const LDS_AS u32x4 *)(p + (((lane >> 4) ^ lane_sw) << 4));
    }
  }

  // NN x fragment: columns n = col0 + l % 16 of the [k][n] B slot, K values
  // 8 (l / 16) + 0..7.  Each transpose read gives a lane 4 K values of one
  // column: in a 16-lane group, source lane 4 e + q points at K row base + e,
  // columns col0 + 4 q .. + 3, and lane i receives column col0 + i.
  __device__ __forceinline__ Frag read_cols(const LDS_AS uint8_t *slot, int col0) const {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int n = col0 + 4 * q;
    u32x4 r;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int kr = 8 * g + 4 * t + e;
      const LDS_AS uint8_t *p = slot + kr * 512 + ((((n >> 3) ^ swz_nn(kr))) << 4) + (n & 7) * 2;
      s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4 *)p);
      u32x2 w = __builtin_bit_cast(u32x2, v);
      r[2 * t] = w[0];
      r[2 * t + 1] = w[1];
    }
    return r;
  }

  // FIRST: the first K slice, whose MFMAs start from an accumulator of 0
  // (an inline constant), so the accumulators are never written by VALU code.
  template <bool FIRST>
  __device__ static __forceinline__ Acc mma(const Frag &x, const Frag &y, const Acc &c, int sx, int sy) {
    // The 16 x 16 forms are written as inline asm with the accumulator tied
    // in place ("+a"): with the builtin the register allocator rotates the
    // 64 accumulator tuples through spare registers on every loop trip.  The
    // compiler still places the LDS waits for the fragment inputs; the
    // accumulators are never written by VALU code and are read by it only
    // after fence_acc().
    if constexpr (KIND == 0) {
      Acc d = c;
      if constexpr (FIRST)
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(d) : "v"(x), "v"(y));
      else
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(x), "v"(y));
      return d;
    } else if constexpr (KIND == 1) {
      Acc d = c;
      if constexpr (FIRST)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, 0" : "=a"(d) : "v"(x), "v"(y));
      else
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+a"(d) : "v"(x), "v"(y));
      return d;
    } else {
      // Format code 0 (OCP FP8 E4M3) for both operands; byte 0 of each scale VGPR.
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, sx, 0, sy);
    }
  }

  // Wait states after the last MFMA before VALU code reads the
  // accumulators.  The empty asm statements redefine every accumulator after
  // the s_nops, so no accumulator read can be scheduled above them.
  __device__ __forceinline__ void fence_acc() {
    mfma_fence();
#pragma unroll
    for (int i = 0; i < kNB; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j) asm volatile("" : "+a"(acc[i][j]));
  }

  // Fragment read R (0 .. 2 kNB - 1) of slot S, in an order that lets the
  // reads reuse the registers of fragments already consumed: the first half
  // of the x blocks, then all y blocks, then the second half of x.
  template <int S, int R>
  __device__ __forceinline__ void read_one(Frags &f) const {
    constexpr int H = kNB / 2;
    if constexpr (R < H || R >= H + kNB) {
      constexpr int i = R < H ? R : R - kNB;
      if constexpr (T::kNN)
        f.x[i] = read_cols(slots.b[S], wave_n * 128 + i * kBlk);
      else
        f.x[i] = read_rows(slots.b[S], wave_n * 128 + i * kBlk);
    } else {
      constexpr int j = R - H;
      f.y[j] = read_rows(slots.a[S], wave_m * 128 + j * kBlk);
    }
  }

  // Load instruction i (0..7) of slice kt into slot S: A panel, then B.
  template <int S>
  __device__ __forceinline__ void load_one(int kt, int i) {
    if (i < 4) {
      la.issue(slots.a[S], wave, kt, a.K, kSliceK, i);
    } else if constexpr (T::kNN) {
      lnn.issue(slots.b[S], wave, kt, a.K, i - 4);
    } else {
      lb.issue(slots.b[S], wave, kt, a.K, kSliceK, i - 4);
    }
  }

  // Scale bytes of slice kt into set P (a slice is half a 128-element
  // scale block).
  template <int P>
  __device__ __forceinline__ void load_scales(int kt) {
    if constexpr (T::kScaled) {
      const bool ok = kt < nk;
      const uint32_t blk = (uint32_t)(kt >> 1);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        sc[P][b] = __builtin_amdgcn_raw_buffer_load_b8(rsb, ok ? soB[b] + blk : kOOB, 0, 0);
        sc[P][4 + b] = __builtin_amdgcn_raw_buffer_load_b8(rsa, ok ? soA[b] + blk : kOOB, 0, 0);
      }
    }
  }

  // MFMA Q of the slice held in slot S (x block Q / kNB times y block
  // Q % kNB), with scale set P.  Every kMfma / 8 MFMAs one load instruction
  // of slice kt + 3 goes out; in the second half, one fragment read of the
  // next slot (slot NX) per MFMA into `nf`.
  template <int S, int P, bool FIRST, int Q>
  __device__ __forceinline__ void mfma_one(int kt, const Frags &f, Frags &nf) {
    constexpr int I = Q / kNB, J = Q % kNB;
    constexpr int kEvery = kMfma / kLoads;
    constexpr int L = (S + kAhead) & 3, NX = (S + 1) & 3;
    if constexpr (Q >= kHalf && Q - kHalf < 2 * kNB) read_one<NX, Q - kHalf>(nf);
    if constexpr (Q % kEvery == kEvery / 2) load_one<L>(kt + kAhead, Q / kEvery);
    if constexpr (T::kScaled)
      acc[I][J] = mma<FIRST>(f.x[I], f.y[J], acc[I][J], sc[P][I], sc[P][4 + J]);
    else
      acc[I][J] = mma<FIRST>(f.x[I], f.y[J], acc[I][J], 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (Q == kHalf - 1) {
      // Slice kt + 1 has landed in slot NX for this wave; once every wave
      // is here it is visible to all, and no wave still reads the slot the
      // next loads will overwrite.
      wait_vm_lgkm0<kWaitVm>();
      barrier();
    }
  }

  template <int S, int P, bool FIRST, int... Q>
  __device__ __forceinline__ void slice_seq(std::integer_sequence<int, Q...>, int kt, const Frags &f, Frags &nf) {
    (mfma_one<S, P, FIRST, Q>(kt, f, nf), ...);
  }

  // One K slice kt from slot S (its fragments already in `f`).
  template <int S, bool FIRST = false>
  __device__ __forceinline__ void step(int kt, const Frags &f, Frags &nf) {
    constexpr int P = S & 1;
    load_scales<P ^ 1>(kt + 1);
    slice_seq<S, P, FIRST>(std::make_integer_sequence<int, kMfma>(), kt, f, nf);
  }

  template <int S, int... R>
  __device__ __forceinline__ void read_all(std::integer_sequence<int, R...>, Frags &f) const {
    (read_one<S, R>(f), ...);
  }

  __device__ __forceinline__ void run() {
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    wave_m = wave >> 1;
    wave_n = wave & 1;
    lane_sw = swz(lane & 15);  // fragment blocks start at multiples of 16 rows

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
    m0 = tm * kTileM;
    n0 = tn * kTileN;
    const int K = a.K;
    nk = a.ksteps;

    la.init(a.A + (size_t)m0 * K * kElem, min(a.M - m0, kTileM), K, kElem, wave, lane);
    if constexpr (T::kNN)
      lnn.init(a.B, K, a.N, n0, wave, lane);
    else
      lb.init(a.B + (size_t)n0 * K * kElem, min(a.N - n0, kTileN), K, kElem, wave, lane);
    if constexpr (T::kScaled) {
      rsa = make_rsrc(a.SA, (uint32_t)a.M * (uint32_t)a.kb);
      rsb = make_rsrc(a.SB, (uint32_t)a.N * (uint32_t)a.kb);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int m = m0 + wave_m * 128 + b * 32 + (lane & 31);
        const int n = n0 + wave_n * 128 + b * 32 + (lane & 31);
        soA[b] = m < a.M ? (uint32_t)m * (uint32_t)a.kb : kOOB;
        soB[b] = n < a.N ? (uint32_t)n * (uint32_t)a.kb : kOOB;
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int b = 0; b < 8; ++b) sc[s][b] = 0;
    if constexpr (T::kScaled) {
#pragma unroll
      for (int i = 0; i < kNB; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) acc[i][j] = Acc{};
    }

    // Prologue: slices 0 .. 2 into slots 0 .. 2 and the scales of slice 0;
    // wait for slice 0.  (With K = 0 every slice is all zeros.)
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_one<0>(0, i);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_one<1>(1, i);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) load_one<2>(2, i);
    load_scales<0>(0);
    wait_vm_lgkm0<2 * kLoads>();
    barrier();
    Frags f0, f1;
    read_all<0>(std::make_integer_sequence<int, 2 * kNB>(), f0);
    // Slice 0 starts the accumulators; then slices go four at a time, one
    // per slot.  The count is padded: slices past nk arrive as zeros and add
    // nothing.  (Leaving the loop early instead makes the register allocator
    // copy the accumulators around and spill.)
    step<0, true>(0, f0, f1);
    for (int kt = 0; kt + 1 < nk; kt += 4) {
      step<1>(kt + 1, f1, f0);
      step<2>(kt + 2, f0, f1);
      step<3>(kt + 3, f1, f0);
      step<0>(kt + 4, f0, f1);
    }
    // Drain the loads still in flight into the ring before the workgroup
    // can finish.
    wait_vm_lgkm0<0>();
    fence_acc();
    epilogue();
  }

  // acc[i][j] covers B rows (C columns) n0 + 128 wave_n + kBlk i and A rows
  // (C rows) m0 + 128 wave_m + kBlk j.  32 x 32 blocks: lane l, register r
  // holds C row l % 32 of the block, column 8 (r / 4) + 4 (l / 32) + r % 4.
  // 16 x 16 blocks: lane l, register r holds row l % 16, column
  // 4 (l / 16) + r.  Either way four consecutive columns leave as one
  // 8-byte store.
  __device__ __forceinline__ void epilogue() {
    constexpr int kRowLanes = kBlk;          // lanes l % kBlk index the row
    constexpr int kGroups = kBlk == 32 ? 4 : 1;
    const int row_l = lane % kRowLanes;
    const int colq = kBlk == 32 ? 4 * (lane >> 5) : 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      const int m = m0 + wave_m * 128 + j * kBlk + row_l;
      if (m >= a.M) continue;
      uint8_t *crow = a.C + (size_t)m * a.N * 2;
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
          const int n = n0 + wave_n * 128 + i * kBlk + g * 8 + colq;
          if (n >= a.N) continue;
          const f32x2 lo = {acc[i][j][4 * g + 0], acc[i][j][4 * g + 1]};
          const f32x2 up = {acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          u32x2 pk;
          if constexpr (KIND == 1) {
            pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, f16x2));
            pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(up, f16x2));
          } else {
            pk[0] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
            pk[1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(up, bf16x2));
          }
          *(u32x2 *)(crow + (size_t)n * 2) = pk;
        }
      }
    }
  }
};

template <int KIND>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(const Args a) {
  // Eight separate arrays (not one indexed array) so the compiler can tell
  // the slot being loaded from the slot being read and does not insert a
  // vmcnt wait in front of every LDS read.
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sA2[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sA3[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sB3[kSlotBytes];
  Slots slots;
  slots.a[0] = (LDS_AS uint8_t *)sA0;
  slots.a[1] = (LDS_AS uint8_t *)sA1;
  slots.a[2] = (LDS_AS uint8_t *)sA2;
  slots.a[3] = (LDS_AS uint8_t *)sA3;
  slots.b[0] = (LDS_AS uint8_t *)sB0;
  slots.b[1] = (LDS_AS uint8_t *)sB1;
  slots.b[2] = (LDS_AS uint8_t *)sB2;
  slots.b[3] = (LDS_AS uint8_t *)sB3;
  Kernel<KIND> k(a, slots);
  k.run();
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
  a.tiles_m = (int)((p.M + kTileM - 1) / kTileM);
  a.tiles_n = (int)((p.N + kTileN - 1) / kTileN);
  const int slice = p.kind == Kind::kMxfp8NT ? 64 : 32;
  a.ksteps = (int)((p.K + slice - 1) / slice);
  a.kb = (int)((p.K + 127) / 128);
  const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(kThreads);
  switch (p.kind) {
    case Kind::kBf16NT:
      hipLaunchKernelGGL(gemm_kernel<0>, grid, block, 0, p.stream, a);
      break;
    case Kind::kF16NN:
      hipLaunchKernelGGL(gemm_kernel<1>, grid, block, 0, p.stream, a);
      break;
    case Kind::kMxfp8NT:
      hipLaunchKernelGGL(gemm_kernel<2>, grid, block, 0, p.stream, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace tgemm
