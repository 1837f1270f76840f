// Tiled dense GEMM kernels for gfx950 (MI355X, CDNA4).
//
// One workgroup of 256 threads (4 wave64s in a 2 x 2 grid) computes a
// 256 x 256 tile of C; each wave owns a 128 x 128 sub-tile held as 4 x 4
// blocks of 32 x 32 fp32 accumulators (256 per lane).  The K loop walks
// 128-byte slices of the A and B row panels (64 bf16/fp16 or 128 fp8
// elements per row), double-buffered in LDS.
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
//    chunks of each 128-byte row are XOR-permuted so the MFMA operand reads
//    hit distinct LDS banks.  Out-of-range rows and the ragged K tail read
//    as zero through the buffer descriptor's range check (the pages' TMA
//    zero OOB fill).
//  * pipelined K loop: the pages use a 3-slot ring with producer and
//    consumer warpgroups and mbarrier parity waits (velog "tilelang",
//    Device IRModule).  Here every wave both loads and computes: while the
//    MFMAs read slot s, the loads for the next K slice fill slot s^1; one
//    s_waitcnt + s_barrier per slice closes the step.
//  * wave-tile MMA: v_mfma_f32_32x32x16_{bf16,f16} and, for the
//    block-scaled path, v_mfma_scale_f32_32x32x64_f8f6f4 with the e8m0
//    block scales as operands (TCGEN05 tutorial, "进阶" (Advanced)).
//  * epilogue: fp32 -> bf16/fp16 with round-to-nearest-even, masked stores.
//    The MFMA is fed B rows as its first operand and A rows as its second,
//    so each lane's accumulators hold 4 consecutive columns of one row of C
//    and leave as one 8-byte store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tgemm_internal.hpp"

namespace tgemm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;                  // bytes of one tile row per K slice
constexpr int kSlotBytes = kTileM * kRowBytes;  // one operand, one slot: 32 KiB
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

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14).
__device__ __forceinline__ void wait_vm0_lgkm0() { __builtin_amdgcn_s_waitcnt(0x0070); }

// Workgroup barrier that orders LDS traffic for the compiler but leaves the
// hardware waits to the caller (no fence, so no implicit vmcnt(0)).
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Chunk permutation inside a 128-byte tile row: row r keeps its logical
// 16-byte chunk c at physical chunk c ^ swz(r).  Any 16 consecutive rows
// read at one logical chunk land on 16 distinct (chunk, row parity) pairs,
// i.e. on distinct banks for both 128-byte and 256-byte bank periods.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

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
// Global -> LDS staging of one K slice of a K-contiguous panel (A of every
// kind, B of the NT kinds).  The slot is 256 rows x 128 bytes.  Wave w moves
// rows [64 w, 64 w + 64) with 8 instructions of 8 rows each; lane l of
// instruction i writes LDS bytes [16 l, 16 l + 16) of its 1 KiB row group,
// i.e. row 64 w + 8 i + l / 8, physical chunk l % 8, and therefore fetches
// logical chunk (l % 8) ^ swz(row) of that row from global memory.
// ---------------------------------------------------------------------------
struct PanelLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[8];   // per instruction: byte offset of this lane's chunk at K slice 0
  int kcol[2];       // element column of this lane's chunk at slice 0 (even / odd i)

  __device__ __forceinline__ void init(const uint8_t *panel, int rows_valid, int K, int elem,
                                       int wave, int lane) {
    rsrc = make_rsrc(panel, (uint32_t)rows_valid * (uint32_t)K * (uint32_t)elem);
    const int chunk_elems = 16 / elem;
    for (int p = 0; p < 2; ++p) kcol[p] = (((lane & 7) ^ (lane >> 3) ^ p)) * chunk_elems;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + (lane >> 3);
      off[i] = r < rows_valid ? (uint32_t)r * (uint32_t)K * (uint32_t)elem + (uint32_t)kcol[i & 1] * elem
                              : kOOB;
    }
  }

  // Per-slice lane predicate: chunks at or past column K (the ragged last
  // slice, or a slice past the end) take an out-of-range offset, so the
  // buffer range check delivers zeros.
  struct Slice {
    uint32_t soff;
    bool ok0, ok1;
  };
  __device__ __forceinline__ Slice slice(int kt, int K, int slice_k) const {
    const int k0 = kt * slice_k;
    return Slice{(uint32_t)kt * kRowBytes, k0 + kcol[0] < K, k0 + kcol[1] < K};
  }
  // Instruction i of slice `sl`: 8 rows x 128 bytes straight into LDS.
  __device__ __forceinline__ void issue_one(LDS_AS uint8_t *slot, int wave, const Slice &sl, int i) const {
    const uint32_t o = ((i & 1) ? sl.ok1 : sl.ok0) ? off[i] : kOOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void *)(slot + wave * 8192 + i * 1024), 16, o,
                                             sl.soff, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// NN B operand (K x N, N-contiguous).  Thread t owns an 8 x 8 block: rows
// k = 8 (t / 32) .. +8 of the slice, columns n = 8 (t % 32) .. +8 of the tile.
// It loads the 8 row pieces (16 bytes each, coalesced across the wave),
// transposes the block in registers and writes 8 LDS rows (one per column n)
// of 8 K values, in the same swizzled [n][k] layout as an NT B slot.
// ---------------------------------------------------------------------------
struct NNLoader {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off0;   // byte offset of row k = 8 (t / 32), column n of this thread, at slice 0
  uint32_t row_stride;
  int krow0;       // first k of this thread's block inside a slice
  bool col_ok;
  u32x4 v[8];

  __device__ __forceinline__ void init(const uint8_t *B, int K, int N, int n0, int tid) {
    rsrc = make_rsrc(B, (uint32_t)K * (uint32_t)N * 2u);
    const int nc = tid & 31;
    krow0 = (tid >> 5) * 8;
    const int n = n0 + nc * 8;
    col_ok = n < N;
    row_stride = (uint32_t)N * 2u;
    off0 = (uint32_t)krow0 * row_stride + (uint32_t)n * 2u;
  }

  // Row j of this thread's block of slice kt (zeros past K or past N).
  __device__ __forceinline__ void load_one(int kt, int K, int j) {
    const int k = kt * 64 + krow0 + j;
    const uint32_t o = (col_ok && k < K) ? off0 + (uint32_t)(kt * 64 + j) * row_stride : kOOB;
    v[j] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, o, 0, 0);
  }

  __device__ __forceinline__ void store(LDS_AS uint8_t *slot, int tid) const {
    const int nc = tid & 31, kc = tid >> 5;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = i >> 1;
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;  // high or low fp16 halves
      u32x4 o;
      o[0] = __builtin_amdgcn_perm(v[1][d], v[0][d], sel);
      o[1] = __builtin_amdgcn_perm(v[3][d], v[2][d], sel);
      o[2] = __builtin_amdgcn_perm(v[5][d], v[4][d], sel);
      o[3] = __builtin_amdgcn_perm(v[7][d], v[6][d], sel);
      const int n = nc * 8 + i;
      *(LDS_AS u32x4 *)(slot + n * kRowBytes + ((kc ^ swz(n)) << 4)) = o;
    }
  }
};

// The kernel.
// ---------------------------------------------------------------------------
struct Slots {
  LDS_AS uint8_t *a[2];
  LDS_AS uint8_t *b[2];
};

template <int KIND>
struct Kernel {
  using T = Traits<KIND>;
  static constexpr int kElem = T::kElem;
  static constexpr int kSliceK = kRowBytes / kElem;     // K elements per slice
  static constexpr int kSubsteps = T::kScaled ? 2 : 4;  // MFMAs along K per slice

  // Operand fragment of one 32-row block for one K substep.
  using Frag = typename std::conditional<T::kScaled, i32x8, u32x4>::type;

  const Args &a;
  Slots slots;
  int tid, lane, wave, wave_m, wave_n, hi, lane_sw;
  int m0, n0;
  int nk;
  PanelLoader la, lb;
  NNLoader lnn;
  __amdgpu_buffer_rsrc_t rsa, rsb;
  uint32_t soA[4], soB[4];
  int sc[2][8];  // per slot: B-row scales of the 4 x blocks, then A-row scales of the 4 y blocks
  f32x16 acc[4][4];

  __device__ __forceinline__ Kernel(const Args &args, const Slots &s) : a(args), slots(s) {}

  __device__ __forceinline__ Frag read_frag(const LDS_AS uint8_t *slot, int row, int sub) const {
    const LDS_AS uint8_t *p = slot + row * kRowBytes;
    if constexpr (T::kScaled) {
      // 32 bytes of K per lane: logical chunks 4 sub + 2 hi and 4 sub + 2 hi + 1.
      const int c0 = 4 * sub + 2 * hi;
      u32x4 u = *(const LDS_AS u32x4 *)(p + ((c0 ^ lane_sw) << 4));
      u32x4 v = *(const LDS_AS u32x4 *)(p + (((c0 + 1) ^ lane_sw) << 4));
      i32x8 r;
      r[0] = u[0]; r[1] = u[1]; r[2] = u[2]; r[3] = u[3];
      r[4] = v[0]; r[5] = v[1]; r[6] = v[2]; r[7] = v[3];
      return r;
    } else {
      // 16 bytes (8 elements) of K per lane: logical chunk 2 sub + hi.
      const int c = 2 * sub + hi;
      return *(const LDS_AS u32x4 *)(p + ((c ^ lane_sw) << 4));
    }
  }

  __device__ static __forceinline__ f32x16 mma(const Frag &x, const Frag &y, const f32x16 &c, int sx, int sy) {
    if constexpr (KIND == 0) {
      return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y),
                                                     c, 0, 0, 0);
    } else if constexpr (KIND == 1) {
      return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, x), __builtin_bit_cast(f16x8, y), c,
                                                    0, 0, 0);
    } else {
      // Format code 0 (OCP FP8 E4M3) for both operands; byte 0 of each scale VGPR.
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, y, c, 0, 0, 0, sx, 0, sy);
    }
  }

  // Fragments of one K substep: x = 4 blocks of B rows, y = 4 blocks of A rows.
  struct Frags {
    Frag x[4], y[4];
  };

  // Fragment read q (0..7) of substep `sub` of slot S, in order of first use
  // by the MFMA sequence (x[0] with y[0..3], then x[1], x[2], x[3]):
  // q = 0 -> x[0], 1..4 -> y[0..3], 5..7 -> x[1..3].
  template <int S>
  __device__ __forceinline__ void read_one(Frags &f, int sub, int q) const {
    if (q >= 1 && q <= 4) {
      const int j = q - 1;
      f.y[j] = read_frag(slots.a[S], wave_m * 128 + j * 32 + (lane & 31), sub);
    } else {
      const int i = q == 0 ? 0 : q - 4;
      f.x[i] = read_frag(slots.b[S], wave_n * 128 + i * 32 + (lane & 31), sub);
    }
  }

  // Load instruction q (0..15) of slice kt into slot S: 8 A-panel DMAs, then
  // the B side (8 DMAs for NT, 8 row loads into registers for NN).
  template <int S>
  __device__ __forceinline__ void load_one(int kt, const PanelLoader::Slice &sa, const PanelLoader::Slice &sb,
                                           int q) {
    if (q < 8) {
      la.issue_one(slots.a[S], wave, sa, q);
    } else if constexpr (T::kNN) {
      lnn.load_one(kt, a.K, q - 8);
    } else {
      lb.issue_one(slots.b[S], wave, sb, q - 8);
    }
  }

  template <int S>
  __device__ __forceinline__ void load_scales(int kt) {
    if constexpr (T::kScaled) {
      const bool ok = kt < nk;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        sc[S][b] = __builtin_amdgcn_raw_buffer_load_b8(rsb, ok ? soB[b] + (uint32_t)kt : kOOB, 0, 0);
        sc[S][4 + b] = __builtin_amdgcn_raw_buffer_load_b8(rsa, ok ? soA[b] + (uint32_t)kt : kOOB, 0, 0);
      }
    }
  }

  // The 16 MFMAs of one substep on fragments `f` with the scales of slot S,
  // interleaved with 8 fragment reads into `nf` (slot RS, substep rsub) and,
  // if LOAD, the 16 load instructions of slice lkt into slot LS.
  template <int S, int RS, int LS, bool LOAD>
  __device__ __forceinline__ void mfma16(const Frags &f, Frags &nf, int rsub, int lkt, const PanelLoader::Slice &sa,
                                         const PanelLoader::Slice &sb) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if constexpr (LOAD) load_one<LS>(lkt, sa, sb, q);
      if ((q & 1) == 0) read_one<RS>(nf, rsub, q >> 1);
      const int i = q >> 2, j = q & 3;
      acc[i][j] = mma(f.x[i], f.y[j], acc[i][j], sc[S][i], sc[S][4 + j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // One K step on slot S (slice kt), entered with substep 0's fragments in
  // f0.  The loads of slice kt + 1 into the other slot go out during
  // substep 0.  Before the last substep the wave waits for them and the
  // workgroup synchronises, so the last substep's MFMAs overlap the first
  // fragment reads of slice kt + 1.
  template <int S>
  __device__ __forceinline__ void step(int kt, Frags &f0, Frags &f1) {
    const auto sa = la.slice(kt + 1, a.K, kSliceK);
    const auto sb = lb.slice(kt + 1, a.K, kSliceK);
    load_scales<S ^ 1>(kt + 1);
    if constexpr (kSubsteps == 4) {
      mfma16<S, S, S ^ 1, true>(f0, f1, 1, kt + 1, sa, sb);
      mfma16<S, S, S ^ 1, false>(f1, f0, 2, kt + 1, sa, sb);
      mfma16<S, S, S ^ 1, false>(f0, f1, 3, kt + 1, sa, sb);
    } else {
      mfma16<S, S, S ^ 1, true>(f0, f1, 1, kt + 1, sa, sb);
    }
    if constexpr (T::kNN) lnn.store(slots.b[S ^ 1], tid);
    wait_vm0_lgkm0();
    barrier();
    mfma16<S, S ^ 1, S ^ 1, false>(f1, f0, 0, kt + 1, sa, sb);
  }

  __device__ __forceinline__ void run() {
    tid = threadIdx.x;
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    wave_m = wave >> 1;
    wave_n = wave & 1;
    hi = lane >> 5;
    lane_sw = swz(lane & 31);  // fragment blocks start at multiples of 32 rows

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);
    m0 = tm * kTileM;
    n0 = tn * kTileN;
    const int K = a.K;
    nk = a.ksteps;

    la.init(a.A + (size_t)m0 * K * kElem, min(a.M - m0, kTileM), K, kElem, wave, lane);
    if constexpr (T::kNN)
      lnn.init(a.B, K, a.N, n0, tid);
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
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    if (nk > 0) {
      {
        const auto sa = la.slice(0, K, kSliceK);
        const auto sb = lb.slice(0, K, kSliceK);
#pragma unroll
        for (int q = 0; q < 16; ++q) load_one<0>(0, sa, sb, q);
        load_scales<0>(0);
        if constexpr (T::kNN) lnn.store(slots.b[0], tid);
        wait_vm0_lgkm0();
        barrier();
      }
      Frags f0, f1;
#pragma unroll
      for (int q = 0; q < 8; ++q) read_one<0>(f0, 0, q);
      // Slices are taken in pairs; with an odd count the last pair's second
      // slice is all zeros.
      for (int kt = 0; kt < nk; kt += 2) {
        step<0>(kt, f0, f1);
        step<1>(kt + 1, f0, f1);
      }
    }
    epilogue();
  }

  // acc[i][j] covers B rows (C columns) n0 + 128 wave_n + 32 i and A rows
  // (C rows) m0 + 128 wave_m + 32 j.  Lane l, register r holds C row l % 32
  // of the block, column 8 (r / 4) + 4 (l / 32) + r % 4.
  __device__ __forceinline__ void epilogue() {
    const int row_l = lane & 31;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wave_m * 128 + j * 32 + row_l;
      if (m >= a.M) continue;
      uint8_t *crow = a.C + (size_t)m * a.N * 2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wave_n * 128 + i * 32 + g * 8 + hi * 4;
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
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[kSlotBytes];
  Slots slots;
  slots.a[0] = (LDS_AS uint8_t *)sA0;
  slots.a[1] = (LDS_AS uint8_t *)sA1;
  slots.b[0] = (LDS_AS uint8_t *)sB0;
  slots.b[1] = (LDS_AS uint8_t *)sB1;
  // An AGPR operand in inline asm keeps AGPR allocation enabled for this
  // kernel, so the MFMAs accumulate in AGPRs instead of spilling VGPRs.
  asm volatile("; agpr %0" ::"a"(0));
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
  const int slice = p.kind == Kind::kMxfp8NT ? 128 : 64;
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
