// gemm.hip -- grouped GEMMs of the non-gated expert MLPs on CDNA4 MFMA, and
// the per-row fp8 quantiser.
//
// Experts are up_proj -> relu^2 -> down_proj with no gate projection (vllm.cpp
// PR "spec(MODEL-TEXT-nemotron-h)"; auto-round PR "feat: support Nemotron-H /
// Nemotron-Cascade-2", log: Linear(2688 -> 1856) and Linear(1856 -> 2688),
// bias=False), so each expert is two plain GEMMs with relu^2 between them;
// relu^2 is fused into the epilogue of the first.
//
// Both operands are K-contiguous (activation rows, and weight rows in the
// nn.Linear [out, in] layout), which is what the MFMA fragments want: a lane
// reads 16 (or 32) contiguous bytes of one row.  A workgroup of 4 waves owns a
// BM x BN output tile of one group (expert); its M tile comes from a schedule
// built on the device from the group offsets, so the host never learns the
// per-expert counts.  A rows are gathered through the routing permutation
// while loading, so the permuted activations never exist in memory.
//
// Kernels, by tile shape (pick_gemm_shape):
//  * decode, a handful of rows per expert (each weight byte feeds one MFMA:
//    the launch is a weight stream): 16 x 64 tiles, gemm_dec_kernel for bf16
//    weights (buffer loads, two stages in flight), gemm_kernel otherwise;
//  * 64 x 128 and 128 x 128 tiles: gemm_kernel, K in 128-byte stages through
//    a double buffer in LDS, the next stage's loads issued before the current
//    stage's MFMAs;
//  * hundreds of rows per expert: 256 x 256 tiles, gemm_ring_kernel (K in
//    64-byte slices fetched straight into a 4-stage LDS ring; fp8 keeps the
//    weight rows two 128-byte steps ahead, the activation rows one);
//  * the router's logits (a dense GEMM against the small gate matrix):
//    gemm_stream_kernel, 16- to 64-row tiles over a DMA ring;
//  * MXFP4 weights: gemm_fp4_kernel (16- or 64-row tiles).
// Every output element accumulates its K steps in ascending order with the
// same MFMA, whichever tile shape computes it (for fp4: the same order for
// both of its shapes), so results do not depend on the launch configuration.
#include <type_traits>

#include "internal.hpp"

namespace moe {

namespace {

constexpr int BKB = 128;             // K bytes per stage and row
constexpr int LDS_STRIDE = BKB + 16; // padded LDS row

template <int KIND>
struct KindTraits;
template <>
struct KindTraits<K_F32> {
  static constexpr int ESZ = 4;   // bytes per element
  static constexpr int STEP = 64; // K bytes consumed by one MFMA group
};
template <>
struct KindTraits<K_BF16> {
  static constexpr int ESZ = 2;
  static constexpr int STEP = 64;
};
template <>
struct KindTraits<K_FP8> {
  static constexpr int ESZ = 1;
  static constexpr int STEP = 128;
};

template <int KIND>
struct Frag {
  using T = i32x4_t;
};
template <>
struct Frag<K_FP8> {
  using T = i32x8_t;
};

// Fragment bytes of one lane: p[0..FB) (LDS or global memory).
template <int KIND>
__device__ __forceinline__ typename Frag<KIND>::T load_frag(const char* p) {
  if constexpr (KIND == K_FP8) {
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(p);
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(p + 16);
    i32x8_t r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  } else {
    return *reinterpret_cast<const i32x4_t*>(p);
  }
}

template <int KIND>
__device__ __forceinline__ f32x4_t mma(typename Frag<KIND>::T a, typename Frag<KIND>::T b,
                                       f32x4_t c) {
  if constexpr (KIND == K_FP8)
    return mfma_fp8(a, b, c);
  else if constexpr (KIND == K_BF16)
    return mfma_bf16(a, b, c);
  else
    return mfma_f32x4(a, b, c);
}

// Which problem, group and rows a workgroup's tile covers.  The problem is
// copied field by field with uniform selects: indexing the kernel-argument
// array by a runtime value would move it to scratch memory.
struct Tile {
  GemmProblem p;
  int g;        // group inside the problem
  int64_t m0;   // first problem row
  int64_t gend; // end of the group's rows
  int n0;       // first output column
};

__device__ __forceinline__ GemmProblem pick_problem(const GemmArgs& pa, bool second) {
  const GemmProblem& a = pa.prob[0];
  const GemmProblem& b = pa.prob[1];
  GemmProblem p;
  p.a = second ? b.a : a.a;
  p.a_scale = second ? b.a_scale : a.a_scale;
  p.row_index = second ? b.row_index : a.row_index;
  p.w = second ? b.w : a.w;
  p.w_scale = second ? b.w_scale : a.w_scale;
  p.w_bscale = second ? b.w_bscale : a.w_bscale;
  p.offsets = second ? b.offsets : a.offsets;
  p.out = second ? b.out : a.out;
  p.a_rows = second ? b.a_rows : a.a_rows;
  p.rows = second ? b.rows : a.rows;
  p.n = second ? b.n : a.n;
  p.k = second ? b.k : a.k;
  p.index_div = second ? b.index_div : a.index_div;
  p.out_bf16 = second ? b.out_bf16 : a.out_bf16;
  return p;
}

// Workgroups are handed to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8), and each XCD has its own L2.  The chip as a whole works through a
// window of about `resident` consecutive tiles at a time (consecutive tiles
// share A rows, and nearby M tiles of one expert share weight tiles through
// the chip-wide cache); inside each window XCD x takes a contiguous slice, so
// the tiles one L2 serves overlap as much as possible.
__device__ __forceinline__ int xcd_tile_order(int b, int grid, int per_xcd) {
  constexpr int XCDS = 8;
  const int W = XCDS * per_xcd;
  const int base = (b / W) * W;
  const int n = min(W, grid - base);  // size of this window
  const int r = b - base;
  const int xcd = r % XCDS, local = r / XCDS;
  const int per = n / XCDS, rem = n % XCDS;
  return base + (xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local);
}

template <int BM, int BN>
__device__ __forceinline__ bool locate_tile(const GemmArgs& pa, Tile& t, int bid) {
  int mt = bid / pa.n_tiles;
  int nt = bid - mt * pa.n_tiles;
  int gs;
  if (pa.sched) {
    // the first problem's M tiles take n_tiles workgroups each and the
    // second's n_tiles2; with second_first the second problem's come first
    const int first = pa.sched[1];
    const int n_second = pa.sched[0] - first;
    const int b2 = bid - (pa.second_first ? n_second * pa.n_tiles2 : first * pa.n_tiles);
    const bool in_second = pa.second_first ? b2 < 0 : b2 >= 0;
    if (in_second) {
      // (a launch without the second problem has n_tiles2 = 0)
      if (n_second <= 0 || pa.n_tiles2 <= 0) return false;
      const int b = pa.second_first ? bid : b2;
      const int m2 = b / pa.n_tiles2;
      if (m2 >= n_second) return false;
      mt = first + m2;
      nt = b - m2 * pa.n_tiles2;
    } else {
      const int b = pa.second_first ? b2 : bid;
      mt = b / pa.n_tiles;
      nt = b - mt * pa.n_tiles;
      if (mt >= first) return false;
    }
    const int32_t e = pa.sched[2 + 2 * mt];
    gs = e & 0xFFFF;
    t.m0 = pa.sched[3 + 2 * mt];
    t.gend = t.m0 + (e >> 16);  // the tile's rows, from the schedule
  } else {  // dense: one group, tiles in row order
    gs = 0;
    t.m0 = int64_t(mt) * BM;
    if (t.m0 >= pa.prob[0].rows) return false;
    t.gend = pa.prob[0].rows;
  }
  // schedule group n_groups is the single group of the second problem
  const bool second = gs >= pa.n_groups;
  t.p = pick_problem(pa, second);
  t.g = second ? 0 : gs;
  t.n0 = nt * BN;
  return t.n0 < t.p.n;
}

__device__ __forceinline__ int64_t src_row(const GemmProblem& p, int64_t r) {
  int64_t src = p.row_index ? int64_t(p.row_index[r]) / p.index_div : r;
  return min<int64_t>(max<int64_t>(src, 0), p.a_rows - 1);
}

// Stores one 16x16 accumulator block: lane holds column `col`, rows r0..r0+3.
template <int KIND, int EPI>
__device__ __forceinline__ void store_block(const Tile& t, f32x4_t acc, int64_t r0, int col) {
  const GemmProblem& p = t.p;
  if (col >= p.n) return;
  const float sw = KIND == K_FP8 ? p.w_scale[int64_t(t.g) * p.n + col] : 1.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t r = r0 + q;
    if (r >= t.gend) return;
    float v = acc[q];
    if (KIND == K_FP8) v = (v * p.a_scale[src_row(p, r)]) * sw;
    if (EPI == EPI_RELU2) {
      v = fmaxf(v, 0.0f);
      v = v * v;
    }
    if (p.out_bf16)
      static_cast<uint16_t*>(p.out)[r * p.n + col] = f32_to_bf16(v);
    else
      static_cast<float*>(p.out)[r * p.n + col] = v;
  }
}

template <int KIND, int BM, int BN, int WM, int WN, int EPI, int NTHR, int XCD_C>
__global__ __launch_bounds__(NTHR) void gemm_kernel(GemmArgs pa) {
  constexpr int G_THREADS = NTHR;
  constexpr int ESZ = KindTraits<KIND>::ESZ;
  constexpr int STEP = KindTraits<KIND>::STEP;
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  static_assert(WM * WN * WAVE == NTHR, "one wave per wave tile");
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
  constexpr int CPR = BKB / 16;  // 16-byte chunks per row and stage
  constexpr int A_CHUNKS = BM * CPR;
  constexpr int B_CHUNKS = BN * CPR;
  constexpr int CA = (A_CHUNKS + G_THREADS - 1) / G_THREADS;
  constexpr int CB = (B_CHUNKS + G_THREADS - 1) / G_THREADS;
  constexpr int RPT = G_THREADS / CPR;  // rows covered per pass of the block
  constexpr int STAGE = (BM + BN) * LDS_STRIDE;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  Tile t;
  const int bid = XCD_C ? xcd_tile_order(blockIdx.x, gridDim.x, XCD_C) : int(blockIdx.x);
  if (!locate_tile<BM, BN>(pa, t, bid)) return;
  const GemmProblem& p = t.p;
  const int tid = threadIdx.x;
  const int64_t kbytes = int64_t(p.k) * ESZ;
  const char* wbase = static_cast<const char*>(p.w) + int64_t(t.g) * p.n * kbytes;
  const int c16 = (tid % CPR) * 16;  // this thread's byte column inside a stage

  // source row of each chunk this thread loads (null = zero fill)
  const char* a_src[CA];
  const char* b_src[CB];
#pragma unroll
  for (int j = 0; j < CA; ++j) {
    const int row = tid / CPR + j * RPT;
    const int64_t r = t.m0 + row;
    a_src[j] = (row < BM && r < t.gend)
                   ? static_cast<const char*>(p.a) + src_row(p, r) * kbytes + c16
                   : nullptr;
  }
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int row = tid / CPR + j * RPT;
    const int n = t.n0 + row;
    b_src[j] = (row < BN && n < p.n) ? wbase + int64_t(n) * kbytes + c16 : nullptr;
  }

  i32x4_t ra[CA], rb[CB];
  auto gload = [&](int it) {
    const int64_t kb = int64_t(it) * BKB;
    const bool kin = kb + c16 < kbytes;
#pragma unroll
    for (int j = 0; j < CA; ++j) {
      ra[j] = i32x4_t{0, 0, 0, 0};
      if (a_src[j] && kin) ra[j] = *reinterpret_cast<const i32x4_t*>(a_src[j] + kb);
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      rb[j] = i32x4_t{0, 0, 0, 0};
      if (b_src[j] && kin) rb[j] = *reinterpret_cast<const i32x4_t*>(b_src[j] + kb);
    }
  };
  auto sstore = [&](int buf) {
    char* As = smem + buf * STAGE;
    char* Bs = As + BM * LDS_STRIDE;
#pragma unroll
    for (int j = 0; j < CA; ++j) {
      const int row = tid / CPR + j * RPT;
      if (row < BM) *reinterpret_cast<i32x4_t*>(As + row * LDS_STRIDE + c16) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      const int row = tid / CPR + j * RPT;
      if (row < BN) *reinterpret_cast<i32x4_t*>(Bs + row * LDS_STRIDE + c16) = rb[j];
    }
  };

  const int wave = tid / WAVE;
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int lane = lane_id();
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  constexpr int FB = STEP / 4;  // fragment bytes per lane

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = static_cast<int>((kbytes + BKB - 1) / BKB);
  gload(0);
  sstore(0);
  __syncthreads();
  for (int it = 0; it < nk; ++it) {
    if (it + 1 < nk) gload(it + 1);
    const char* As = smem + (it & 1) * STAGE + (wm * (BM / WM) + lrow) * LDS_STRIDE + lgrp * FB;
    const char* Bs = smem + (it & 1) * STAGE + BM * LDS_STRIDE +
                     (wn * (BN / WN) + lrow) * LDS_STRIDE + lgrp * FB;
#pragma unroll
    for (int ks = 0; ks < BKB / STEP; ++ks) {
      typename Frag<KIND>::T af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = load_frag<KIND>(As + i * 16 * LDS_STRIDE + ks * STEP);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = load_frag<KIND>(Bs + j * 16 * LDS_STRIDE + ks * STEP);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma<KIND>(af[i], bfr[j], acc[i][j]);
    }
    if (it + 1 < nk) sstore((it + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      store_block<KIND, EPI>(t, acc[i][j], t.m0 + wm * (BM / WM) + i * 16 + lgrp * 4,
                             t.n0 + wn * (BN / WN) + j * 16 + lrow);
}

// ------------------------------------------------------------ ring kernel
//
// Large grouped GEMMs (hundreds of rows per expert and up): a 256 x 256 tile
// per workgroup of 8 waves (2 along M x 4 along N, 128 x 64 each), K streamed
// in 64-byte row slices through a ring of four LDS stages.  The slices are
// fetched straight into LDS (global_load_lds_dwordx4: lane L of a wave's
// instruction lands at byte 16 L of a 1 KB block) three stages ahead of their
// use, so HBM and cache latency hide behind three stages of MFMA work and no
// registers are spent on staging.  One barrier per stage.
//
// LDS layout of a stage: 16-row blocks of 1 KB, A blocks then B blocks; row r
// of a block holds its 16-byte chunk c in slot c ^ swz(r), swz(r) = 3 for
// rows 8..15 and 0 below.  The layout is set by the LDS's banking as measured
// on gfx950: 64 banks of 4 bytes, and a ds_read_b128 serves 16 lanes a clock,
// the lanes with the same bit 5 and the same parity of bits 2..4 of the lane
// id (lanes 0-3, 12-15 and 20-27 share a clock, and so on).  A fragment read
// has lane l on row l & 15 and chunk l >> 4, so each clock's 16 lanes cover
// the 16 rows once; rows r, r + 4, r + 8, r + 12 fall on the same 64 banks'
// quarter, and the swizzle gives their four chunks four different slots.  The
// reads are then conflict-free (two-way with no swizzle, or with a swizzle that
// assumes consecutive lanes share a clock: half the LDS rate).  The fp8 loop's
// paired-chunk reads are conflict-free with the same swizzle.  Each lane still
// receives the same K elements as in gemm_kernel, so both kernels give
// identical results.
constexpr int RG_BM = 256, RG_BN = 256;
constexpr int RG_ROWB = 64;                          // K bytes per row and stage
constexpr int RG_ABYTES = RG_BM * RG_ROWB;           // A part of a stage
constexpr int RG_STAGE = (RG_BM + RG_BN) * RG_ROWB;  // 32 KB
constexpr int RG_BLOCKS = (RG_BM + RG_BN) / 16;      // 1 KB blocks per stage

__device__ __forceinline__ int rg_swizzle(int r) { return 3 * ((r >> 3) & 1); }

#define MOE_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))


// s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}
constexpr int WAIT_VM0 = waitcnt_imm(0, 15);

__device__ __forceinline__ void block_sync_lds() {
  // Orders the DMA waits and LDS reads around the barrier for the compiler
  // without the full fence of __syncthreads (which would wait for every
  // stage in flight).
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// LDS of a ring kernel: RING stages (bf16); for fp8 two activation slots and
// three weight slots of two stages each, 160 KB.
template <int KIND, int NW, int RING>
constexpr int ring_bytes() {
  return KIND == K_FP8 ? 5 * RG_STAGE : RING * RG_STAGE;
}

// One 256 x 256 tile `t` of a ring kernel; `ring` is the kernel's LDS ring
// (its only __shared__ object).  NW waves in a 2 x (NW / 2) grid; wave
// (wm, wn) owns the 16-row blocks wm + 2 i and the 16-column blocks
// wn + (NW / 2) j of the tile, dealt round-robin so that partial tiles leave
// every SIMD about the same work.
template <int KIND, int EPI, int NW, int RING>
__device__ __forceinline__ void ring_tile(const Tile& t, char* ring) {
  constexpr int WM = 2, WN = NW / 2;
  constexpr int FM = RG_BM / WM / 16;  // 8
  constexpr int FN = RG_BN / WN / 16;  // 4 (8 waves) or 8 (4 waves)
  constexpr int DMA_PER_WAVE = RG_BLOCKS / NW;  // per stage
  constexpr int QUARTERS = 4;
  static_assert(KIND == K_BF16 || KIND == K_FP8, "the ring kernel takes bf16 or fp8 operands");
  static_assert(DMA_PER_WAVE % QUARTERS == 0 && FN % QUARTERS == 0, "quarter split");
  // (a fifth bf16 slot, 160 KB in all, measured 2-3% slower)
  static_assert(KIND == K_BF16 ? (RING == 4 || RING == 5) : RING == 4, "ring depth");
  static_assert(KIND != K_FP8 || NW * WAVE == RG_BM + RG_BN, "one scale per thread");
  const GemmProblem& p = t.p;
  // (the wave index through readfirstlane: the compiler then knows it, and all
  // that derives from it, to be the same on every lane of the wave, so tests
  // on it are scalar branches instead of per-lane exec masks)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int lane = lane_id();
  const int64_t kbytes = int64_t(p.k) * KindTraits<KIND>::ESZ;
  const int nk = static_cast<int>(kbytes / RG_ROWB);  // the host guarantees K bytes % 64 == 0

  // DMA sources: wave w fetches the 16-row blocks w + NW q of the stage
  // (blocks 0..15 are A rows, 16..31 B rows).  Lane L covers row L >> 2 of a
  // block and LDS chunk slot L & 3, which holds global chunk (L & 3) ^
  // swizzle.  Rows past the group end (A) or past N (B) re-read the last
  // valid row: they feed only outputs that are never stored.
  const int r_in = lane >> 2;
  const int chunk = (lane & 3) ^ rg_swizzle(r_in);
  const char* wbase = static_cast<const char*>(p.w) + int64_t(t.g) * p.n * kbytes;
  // (blocks w + NW q with q < 16 / NW are A rows, the rest B rows; the A
  // rows' permutation indices are all loaded before any is used, from a
  // harmless address when the problem has no permutation)
  static_assert(16 % NW == 0, "A and B blocks split by q");
  constexpr int QA = 16 / NW;
  // (fp8, whose registers are full, resolves them one at a time)
  const char* src[DMA_PER_WAVE];
  int32_t perm[QA];
  if constexpr (KIND != K_FP8) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int64_t r = min<int64_t>(t.m0 + (wave + NW * q) * 16 + r_in, t.gend - 1);
      perm[q] = *(p.row_index ? p.row_index + r : static_cast<const int32_t*>(p.a));
    }
  }
#pragma unroll
  for (int q = 0; q < DMA_PER_WAVE; ++q) {
    const int blk = wave + NW * q;
    const int row = (blk % 16) * 16 + r_in;
    if (KIND == K_FP8 ? blk < 16 : q < QA) {
      int64_t a_row;
      if constexpr (KIND == K_FP8) {
        a_row = src_row(p, min<int64_t>(t.m0 + row, t.gend - 1));
      } else {
        const int64_t r = min<int64_t>(t.m0 + row, t.gend - 1);
        a_row = p.row_index ? int64_t(perm[q] / p.index_div) : r;
        a_row = min<int64_t>(max<int64_t>(a_row, 0), p.a_rows - 1);
      }
      src[q] = static_cast<const char*>(p.a) + a_row * kbytes + chunk * 16;
    } else {
      const int n = min(t.n0 + row, p.n - 1);
      src[q] = wbase + int64_t(n) * kbytes + chunk * 16;
    }
  }
  // fp8: the fetch sources again, as a uniform base plus a 32-bit lane offset
  // (the host keeps a_rows K and N K below 2^32 for this kernel), which the
  // main K steps advance with scalar adds only
  const char* const a_base = static_cast<const char*>(p.a);
  uint32_t a_off[2] = {0, 0}, w_off[2] = {0, 0};
  if constexpr (KIND == K_FP8) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      a_off[q] = static_cast<uint32_t>(src[q] - a_base);
      w_off[q] = static_cast<uint32_t>(src[q + 2] - wbase);
    }
  }
  int dma_on = 0;  // bit q: block wave + NW q is fetched (set with the tile's extent below)
  auto dma_one = [&](int q, int s, char* buf) {
    const int64_t kb = int64_t(min(s, nk - 1)) * RG_ROWB;  // past the end: harmless re-read
    // (through a plain pointer: clang drops the host launch stub of this
    // template when an element of the dependently sized array is passed to
    // the builtin directly)
    const void* from = src[q] + kb;
    if (KIND != K_FP8 || (dma_on & (1 << q)))
      __builtin_amdgcn_global_load_lds(from, MOE_LDS_PTR(buf + (wave + NW * q) * 1024), 16, 0, 0);
  };
  auto dma = [&](int s, char* buf) {
#pragma unroll
    for (int q = 0; q < DMA_PER_WAVE; ++q) dma_one(q, s, buf);
  };

  // fp8: thread i holds scale i of the tile (the activation rows' scales,
  // then the weight rows'); they move into the ring once the K loop has
  // freed it, for the epilogue.
  float* sc_row = reinterpret_cast<float*>(ring);
  float* sc_col = sc_row + RG_BM;
  float my_scale = 0.0f;
  if constexpr (KIND == K_FP8) {
    const int i = threadIdx.x;
    if (i < RG_BM) {
      const int64_t r = t.m0 + i;
      my_scale = r < t.gend ? p.a_scale[src_row(p, r)] : 0.0f;
    } else {
      const int n = t.n0 + i - RG_BM;
      my_scale = n < p.n ? p.w_scale[int64_t(t.g) * p.n + n] : 0.0f;
    }
  }

  const int wm = wave % WM;
  const int wn = wave / WM;
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int lofs = lrow * RG_ROWB + ((lgrp ^ rg_swizzle(lrow)) * 16);

  // Work skipped in partial tiles: fragments whose 16 rows all lie past the
  // group end, or whose 16 columns all lie past N.
  const int mblk = static_cast<int>((min<int64_t>(t.gend - t.m0, RG_BM) + 15) / 16);
  const int fm_valid = min(max((mblk - wm + WM - 1) / WM, 0), FM);
  const int nblk = (min(p.n - t.n0, RG_BN) + 15) / 16;
  const int fn_valid = min(max((nblk - wn + WN - 1) / WN, 0), FN);
  const bool full_n = nblk * 16 >= RG_BN;
  // fp8: the DMA skips 16-row blocks of activation rows wholly past the group
  // end; only skipped fragments would read them, and they are fetched before
  // the weight rows, which the waits count.  Weight blocks past N are fetched
  // (their rows clamped to N - 1), so every wave has four weight fetches per
  // step.  (The bf16 loop's waits count all its fetches; skipping there
  // measured 4-7% slower.)
  if constexpr (KIND == K_FP8) {
#pragma unroll
    for (int q = 0; q < DMA_PER_WAVE; ++q) {
      const int blk = wave + NW * q;
      const bool on = blk < 16 ? blk < mblk : true;
      dma_on |= on ? 1 << q : 0;
    }
  }

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragment reads and MFMAs of one stage, in four quarters: quarter q reads
  // B fragments [q FN/4, (q+1) FN/4) and A fragments 2q, 2q + 1, and does the
  // MFMAs of A rows 2q, 2q + 1 (FMV row fragments in all; the first FNV
  // column fragments, or the first fn_valid when FNV is -1).
  auto load_quarter = [&](int q, const char* buf, i32x4_t (&af)[FM], i32x4_t (&bf)[FN],
                          auto fmv_c, auto full_c) {
    constexpr int FMV = decltype(fmv_c)::value;
    constexpr int FNV = decltype(full_c)::value;
#pragma unroll
    for (int j = q * (FN / QUARTERS); j < (q + 1) * (FN / QUARTERS); ++j)
      if (FNV >= 0 ? j < FNV : j < fn_valid)
        bf[j] = *reinterpret_cast<const i32x4_t*>(buf + RG_ABYTES + (wn + WN * j) * 1024 + lofs);
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i)
      if (i < FMV) af[i] = *reinterpret_cast<const i32x4_t*>(buf + (wm + WM * i) * 1024 + lofs);
  };
  auto mma_quarter = [&](int q, const i32x4_t (&af)[FM], const i32x4_t (&bf)[FN], auto fmv_c,
                         auto full_c) {
    constexpr int FMV = decltype(fmv_c)::value;
    constexpr int FNV = decltype(full_c)::value;
#pragma unroll
    for (int i = 2 * q; i < 2 * q + 2; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (i < FMV && (FNV >= 0 ? j < FNV : j < fn_valid))
          acc[i][j] = mfma_bf16(bf[j], af[i], acc[i][j]);
  };

  // Stage s lives in ring slot s % RING and is fetched RING - 1 stages ahead.
  // Its fragments are read from LDS one stage ahead, during the MFMAs of
  // stage s - 1, so LDS latency hides behind MFMA work.  At the top of step s
  // the wave waits for its DMA of stage s+1 (stages s+2 .. s+RING-2 may still
  // fly) and for its fragment reads of stage s, issued a whole step earlier
  // (so that nothing waits on the reads it issues next); the barrier then
  // makes stage s+1 visible to all waves and ensures slot (s - 1) % RING, read
  // for stage s-1 during step s-2, is free for stage s + RING - 1.  The
  // step's DMA and LDS reads are spread between its MFMAs, a quarter at a
  // time, so that no burst of memory instructions holds up MFMA issue.
  constexpr int WAIT_NEXT = waitcnt_imm((RING - 3) * DMA_PER_WAVE, 0);
  constexpr int WAIT_FIRST = waitcnt_imm((RING - 2) * DMA_PER_WAVE, 15);
  auto slot = [&](int s) { return ring + (s % RING) * RG_STAGE; };
  auto step = [&](int s, const i32x4_t (&ca)[FM], const i32x4_t (&cb)[FN], i32x4_t (&na)[FM],
                  i32x4_t (&nb)[FN], auto fmv_c, auto full_c) {
    __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    block_sync_lds();
    char* dbuf = slot(s + RING - 1);
    const char* nbuf = slot(s + 1);
#pragma unroll
    for (int q = 0; q < QUARTERS; ++q) {
#pragma unroll
      for (int d = q * (DMA_PER_WAVE / QUARTERS); d < (q + 1) * (DMA_PER_WAVE / QUARTERS); ++d)
        dma_one(d, s + RING - 1, dbuf);
      load_quarter(q, nbuf, na, nb, fmv_c, full_c);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the MFMAs
      mma_quarter(q, ca, cb, fmv_c, full_c);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // (the first RING - 1 stages are fetched before the loop instance is
  // chosen, which waits for the group's extent)
  auto k_loop = [&](auto fmv_c, auto full_c) {
    i32x4_t a0[FM], b0[FN], a1[FM], b1[FN];
    __builtin_amdgcn_s_waitcnt(WAIT_FIRST);
    block_sync_lds();
#pragma unroll
    for (int q = 0; q < QUARTERS; ++q) load_quarter(q, ring, a0, b0, fmv_c, full_c);
    for (int s = 0; s < nk; s += 2) {
      step(s, a0, b0, a1, b1, fmv_c, full_c);
      if (s + 1 >= nk) break;
      step(s + 1, a1, b1, a0, b0, fmv_c, full_c);
    }
    // no LDS write may still be in flight when the workgroup ends
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
  };

  // fp8: one MFMA K step (16x16x128) takes 128 bytes of each row, ring
  // stages 2u and 2u + 1; lane group g holds bytes [32 g, 32 g + 32), i.e.
  // chunks 2 (g & 1) and 2 (g & 1) + 1 of stage 2u + (g >> 1).  The
  // activation rows (from L2) of step u sit in slot u % 2 of their own
  // region, fetched one step ahead at the top of the step; the weight rows
  // (from HBM) in slot u % 3 of theirs, fetched two steps ahead halfway
  // through the step's MFMAs.  Each slot holds the step's two
  // stages.  A stage past the end of K (K / 64 odd) is zero-filled in LDS,
  // so the last step adds exact zeros.
  auto k_loop_fp8 = [&](auto fmv_c, auto full_c) {
    constexpr int FMV = decltype(fmv_c)::value;
    constexpr int FNV = decltype(full_c)::value;
    constexpr int HALF = RG_ABYTES;  // one stage of one operand
    char* const a_region = ring;             // 2 slots
    char* const b_region = ring + 4 * HALF;  // 3 slots
    const int c0 = 2 * (lgrp & 1);
    const int o0 = lrow * RG_ROWB + ((c0 ^ rg_swizzle(lrow)) * 16);
    const int o1 = lrow * RG_ROWB + (((c0 + 1) ^ rg_swizzle(lrow)) * 16);
    auto frag = [&](const char* p8) {
      const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(p8 + o0);
      const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(p8 + o1);
      i32x8_t r;
      r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
      r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
      return r;
    };
    // stage s of one operand: this wave's blocks q0 and q0 + 1 (block b of
    // the stage lands at dst + 1 KB b)
    auto fill_half = [&](int s, char* dst, int q0) {
      if (s < nk) {
        dma_one(q0, s, dst);
        dma_one(q0 + 1, s, dst);
      } else {
#pragma unroll
        for (int q = q0; q < q0 + 2; ++q)
          *reinterpret_cast<i32x4_t*>(dst + (wave + NW * q) * 1024 + lane * 16) =
              i32x4_t{0, 0, 0, 0};
      }
    };
    auto fill_a = [&](int u) {
      char* a = a_region + (u & 1) * 2 * HALF;
      fill_half(2 * u, a, 0);
      fill_half(2 * u + 1, a + HALF, 0);
    };
    auto fill_b = [&](int u) {
      char* b = b_region + (u % 3) * 2 * HALF - HALF;  // weight blocks are 16..31
      fill_half(2 * u, b, 2);
      fill_half(2 * u + 1, b + HALF, 2);
    };
    const int nsteps = (nk + 1) / 2;
    // one step: wait, barrier, the activation rows of step u + 1, the
    // fragment reads and first half of the MFMAs, the weight rows of step
    // u + 2, the second half.  The wait is for this wave's fetches of step u
    // (and its reads of step u - 1); the weights of step u + 1, this wave's
    // four youngest fetches, may still fly when `relaxed`.  `fa` and `fb`
    // issue the fetches; a_slot and b_slot are the step's LDS slots.
    auto step = [&](int u, bool relaxed, int a_slot, int b_slot, auto fa, auto fb) {
      if (relaxed)
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(4, 0));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
      block_sync_lds();
      fa(u + 1);
      const char* ca = a_region + a_slot * 2 * HALF + (lgrp >> 1) * HALF;
      const char* cb = b_region + b_slot * 2 * HALF + (lgrp >> 1) * HALF;
      i32x8_t af[FM], bf[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if (FNV >= 0 ? j < FNV : j < fn_valid) bf[j] = frag(cb + (wn + WN * j) * 1024);
#pragma unroll
      for (int i = 0; i < FMV; ++i) af[i] = frag(ca + (wm + WM * i) * 1024);
#pragma unroll
      for (int i = 0; i < FMV / 2; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (FNV >= 0 ? j < FNV : j < fn_valid) acc[i][j] = mfma_fp8(bf[j], af[i], acc[i][j]);
      // the weights of step u + 2 between the two halves of the MFMAs: the
      // fragment reads go first, and the fetches have two steps to land
      __builtin_amdgcn_sched_barrier(0);
      fb(u + 2);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = FMV / 2; i < FMV; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          if (FNV >= 0 ? j < FNV : j < fn_valid) acc[i][j] = mfma_fp8(bf[j], af[i], acc[i][j]);
    };
    fill_a(0);
    fill_b(0);
    if (nsteps > 1) fill_b(1);
    // Main steps: every fetch they issue (stages 2u + 2 .. 2u + 5) lies
    // inside K, so they fetch without tests; the fetch sources advance from
    // uniform bases (addresses of one scalar base and a 32-bit lane offset),
    // and the slots rotate in scalar registers.
    const int u_main = max((nk - 4) / 2, 0);
    int a_slot = 0, b_slot = 0;
    int u = 0;
    for (; u < u_main; ++u) {
      const int a_next = a_slot ^ 1;
      const int b_next2 = b_slot == 0 ? 2 : b_slot - 1;  // (u + 2) % 3
      step(u, true, a_slot, b_slot,
           [&](int v) {
             char* dst = a_region + a_next * 2 * HALF;
             const char* from = a_base + int64_t(2 * v) * RG_ROWB;
#pragma unroll
             for (int h = 0; h < 2; ++h)
#pragma unroll
               for (int q = 0; q < 2; ++q)
                 if (dma_on & (1 << q))
                   __builtin_amdgcn_global_load_lds(from + h * RG_ROWB + a_off[q],
                                                    MOE_LDS_PTR(dst + h * HALF +
                                                                (wave + NW * q) * 1024),
                                                    16, 0, 0);
           },
           [&](int v) {
             char* dst = b_region + b_next2 * 2 * HALF - HALF;  // weight blocks are 16..31
             const char* from = wbase + int64_t(2 * v) * RG_ROWB;
#pragma unroll
             for (int h = 0; h < 2; ++h)
#pragma unroll
               for (int q = 0; q < 2; ++q)
                 __builtin_amdgcn_global_load_lds(from + h * RG_ROWB + w_off[q],
                                                  MOE_LDS_PTR(dst + h * HALF +
                                                              (wave + NW * (q + 2)) * 1024),
                                                  16, 0, 0);
           });
      a_slot = a_next;
      b_slot = b_slot == 2 ? 0 : b_slot + 1;
    }
    // The last steps: fetches past the end of K zero-fill their stage.
    for (; u < nsteps; ++u) {
      step(u, 2 * u + 3 < nk, u & 1, u % 3,
           [&](int v) {
             if (v < nsteps) fill_a(v);
           },
           [&](int v) {
             if (v < nsteps) fill_b(v);
           });
    }
    __builtin_amdgcn_s_waitcnt(WAIT_VM0);
  };

  auto with_rows = [&](auto& loop, auto full_c) {
    using I = int;
    switch (fm_valid) {
      case 8: loop(std::integral_constant<I, 8>{}, full_c); break;
      case 7: loop(std::integral_constant<I, 7>{}, full_c); break;
      case 6: loop(std::integral_constant<I, 6>{}, full_c); break;
      case 5: loop(std::integral_constant<I, 5>{}, full_c); break;
      case 4: loop(std::integral_constant<I, 4>{}, full_c); break;
      case 3: loop(std::integral_constant<I, 3>{}, full_c); break;
      case 2: loop(std::integral_constant<I, 2>{}, full_c); break;
      case 1: loop(std::integral_constant<I, 1>{}, full_c); break;
      default: loop(std::integral_constant<I, 0>{}, full_c); break;
    }
  };
  // The loop instance also fixes the wave's count of valid column fragments
  // when it is FN, 2 or 1 (the last N tile of N = 1856, 2688 or 3712 leaves
  // each wave one or two); other counts test it at run time.
  auto run = [&](auto& loop) {
    using I = int;
    if (full_n || fn_valid == FN)
      with_rows(loop, std::integral_constant<I, FN>{});
    else if (fn_valid == 2)
      with_rows(loop, std::integral_constant<I, 2>{});
    else if (fn_valid == 1)
      with_rows(loop, std::integral_constant<I, 1>{});
    else
      with_rows(loop, std::integral_constant<I, -1>{});
  };
  if constexpr (KIND == K_FP8) {
    run(k_loop_fp8);
    __syncthreads();  // every wave is past its last fragment read
    sc_row[threadIdx.x] = my_scale;
    __syncthreads();
  } else {
#pragma unroll
    for (int s = 0; s < RING - 1; ++s) dma(s, ring + s * RG_STAGE);
    run(k_loop);
  }

  // Epilogue: the same arithmetic as store_block, fp8 scales from LDS.  The
  // MFMAs take the weight fragment as their first operand, so a lane holds
  // the transposed block: one row and four consecutive columns, written
  // with one 8-byte (bf16) or 16-byte (fp32) store.  Each row fragment
  // computes one address; a wave's column blocks are 16 WN columns apart,
  // constant offsets from it.  N is a multiple of 16, so whether a column
  // block lies inside N is the same for every lane of the wave.
  const int nvalid = min(p.n - t.n0, RG_BN);
  const int c0 = wn * 16 + lgrp * 4;  // tile-local first column of block j = 0
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int rl = (wm + WM * i) * 16 + lrow;  // tile-local row
    const int64_t r = t.m0 + rl;
    if (r >= t.gend) continue;
    const float sa = KIND == K_FP8 ? sc_row[rl] : 1.0f;
    const int64_t e0 = r * p.n + t.n0 + c0;  // output element of block j = 0
    uint16_t* const row16 = static_cast<uint16_t*>(p.out) + e0;
    float* const row32 = static_cast<float*>(p.out) + e0;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      if ((wn + WN * j) * 16 >= nvalid) continue;
      const int cl = c0 + WN * 16 * j;
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = acc[i][j][q];
        if (KIND == K_FP8) v[q] = (v[q] * sa) * sc_col[cl + q];
        if (EPI == EPI_RELU2) {
          v[q] = fmaxf(v[q], 0.0f);
          v[q] = v[q] * v[q];
        }
      }
      if (p.out_bf16) {
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(row16 + WN * 16 * j) = w;
      } else {
        *reinterpret_cast<f32x4_t*>(row32 + WN * 16 * j) = f32x4_t{v[0], v[1], v[2], v[3]};
      }
    }
  }
}

template <int KIND, int EPI, int NW, int RING>
__global__ __launch_bounds__(NW * WAVE) void gemm_ring_kernel(GemmArgs pa) {
  __shared__ __attribute__((aligned(1024))) char ring[ring_bytes<KIND, NW, RING>()];
  Tile t;
  const int bid = xcd_tile_order(blockIdx.x, gridDim.x, 32);
  if (!locate_tile<RG_BM, RG_BN>(pa, t, bid)) return;
  ring_tile<KIND, EPI, NW, RING>(t, ring);
}

// fp8 routed experts (prob[0]) and a bf16 shared expert (prob[1]) in one
// launch: each workgroup runs its tile's kind, so the shared expert's tiles
// fill the routed ones' last rounds instead of forming a launch of their own.
// The tiles give the bits of the single-kind kernels.
template <int EPI>
__global__ __launch_bounds__(8 * WAVE) void gemm_ring_mixed_kernel(GemmArgs pa) {
  constexpr int BYTES = ring_bytes<K_FP8, 8, 4>() > ring_bytes<K_BF16, 8, 4>()
                            ? ring_bytes<K_FP8, 8, 4>()
                            : ring_bytes<K_BF16, 8, 4>();
  __shared__ __attribute__((aligned(1024))) char ring[BYTES];
  Tile t;
  const int bid = xcd_tile_order(blockIdx.x, gridDim.x, 32);
  if (!locate_tile<RG_BM, RG_BN>(pa, t, bid)) return;
  if (t.p.w_scale)  // the fp8 experts carry per-row weight scales
    ring_tile<K_FP8, EPI, 8, 4>(t, ring);
  else
    ring_tile<K_BF16, EPI, 8, 4>(t, ring);
}

// ---------------------------------------------------------- stream kernel
//
// Thin tiles (16, 32 or 64 rows) of bf16 GEMMs that stream their operands:
// the router's logits, where the gate matrix is small and every tile reads
// all of it.  There is little MFMA work per byte, so what matters is how many bytes
// each CU keeps in flight: K moves in 64-byte row slices (the ring kernel's
// swizzled 1 KB block layout) through a ring of SK_RING LDS stages filled by
// global_load_lds_dwordx4 SK_RING - 1 stages ahead, with no staging
// registers.  A stage is FM activation blocks and BN / 16 weight blocks (9 KB
// for 16 x 128 tiles, 12 KB for 64 x 128).  Wider tiles re-read the weights
// from L2 less often.  Same MFMA and per-lane K bytes as gemm_kernel, so the
// same results whatever the tile.
constexpr int SK_RING = 8;

template <int KIND, int FM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_stream_kernel(GemmArgs pa) {
  static_assert(KIND == K_BF16, "the stream kernel takes bf16 operands");
  constexpr int BM = 16 * FM;
  constexpr int NBLK = FM + BN / 16;         // 1 KB blocks per stage: A, then B
  constexpr int STAGE = NBLK * 1024;
  constexpr int FN = BN / 64;                // column fragments per wave (4 waves along N)
  constexpr int MAXQ = (NBLK + 3) / 4;       // blocks one wave fetches per stage, at most
  static_assert(MAXQ <= 3, "the waits below count at most three fetches per stage");
  __shared__ __attribute__((aligned(1024))) char ring[SK_RING * STAGE];

  Tile t;
  if (!locate_tile<BM, BN>(pa, t, blockIdx.x)) return;
  const GemmProblem& p = t.p;
  const int wave = threadIdx.x / WAVE;
  const int lane = lane_id();
  const int64_t kbytes = int64_t(p.k) * 2;
  const int nk = static_cast<int>(kbytes / RG_ROWB);  // the host guarantees K bytes % 64 == 0

  // wave w fetches blocks w, w + 4, w + 8 (< NBLK); rows past the group end
  // or past N re-read the last valid row (their outputs are never stored)
  const int r_in = lane >> 2;
  const int chunk = (lane & 3) ^ rg_swizzle(r_in);
  const char* wbase = static_cast<const char*>(p.w) + int64_t(t.g) * p.n * kbytes;
  const char* src[MAXQ];
#pragma unroll
  for (int q = 0; q < MAXQ; ++q) {
    const int blk = min(wave + 4 * q, NBLK - 1);
    if (blk < FM) {
      const int64_t r = min<int64_t>(t.m0 + blk * 16 + r_in, t.gend - 1);
      src[q] = static_cast<const char*>(p.a) + src_row(p, r) * kbytes + chunk * 16;
    } else {
      const int n = min(t.n0 + (blk - FM) * 16 + r_in, p.n - 1);
      src[q] = wbase + int64_t(n) * kbytes + chunk * 16;
    }
  }
  const int mine = (NBLK - wave + 3) / 4;  // blocks this wave fetches per stage
  auto dma = [&](int s, char* buf) {
    const int64_t kb = int64_t(min(s, nk - 1)) * RG_ROWB;  // past the end: harmless re-read
#pragma unroll
    for (int q = 0; q < MAXQ; ++q) {
      if (q < mine) {
        const void* from = src[q] + kb;
        __builtin_amdgcn_global_load_lds(from, MOE_LDS_PTR(buf + (wave + 4 * q) * 1024), 16, 0,
                                         0);
      }
    }
  };
  // wait until this wave's DMA of the oldest stage in flight has landed, the
  // SK_RING - 2 younger stages may still fly; and its LDS reads are done
  auto wait_oldest = [&]() {
    if (mine >= 3)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm((SK_RING - 2) * 3, 0));
    else if (mine == 2)
      __builtin_amdgcn_s_waitcnt(waitcnt_imm((SK_RING - 2) * 2, 0));
    else
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(SK_RING - 2, 0));
  };

  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int lofs = lrow * RG_ROWB + ((lgrp ^ rg_swizzle(lrow)) * 16);
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < SK_RING - 1; ++s) dma(s, ring + s * STAGE);
  for (int s = 0; s < nk; ++s) {
    wait_oldest();
    block_sync_lds();  // stage s is in LDS for all waves; slot (s - 1) % SK_RING is free
    dma(s + SK_RING - 1, ring + ((s + SK_RING - 1) % SK_RING) * STAGE);
    const char* buf = ring + (s % SK_RING) * STAGE;
    i32x4_t af[FM], bf[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const i32x4_t*>(buf + i * 1024 + lofs);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      bf[j] = *reinterpret_cast<const i32x4_t*>(buf + (FM + wave * FN + j) * 1024 + lofs);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma_bf16(af[i], bf[j], acc[i][j]);
  }
  // no LDS write may still be in flight when the workgroup ends
  __builtin_amdgcn_s_waitcnt(WAIT_VM0);

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      store_block<KIND, EPI>(t, acc[i][j], t.m0 + 16 * i + lgrp * 4,
                             t.n0 + (wave * FN + j) * 16 + lrow);
}

// ------------------------------------------------------------ fp4 kernel
//
// MXFP4 weights (an e2m1 code times the E8M0 power of two of its 32-element
// block) with bf16 activations.  Codes are widened where an MFMA fragment is
// built, by v_cvt_scalef32_pk_bf16_fp4, which applies the block's power of
// two; an e2m1 value times a power of two is a bf16 value, so the bf16 MFMA
// sees the dequantised weight exactly.
//
// A workgroup of four waves owns a (16 FM) x 64 output tile; each wave owns
// 16 weight rows and all FM 16-row fragments of the activations.  K streams
// through LDS in 256-element stages, double buffered, with the loads of the
// next D stages in registers.  Every load is a buffer load issued
// unconditionally: what lies past K, past the group's rows or past the last
// stage is out of the buffer's range and reads as zero without touching
// memory, so the number of loads in flight is the same on every path and the
// waits are exact.  A stage row of codes is 128 bytes, one whole cache line,
// read by 8 consecutive lanes; the activation stage (16 FM rows of 512
// bytes) is shared by the four waves.
//
// Element order inside a stage: in super-block h (128 elements, h = 0, 1)
// lane group g (lanes 16 g .. 16 g + 15) owns scale block 4 h + g, and MFMA
// step s (0..3) gives every lane elements 8 s .. 8 s + 7 of its own block, of
// the activation row and of the weight row alike; the four steps cover the
// super-block once.  A lane's codes for a super-block are one 16-byte LDS
// read and one scale.  Each output element is one MFMA chain over the
// super-blocks and steps in ascending order whatever FM is, so the tile
// shape does not change results.  The tile's block scales (64 rows x K/32
// bytes, contiguous) sit in dynamic LDS sized to K.
constexpr int F4_BN = 64;
constexpr int F4_KE = 256;         // K elements per stage
constexpr int F4_WROW = 128 + 16;  // LDS bytes per weight row (padded)
constexpr int F4_AROW = 512 + 16;  // LDS bytes per activation row (padded)
constexpr uint32_t F4_OOB = 0x80000000u;  // a buffer offset past every range here

__device__ __forceinline__ i32x4_t fp4x8_to_bf16(uint32_t codes, float scale) {
  i32x4_t r;
  r[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0));
  r[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1));
  r[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2));
  r[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3));
  return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t f4_rsrc(const void* base, uint32_t bytes) {
  // raw buffer, no swizzle; offsets at or past `bytes` read as zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int EPI, int D, int FM>
__global__ __launch_bounds__(256) void gemm_fp4_kernel(GemmArgs pa) {
  constexpr int BM = 16 * FM, BN = F4_BN;
  constexpr int AQ = 2 * FM;  // activation chunks per thread and stage
  constexpr int WSZ = BN * F4_WROW;
  constexpr int STAGE = WSZ + BM * F4_AROW;
  constexpr int SC_PT = F4_SCALE_LDS / 16 / 256;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  extern __shared__ __attribute__((aligned(16))) uint8_t scl[];

  Tile t;
  if (!locate_tile<BM, BN>(pa, t, blockIdx.x)) return;
  const GemmProblem& p = t.p;
  const int tid = threadIdx.x;
  const int wave = tid / WAVE;
  const int lane = lane_id();
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const int nblk = p.k / 32;  // the host guarantees K % 64 == 0
  const uint32_t wbytes = p.k / 2;
  const uint32_t abytes = p.k * 2;
  const int nst = (p.k + F4_KE - 1) / F4_KE;

  // weights and scales of the tile (N % 64 == 0: the tile is whole)
  const int sc_bytes = BN * nblk;
  const int64_t row0 = int64_t(t.g) * p.n + t.n0;
  const __amdgpu_buffer_rsrc_t wr = f4_rsrc(static_cast<const char*>(p.w) + row0 * wbytes,
                                            BN * wbytes);
  const __amdgpu_buffer_rsrc_t sr = f4_rsrc(p.w_bscale + row0 * nblk, sc_bytes);
  i32x4_t scv[SC_PT];
#pragma unroll
  for (int q = 0; q < SC_PT; ++q)
    scv[q] = __builtin_amdgcn_raw_buffer_load_b128(sr, (tid + q * 256) * 16, 0, 0);

  // this thread's chunks: weight rows tid / 8 + 32 q at byte (tid % 8) * 16
  // of the stage; activation rows tid / 32 + 8 q at byte (tid % 32) * 16
  const uint32_t wc = (tid % 8) * 16;
  const uint32_t ac = (tid % 32) * 16;
  uint32_t wbase[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) wbase[q] = (tid / 8 + 32 * q) * wbytes;
  struct Regs {
    i32x4_t w[2], a[AQ];
  };
  Regs R[D];
  auto gload_w = [&](int st, Regs& r) {
    const uint32_t k = st * 128 + wc;  // past K or past the last stage: zero
#pragma unroll
    for (int q = 0; q < 2; ++q)
      r.w[q] = __builtin_amdgcn_raw_buffer_load_b128(wr, k < wbytes ? wbase[q] + k : F4_OOB, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) gload_w(d, R[d]);  // the weights do not wait for the rows

  // (the host keeps a_rows * K * 2 below 2^31 for fp4 weights)
  const int64_t a_all = p.a_rows * int64_t(abytes);
  const uint32_t a_range = __builtin_amdgcn_readfirstlane(
      static_cast<int>(a_all > 0x7fffffff ? 0x7fffffff : a_all));
  const __amdgpu_buffer_rsrc_t ar = f4_rsrc(p.a, a_range);
  // row starts of this thread's activation rows; past the group end the
  // start is F4_OOB, so every offset from it is out of range too
  uint32_t abase[AQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int64_t r = t.m0 + tid / 32 + 8 * q;
    abase[q] = r < t.gend ? static_cast<uint32_t>(src_row(p, r) * abytes) : F4_OOB;
  }
  auto gload_a = [&](int st, Regs& r) {
    const uint32_t k = st * 512 + ac;  // past K or past the last stage: zero
#pragma unroll
    for (int q = 0; q < AQ; ++q)
      r.a[q] = __builtin_amdgcn_raw_buffer_load_b128(ar, k < abytes ? abase[q] + k : F4_OOB, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) gload_a(d, R[d]);
  auto sstore = [&](int buf, const Regs& r) {
    char* ws = smem + buf * STAGE;
    char* as = ws + WSZ;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<i32x4_t*>(ws + (tid / 8 + 32 * q) * F4_WROW + wc) = r.w[q];
#pragma unroll
    for (int q = 0; q < AQ; ++q)
      *reinterpret_cast<i32x4_t*>(as + (tid / 32 + 8 * q) * F4_AROW + ac) = r.a[q];
  };
#pragma unroll
  for (int q = 0; q < SC_PT; ++q) {
    const int off = (tid + q * 256) * 16;
    if (off < sc_bytes) *reinterpret_cast<i32x4_t*>(scl + off) = scv[q];
  }
  sstore(0, R[0]);
  __syncthreads();

  f32x4_t acc[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint8_t* my_scl = scl + (16 * wave + lrow) * nblk;
  for (int st0 = 0; st0 < nst; st0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int st = st0 + d;
      if (st >= nst) break;
      // R[d] held stage st (stored last step); it now takes stage st + D
      gload_w(st + D, R[d]);
      gload_a(st + D, R[d]);
      const char* ws = smem + (st & 1) * STAGE + (16 * wave + lrow) * F4_WROW + 16 * lgrp;
      const char* as = smem + (st & 1) * STAGE + WSZ + lrow * F4_AROW + 64 * lgrp;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int blk = 8 * st + 4 * h + lgrp;
        const uint32_t c = my_scl[min(blk, nblk - 1)];
        const uint32_t code = blk < nblk ? c : 0u;        // past K: zero codes anyway
        const float scale = __uint_as_float(code << 23);  // 2^(code - 127)
        const i32x4_t w = *reinterpret_cast<const i32x4_t*>(ws + 64 * h);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const i32x4_t b = fp4x8_to_bf16(static_cast<uint32_t>(w[s]), scale);
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const i32x4_t a =
                *reinterpret_cast<const i32x4_t*>(as + 16 * i * F4_AROW + 256 * h + 16 * s);
            acc[i] = mfma_bf16(a, b, acc[i]);
          }
        }
      }
      if (st + 1 < nst) sstore((st + 1) & 1, R[(d + 1) % D]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i)
    store_block<K_BF16, EPI>(t, acc[i], t.m0 + 16 * i + 4 * lgrp, t.n0 + 16 * wave + lrow);
}

template <int EPI>
hipError_t launch_fp4(const GemmArgs& p, GemmShape shape, unsigned grid, hipStream_t stream,
                      Timing t) {
  // dynamic LDS: the block scales of a tile, for the larger K of the problems
  const int kmax = std::max(p.prob[0].k, p.prob[1].w ? p.prob[1].k : 0);
  const unsigned shm = static_cast<unsigned>((F4_BN * (kmax / 32) + 15) / 16 * 16);
  const dim3 g(grid), b(256);
  if (shape.bn != F4_BN) return hipErrorInvalidValue;
  // decode tiles: two stages in flight; 64-row tiles: one (registers)
  if (shape.bm == 16) return launch_k_shm(gemm_fp4_kernel<EPI, 2, 1>, g, b, shm, stream, t, p);
  if (shape.bm == 64) return launch_k_shm(gemm_fp4_kernel<EPI, 1, 4>, g, b, shm, stream, t, p);
  return hipErrorInvalidValue;
}

// --------------------------------------------------------- bf16 decode kernel
//
// Decode tiles (16 rows) of bf16 weights, where the launch is a weight
// stream: gemm_kernel's layout (four waves split N, K through LDS in
// KB-byte row stages, double buffered) with the loads issued as buffer loads
// on every path, out-of-range ones (past K, past N, past the group's rows,
// past the last stage) reading zero without touching memory.  The number of
// loads in flight is then the same everywhere, the waits are exact, and D
// stages of loads stay in flight.  Each output element is the same MFMA
// chain over K, in ascending 32-element steps from zero, as in gemm_kernel,
// so results do not depend on which kernel computes a tile.
template <int EPI, int BN, int D, int KB>
__global__ __launch_bounds__(256) void gemm_dec_kernel(GemmArgs pa) {
  constexpr int BM = 16;
  constexpr int ROW = KB + 16;                 // padded LDS row
  constexpr int CPR = KB / 16;                 // 16-byte chunks per row and stage
  constexpr int WQ = BN * CPR / 256;           // weight chunks per thread
  constexpr int AQ = (BM * CPR + 255) / 256;   // activation chunks per thread
  constexpr int FN = BN / 64;                  // 16-column fragments per wave
  constexpr int WSZ = BN * ROW;
  constexpr int STAGE = WSZ + BM * ROW;
  static_assert(WQ * 256 == BN * CPR, "weight chunks split evenly");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  Tile t;
  if (!locate_tile<BM, BN>(pa, t, blockIdx.x)) return;
  const GemmProblem& p = t.p;
  const int tid = threadIdx.x;
  const int wave = tid / WAVE;
  const int lane = lane_id();
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  const uint32_t kbytes = uint32_t(p.k) * 2;
  const int nst = static_cast<int>((kbytes + KB - 1) / KB);

  // rows of the tile past N lie past the weight buffer's range
  const int nrows = min(BN, p.n - t.n0);
  const __amdgpu_buffer_rsrc_t wr =
      f4_rsrc(static_cast<const char*>(p.w) + (int64_t(t.g) * p.n + t.n0) * kbytes,
              uint32_t(nrows) * kbytes);
  uint32_t wbase[WQ], wcol[WQ];
#pragma unroll
  for (int q = 0; q < WQ; ++q) {
    const int c = tid + 256 * q;
    wbase[q] = uint32_t(c / CPR) * kbytes;
    wcol[q] = (c % CPR) * 16;
  }
  struct Regs {
    i32x4_t w[WQ], a[AQ];
  };
  Regs R[D];
  auto gload_w = [&](int st, Regs& r) {
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const uint32_t k = st * KB + wcol[q];  // past K or past the last stage: zero
      r.w[q] = __builtin_amdgcn_raw_buffer_load_b128(wr, k < kbytes ? wbase[q] + k : F4_OOB, 0, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) gload_w(d, R[d]);  // the weights do not wait for the rows

  // (the launcher keeps a_rows * K * 2 below 2^31 for this kernel)
  const int64_t a_all = p.a_rows * int64_t(kbytes);
  const uint32_t a_range = __builtin_amdgcn_readfirstlane(
      static_cast<int>(a_all > 0x7fffffff ? 0x7fffffff : a_all));
  const __amdgpu_buffer_rsrc_t ar = f4_rsrc(p.a, a_range);
  uint32_t abase[AQ], acol[AQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int c = tid + 256 * q;
    const int64_t r = t.m0 + c / CPR;
    acol[q] = (c % CPR) * 16;
    abase[q] = (c < BM * CPR && r < t.gend) ? static_cast<uint32_t>(src_row(p, r) * kbytes)
                                              : F4_OOB;
  }
  auto gload_a = [&](int st, Regs& r) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const uint32_t k = st * KB + acol[q];
      r.a[q] = __builtin_amdgcn_raw_buffer_load_b128(ar, k < kbytes ? abase[q] + k : F4_OOB, 0, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) gload_a(d, R[d]);
  auto sstore = [&](int buf, const Regs& r) {
    char* ws = smem + buf * STAGE;
    char* as = ws + WSZ;
#pragma unroll
    for (int q = 0; q < WQ; ++q) {
      const int c = tid + 256 * q;
      *reinterpret_cast<i32x4_t*>(ws + (c / CPR) * ROW + wcol[q]) = r.w[q];
    }
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const int c = tid + 256 * q;
      if (c < BM * CPR) *reinterpret_cast<i32x4_t*>(as + (c / CPR) * ROW + acol[q]) = r.a[q];
    }
  };
  sstore(0, R[0]);
  __syncthreads();

  f32x4_t acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int st0 = 0; st0 < nst; st0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int st = st0 + d;
      if (st >= nst) break;
      // R[d] held stage st (stored last step); it now takes stage st + D
      gload_w(st + D, R[d]);
      gload_a(st + D, R[d]);
      const char* buf = smem + (st & 1) * STAGE;
      const char* as = buf + WSZ + lrow * ROW + 16 * lgrp;
      const char* ws = buf + (wave * (BN / 4) + lrow) * ROW + 16 * lgrp;
#pragma unroll
      for (int ks = 0; ks < KB / 64; ++ks) {
        if (st * KB + 64 * ks >= int(kbytes)) break;  // no steps past K
        const i32x4_t a = *reinterpret_cast<const i32x4_t*>(as + 64 * ks);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const i32x4_t b = *reinterpret_cast<const i32x4_t*>(ws + 16 * j * ROW + 64 * ks);
          acc[j] = mfma_bf16(a, b, acc[j]);
        }
      }
      if (st + 1 < nst) sstore((st + 1) & 1, R[(d + 1) % D]);
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < FN; ++j)
    store_block<K_BF16, EPI>(t, acc[j], t.m0 + 4 * lgrp, t.n0 + wave * (BN / 4) + 16 * j + lrow);
}

// One wave per row: amax, scale = amax / 448 (0 -> 1), e4m3 codes of v / scale
// (the division correctly rounded, as the compiler emits it without fast-math
// flags).  v / scale is clamped to +-448 (it exceeds 448 by more than an ulp
// only when the scale is an fp32 subnormal), then v_cvt_pk_fp8_f32 rounds it
// to nearest even into OCP e4m3fn (gfx950's fp8 format); a code that rounds
// to zero is written as +0 (the instruction keeps the sign).  Rows up to
// QV_MAX * 256 columns are read once into registers (all loads in flight
// together); longer rows are read twice.
constexpr int QV_MAX = 12;
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs p) {
  const int64_t row = int64_t(blockIdx.x) * 4 + threadIdx.x / WAVE;
  if (row >= p.rows) return;
  const int lane = lane_id();
  const int cols = p.cols;
  auto ld4 = [&](int c, float* v) {
    if (p.in_bf16) {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      const u32x2_t u = __builtin_nontemporal_load(
          reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(p.in) + row * cols + c));
      v[0] = __uint_as_float(u.x << 16);
      v[1] = __uint_as_float(u.x & 0xFFFF0000u);
      v[2] = __uint_as_float(u.y << 16);
      v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      const f32x4_t f = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p.in) + row * cols + c));
      v[0] = f[0];
      v[1] = f[1];
      v[2] = f[2];
      v[3] = f[3];
    }
  };
  auto quant4 = [&](const float* v, float s) {
    float r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = __builtin_amdgcn_fmed3f(v[q] / s, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], w, true);
    // bit 7 of each byte of m: the byte's magnitude bits are not all zero
    const uint32_t u = static_cast<uint32_t>(w);
    const uint32_t m = (u & 0x7F7F7F7Fu) + 0x7F7F7F7Fu;
    return u & (0x7F7F7F7Fu | (m & 0x80808080u));
  };
  auto row_scale = [&](float amax) {
#pragma unroll
    for (int off = WAVE / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float s = amax / 448.0f;
    return s == 0.0f ? 1.0f : s;
  };
  float s;
  if (cols <= QV_MAX * WAVE * 4) {
    float v[QV_MAX][4];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < QV_MAX; ++i) {
      const int c = (i * WAVE + lane) * 4;
      if (c < cols) ld4(c, v[i]);
    }
#pragma unroll
    for (int i = 0; i < QV_MAX; ++i) {
      const int c = (i * WAVE + lane) * 4;
      if (c < cols)
#pragma unroll
        for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fabsf(v[i][q]));
    }
    s = row_scale(amax);
#pragma unroll
    for (int i = 0; i < QV_MAX; ++i) {
      const int c = (i * WAVE + lane) * 4;
      if (c < cols) *reinterpret_cast<uint32_t*>(p.q + row * cols + c) = quant4(v[i], s);
    }
  } else {
    float amax = 0.0f;
    for (int c = lane * 4; c < cols; c += WAVE * 4) {
      float v[4];
      ld4(c, v);
#pragma unroll
      for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fabsf(v[q]));
    }
    s = row_scale(amax);
    for (int c = lane * 4; c < cols; c += WAVE * 4) {
      float v[4];
      ld4(c, v);
      *reinterpret_cast<uint32_t*>(p.q + row * cols + c) = quant4(v, s);
    }
  }
  if (lane == 0) p.scale[row] = s;
}

template <int KIND, int EPI>
hipError_t launch_kind_epi(const GemmArgs& p, GemmShape shape, unsigned grid, hipStream_t stream,
                           Timing t) {
  const dim3 g(grid);
  if constexpr (KIND == K_BF16) {
    if (shape.stream && shape.bn == 128) {
      if (shape.bm == 16)
        return launch_k(gemm_stream_kernel<KIND, 1, 128, EPI>, g, dim3(256), stream, t, p);
      if (shape.bm == 32)
        return launch_k(gemm_stream_kernel<KIND, 2, 128, EPI>, g, dim3(256), stream, t, p);
      if (shape.bm == 64)
        return launch_k(gemm_stream_kernel<KIND, 4, 128, EPI>, g, dim3(256), stream, t, p);
    }
  }
  if constexpr (KIND == K_BF16) {
    // decode tiles; its buffer offsets are 32-bit, else gemm_kernel below
    const bool fits = p.prob[0].a_rows * int64_t(p.prob[0].k) * 2 <= 0x7fffffff &&
                      p.prob[1].a_rows * int64_t(p.prob[1].k) * 2 <= 0x7fffffff;
    // two stages of 256-byte rows in flight
    if (shape.bm == 16 && shape.bn == 64 && fits)
      return launch_k(gemm_dec_kernel<EPI, 64, 2, 256>, g, dim3(256), stream, t, p);
  }
  if (shape.bm == 16 && shape.bn == 64)
    return launch_k(gemm_kernel<KIND, 16, 64, 1, 4, EPI, 256, 0>, g, dim3(256), stream, t, p);
  if (shape.bm == 64)
    return launch_k(gemm_kernel<KIND, 64, 128, 2, 2, EPI, 256, 0>, g, dim3(256), stream, t, p);
  if constexpr (KIND == K_BF16) {
    if (shape.bm == RG_BM)
      return launch_k(gemm_ring_kernel<KIND, EPI, 8, 4>, g, dim3(8 * WAVE), stream, t, p);
  }
  if constexpr (KIND == K_FP8) {
    // (the ring kernel addresses fp8 rows by 32-bit offsets)
    auto fits = [](const GemmProblem& q) {
      return !q.w || (q.a_rows * q.k < (int64_t(1) << 32) && int64_t(q.n) * q.k < (int64_t(1) << 32));
    };
    const bool ring = shape.bm == RG_BM && fits(p.prob[0]) && fits(p.prob[1]);
    if (p.prob[1].w && !p.prob[1].w_scale) {  // a bf16 second problem: the mixed ring kernel only
      if (!ring) return hipErrorInvalidValue;
      return launch_k(gemm_ring_mixed_kernel<EPI>, g, dim3(8 * WAVE), stream, t, p);
    }
    if (ring) return launch_k(gemm_ring_kernel<KIND, EPI, 8, 4>, g, dim3(8 * WAVE), stream, t, p);
  }
  // two workgroups per CU: 64 tiles per XCD in flight
  return launch_k(gemm_kernel<KIND, 128, 128, 2, 2, EPI, 256, 64>, g, dim3(256), stream, t, p);
}

template <int KIND>
hipError_t launch_kind(const GemmArgs& p, int epi, GemmShape shape, unsigned grid,
                       hipStream_t stream, Timing t) {
  return epi == EPI_RELU2 ? launch_kind_epi<KIND, EPI_RELU2>(p, shape, grid, stream, t)
                          : launch_kind_epi<KIND, EPI_PLAIN>(p, shape, grid, stream, t);
}

}  // namespace

GemmShape pick_gemm_shape(int kind, int64_t rows, int groups) {
  const int64_t avg = groups > 0 ? rows / groups : rows;
  // 4-bit weights: a weight stream for decode; wider M tiles re-read it less
  if (kind == K_FP4) return GemmShape{avg <= 24 ? 16 : 64, 64};
  // decode: a weight stream, in 16 x 64 tiles (more tiles in flight than
  // 128-wide ones)
  if (avg <= 24) return GemmShape{16, 64};
  if (avg <= 80) return GemmShape{64, 128};
  if (avg < 128 || kind == K_F32) return GemmShape{128, 128};
  return GemmShape{256, 256};
}

int64_t max_mtiles(int64_t rows, int groups, int bm) {
  const int64_t bound = (rows + int64_t(groups) * (bm - 1)) / bm;
  return rows < bound ? rows : bound;
}

hipError_t launch_gemm(const GemmArgs& p, int kind, int epi, GemmShape shape, int64_t mtiles_first,
                       int64_t mtiles_second, hipStream_t stream, Timing t) {
  const int64_t grid64 = mtiles_first * p.n_tiles + mtiles_second * p.n_tiles2;
  if (grid64 <= 0) return hipSuccess;
  if (grid64 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const unsigned grid = static_cast<unsigned>(grid64);
  if (kind == K_FP4)
    return epi == EPI_RELU2 ? launch_fp4<EPI_RELU2>(p, shape, grid, stream, t)
                            : launch_fp4<EPI_PLAIN>(p, shape, grid, stream, t);
  if (kind == K_FP8) return launch_kind<K_FP8>(p, epi, shape, grid, stream, t);
  if (kind == K_BF16) return launch_kind<K_BF16>(p, epi, shape, grid, stream, t);
  return launch_kind<K_F32>(p, epi, shape, grid, stream, t);
}

hipError_t launch_quant(const QuantArgs& p, hipStream_t stream, Timing t) {
  if (p.rows <= 0) return hipSuccess;
  const int64_t blocks = (p.rows + 3) / 4;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  return launch_k(quant_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), stream, t, p);
}

}  // namespace moe
