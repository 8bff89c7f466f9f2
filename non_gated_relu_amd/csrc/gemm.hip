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
// per-expert counts.  K is streamed in 128-byte stages through a double
// buffer in LDS (rows padded to 144 bytes against bank conflicts): the next
// stage's global loads are issued before the current stage's MFMAs.  A rows
// are gathered through the routing permutation while loading, so the permuted
// activations never exist in memory.
#include "internal.hpp"

namespace moe {

namespace {

constexpr int G_THREADS = 256;
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

template <int KIND>
__device__ __forceinline__ typename Frag<KIND>::T lds_frag(const char* p) {
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

template <int KIND, int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(G_THREADS) void gemm_kernel(GemmArgs p) {
  constexpr int ESZ = KindTraits<KIND>::ESZ;
  constexpr int STEP = KindTraits<KIND>::STEP;
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  static_assert(WM * WN == 4, "four waves");
  static_assert(FM >= 1 && FN >= 1, "tile too small for the wave grid");
  constexpr int CPR = BKB / 16;  // 16-byte chunks per row and stage
  constexpr int A_CHUNKS = BM * CPR;
  constexpr int B_CHUNKS = BN * CPR;
  constexpr int CA = (A_CHUNKS + G_THREADS - 1) / G_THREADS;
  constexpr int CB = (B_CHUNKS + G_THREADS - 1) / G_THREADS;
  constexpr int RPT = G_THREADS / CPR;  // rows covered per pass of the block
  constexpr int STAGE = (BM + BN) * LDS_STRIDE;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int n_mt = p.sched[0];
  const int mt = blockIdx.x / p.n_tiles;
  const int nt = blockIdx.x - mt * p.n_tiles;
  if (mt >= n_mt) return;
  const int g = p.sched[2 + 2 * mt];
  const int64_t m0 = p.sched[3 + 2 * mt];
  // no offsets: a single group spans every row
  const int64_t gend =
      p.offsets ? min<int64_t>(max<int64_t>(p.offsets[g + 1], 0), p.rows) : p.rows;
  const int n0 = nt * BN;
  if (n0 >= p.n) return;
  const int64_t kbytes = int64_t(p.k) * ESZ;
  const char* wbase = static_cast<const char*>(p.w) + int64_t(g) * p.n * kbytes;
  const int c16 = (tid % CPR) * 16;  // this thread's byte column inside a stage

  // source row of each chunk this thread loads (null = zero fill)
  const char* a_src[CA];
  const char* b_src[CB];
#pragma unroll
  for (int j = 0; j < CA; ++j) {
    const int row = tid / CPR + j * RPT;
    const int64_t r = m0 + row;
    a_src[j] = nullptr;
    if (row < BM && r < gend) {
      int64_t src = p.row_index ? int64_t(p.row_index[r]) / p.index_div : r;
      src = min<int64_t>(max<int64_t>(src, 0), p.a_rows - 1);
      a_src[j] = static_cast<const char*>(p.a) + src * kbytes + c16;
    }
  }
#pragma unroll
  for (int j = 0; j < CB; ++j) {
    const int row = tid / CPR + j * RPT;
    const int n = n0 + row;
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
      for (int i = 0; i < FM; ++i) af[i] = lds_frag<KIND>(As + i * 16 * LDS_STRIDE + ks * STEP);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = lds_frag<KIND>(Bs + j * 16 * LDS_STRIDE + ks * STEP);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mma<KIND>(af[i], bfr[j], acc[i][j]);
    }
    if (it + 1 < nk) sstore((it + 1) & 1);
    __syncthreads();
  }

  // epilogue: lane holds column lrow of each 16x16 block, rows 4*lgrp .. +3
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = m0 + wm * (BM / WM) + i * 16 + lgrp * 4 + q;
      if (r >= gend) continue;
      float sa = 1.0f;
      if (KIND == K_FP8) {
        int64_t src = p.row_index ? int64_t(p.row_index[r]) / p.index_div : r;
        src = min<int64_t>(max<int64_t>(src, 0), p.a_rows - 1);
        sa = p.a_scale[src];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * (BN / WN) + j * 16 + lrow;
        if (col >= p.n) continue;
        float v = acc[i][j][q];
        if (KIND == K_FP8) v = (v * sa) * p.w_scale[int64_t(g) * p.n + col];
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
  }
}

// One wave per row: amax, scale = amax / 448 (0 -> 1), e4m3 codes of v / scale.
__global__ __launch_bounds__(256) void quant_rows_kernel(QuantArgs p) {
  const int64_t row = int64_t(blockIdx.x) * 4 + threadIdx.x / WAVE;
  if (row >= p.rows) return;
  const int lane = lane_id();
  const int cols = p.cols;
  auto ld4 = [&](int c, float* v) {
    if (p.in_bf16) {
      const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.in) +
                                                      row * cols + c);
      v[0] = __uint_as_float(u.x << 16);
      v[1] = __uint_as_float(u.x & 0xFFFF0000u);
      v[2] = __uint_as_float(u.y << 16);
      v[3] = __uint_as_float(u.y & 0xFFFF0000u);
    } else {
      const f32x4_t f = *reinterpret_cast<const f32x4_t*>(static_cast<const float*>(p.in) +
                                                         row * cols + c);
      v[0] = f[0];
      v[1] = f[1];
      v[2] = f[2];
      v[3] = f[3];
    }
  };
  float amax = 0.0f;
  for (int c = lane * 4; c < cols; c += WAVE * 4) {
    float v[4];
    ld4(c, v);
#pragma unroll
    for (int q = 0; q < 4; ++q) amax = fmaxf(amax, fabsf(v[q]));
  }
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  float s = amax / 448.0f;
  if (s == 0.0f) s = 1.0f;
  for (int c = lane * 4; c < cols; c += WAVE * 4) {
    float v[4];
    ld4(c, v);
    uint32_t w = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) w |= f32_to_e4m3(v[q] / s) << (8 * q);
    *reinterpret_cast<uint32_t*>(p.q + row * cols + c) = w;
  }
  if (lane == 0) p.scale[row] = s;
}

template <int KIND, int EPI>
hipError_t launch_kind_epi(const GemmArgs& p, GemmShape shape, unsigned grid, hipStream_t stream,
                           Timing t) {
  if (shape.bm == 16)
    return launch_k(gemm_kernel<KIND, 16, 128, 1, 4, EPI>, dim3(grid), dim3(G_THREADS), stream, t,
                    p);
  if (shape.bm == 64)
    return launch_k(gemm_kernel<KIND, 64, 128, 2, 2, EPI>, dim3(grid), dim3(G_THREADS), stream, t,
                    p);
  return launch_k(gemm_kernel<KIND, 128, 128, 2, 2, EPI>, dim3(grid), dim3(G_THREADS), stream, t,
                  p);
}

template <int KIND>
hipError_t launch_kind(const GemmArgs& p, int epi, GemmShape shape, unsigned grid,
                       hipStream_t stream, Timing t) {
  return epi == EPI_RELU2 ? launch_kind_epi<KIND, EPI_RELU2>(p, shape, grid, stream, t)
                          : launch_kind_epi<KIND, EPI_PLAIN>(p, shape, grid, stream, t);
}

}  // namespace

GemmShape pick_gemm_shape(int kind, int64_t rows, int groups) {
  (void)kind;
  const int64_t avg = groups > 0 ? rows / groups : rows;
  if (avg <= 24) return GemmShape{16, 128};
  if (avg <= 80) return GemmShape{64, 128};
  return GemmShape{128, 128};
}

int64_t max_mtiles(int64_t rows, int groups, int bm) {
  const int64_t bound = (rows + int64_t(groups) * (bm - 1)) / bm;
  return rows < bound ? rows : bound;
}

hipError_t launch_gemm(const GemmArgs& p, int kind, int epi, GemmShape shape, int64_t mtiles_bound,
                       hipStream_t stream, Timing t) {
  const int64_t grid64 = mtiles_bound * p.n_tiles;
  if (grid64 <= 0) return hipSuccess;
  if (grid64 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const unsigned grid = static_cast<unsigned>(grid64);
  if (kind == K_FP8) return launch_kind<K_FP8>(p, epi, shape, grid, stream, t);
  if (kind == K_BF16) return launch_kind<K_BF16>(p, epi, shape, grid, stream, t);
  return launch_kind<K_F32>(p, epi, shape, grid, stream, t);
}

hipError_t launch_quant(const QuantArgs& p, hipStream_t stream, Timing t) {
  if (p.rows <= 0) return hipSuccess;
  const int64_t blocks = (p.rows + 3) / 4;
  return launch_k(quant_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), stream, t, p);
}

}  // namespace moe
