// route.hip -- router logits and grouped top-k selection.
//
// Layer statement: baseRT issue "Requesting converter + runtime support for
// the Nemotron-H architecture", section "Architecture (config.json)" (128
// experts, 6 per token, n_groups=8, topk_group=1, routed_scaling_factor=2.5,
// norm_topk_prob); the fp32 correction bias: auto-round PR "feat: support
// Nemotron-H / Nemotron-Cascade-2", discussion.  Sigmoid scoring, the top-2
// group score and selection-only use of the bias are this library's reading.
//
// Logits l = x Wg^T accumulate in fp32 on MFMA (bf16 16x16x32, or four f32
// 16x16x4 steps per 64 bytes of K), one MFMA per K step in ascending K, the
// same order the grouped GEMM kernels use.  Three ways to get them give the
// same bits, so a token's routing does not depend on how many tokens share
// the call:
//   * route_logits_kernel (very few tokens): one wave per (16 tokens, 16
//     experts) block, so the gate matrix streams through many compute units
//     instead of one; logits go to the workspace, then route_select_kernel.
//   * route_kernel (few tokens, or no workspace): one workgroup per 16 tokens
//     computes all their logits and selects from LDS.
//   * many tokens: the logits are one dense GEMM (gemm.hip) into the
//     workspace, then route_select_kernel.
// Operands go from global memory straight into MFMA registers (x rows and
// gate rows are K-contiguous: 16 contiguous bytes per lane).
#include "select.hpp"

namespace moe {

namespace {

constexpr int RT_TOK = 16;     // tokens per block
constexpr int RT_WAVES = 8;    // waves of route_kernel
constexpr int ROUTE_U = 8;     // K steps in flight per wave (route_kernel)
constexpr int LOGIT_U = 28;    // K steps in flight per wave (route_logits_kernel)

// Logits of 16 tokens x 16 experts: lane holds expert row, tokens 4*grp..+3.
template <int KIND, int U>
__device__ __forceinline__ f32x4_t logit_block(const char* xrow, const char* grow, int steps) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < steps; s0 += U) {
    i32x4_t a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u < steps) {
        a[u] = *reinterpret_cast<const i32x4_t*>(xrow + (s0 + u) * 64);
        b[u] = *reinterpret_cast<const i32x4_t*>(grow + (s0 + u) * 64);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (s0 + u < steps)
        acc = KIND == K_F32 ? mfma_f32x4(a[u], b[u], acc) : mfma_bf16(a[u], b[u], acc);
  }
  return acc;
}

template <int KIND>
__global__ __launch_bounds__(RT_WAVES * WAVE) void route_kernel(RouteArgs p) {
  __shared__ float lds_logit[RT_TOK * (RT_MAXE + 1)];
  __shared__ SelScratch scr[RT_WAVES];
  const int64_t t0 = int64_t(blockIdx.x) * RT_TOK;
  const int lane = lane_id();
  const int wave = threadIdx.x / WAVE;
  const int row = lane & 15;
  const int grp = lane >> 4;
  const int row_bytes = p.hidden * (KIND == K_F32 ? 4 : 2);
  const int64_t t = min<int64_t>(t0 + row, p.tokens - 1);  // tail rows read the last token
  const char* xrow = static_cast<const char*>(p.x) + t * row_bytes + grp * 16;
  for (int nb = wave; nb < p.n_experts / 16; nb += RT_WAVES) {
    const char* grow =
        static_cast<const char*>(p.w_gate) + int64_t(nb * 16 + row) * row_bytes + grp * 16;
    const f32x4_t acc = logit_block<KIND, ROUTE_U>(xrow, grow, row_bytes / 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_logit[(4 * grp + i) * (RT_MAXE + 1) + nb * 16 + row] = acc[i];
  }
  __syncthreads();
  for (int i = wave; i < RT_TOK; i += RT_WAVES) {
    const int64_t tt = t0 + i;
    if (tt >= p.tokens) break;
    select_one(p, lds_logit + i * (RT_MAXE + 1), tt, scr[wave], p.e_bias);
  }
}

// One wave per (token block, expert block): logits [tokens, E] to the workspace.
template <int KIND>
__global__ __launch_bounds__(WAVE) void route_logits_kernel(RouteArgs p) {
  const int nblk = p.n_experts / 16;
  const int nb = blockIdx.x % nblk;
  const int64_t t0 = int64_t(blockIdx.x / nblk) * RT_TOK;
  const int lane = lane_id();
  const int row = lane & 15;
  const int grp = lane >> 4;
  const int row_bytes = p.hidden * (KIND == K_F32 ? 4 : 2);
  const int64_t t = min<int64_t>(t0 + row, p.tokens - 1);
  const char* xrow = static_cast<const char*>(p.x) + t * row_bytes + grp * 16;
  const char* grow =
      static_cast<const char*>(p.w_gate) + int64_t(nb * 16 + row) * row_bytes + grp * 16;
  const f32x4_t acc = logit_block<KIND, LOGIT_U>(xrow, grow, row_bytes / 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t tok = t0 + 4 * grp + i;
    if (tok < p.tokens) p.logits[tok * p.n_experts + nb * 16 + row] = acc[i];
  }
}

// Selection from logits [tokens, E] in global memory, one wave per token.
// The wave stages its token's logits and the correction bias in LDS with the
// same round trip, so the selection itself touches no global memory.
__global__ __launch_bounds__(256) void route_select_kernel(RouteArgs p) {
  __shared__ float lds_l[4][RT_MAXE];
  __shared__ float lds_b[4][RT_MAXE];
  __shared__ SelScratch scr[4];
  const int wave = threadIdx.x / WAVE;
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * 4 + wave;
  if (t >= p.tokens) return;
  float l[RT_EPL], b[RT_EPL];
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    const int e = lane + WAVE * j;
    if (e < p.n_experts) {
      l[j] = p.logits[t * p.n_experts + e];
      b[j] = p.e_bias[e];
    }
  }
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    const int e = lane + WAVE * j;
    if (e < p.n_experts) {
      lds_l[wave][e] = l[j];
      lds_b[wave][e] = b[j];
    }
  }
  wave_lds_sync();
  select_one(p, lds_l[wave], t, scr[wave], lds_b[wave]);
}

}  // namespace

hipError_t launch_route_logits_waves(const RouteArgs& p, int kind, hipStream_t stream, Timing t) {
  dim3 grid(static_cast<unsigned>((p.tokens + RT_TOK - 1) / RT_TOK * (p.n_experts / 16)));
  if (kind == K_F32) return launch_k(route_logits_kernel<K_F32>, grid, dim3(WAVE), stream, t, p);
  return launch_k(route_logits_kernel<K_BF16>, grid, dim3(WAVE), stream, t, p);
}

hipError_t launch_route(const RouteArgs& p, int kind, int mode, hipStream_t stream, Timing t) {
  const Timing first{t.start, nullptr};
  hipError_t e = hipSuccess;
  if (mode == ROUTE_ONE_KERNEL) {
    dim3 grid(static_cast<unsigned>((p.tokens + RT_TOK - 1) / RT_TOK));
    dim3 block(RT_WAVES * WAVE);
    if (kind == K_F32) return launch_k(route_kernel<K_F32>, grid, block, stream, t, p);
    return launch_k(route_kernel<K_BF16>, grid, block, stream, t, p);
  }
  if (mode == ROUTE_WAVES) {
    e = launch_route_logits_waves(p, kind, stream, first);
  } else {  // ROUTE_GEMM: the logits as a dense GEMM
    GemmArgs g{};
    GemmProblem& q = g.prob[0];
    q.a = p.x;
    q.w = p.w_gate;
    q.out = p.logits;
    q.a_rows = p.tokens;
    q.rows = p.tokens;
    q.n = p.n_experts;
    q.k = p.hidden;
    q.index_div = 1;
    g.sched = nullptr;
    g.n_groups = 1;
    // Every M tile streams the whole (small, E x d) gate matrix from L2
    // through the DMA-ring kernel: the widest tile (16, 32 or 64 rows) that
    // still gives every CU a tile re-reads it least.  Every shape gives the
    // same logits (one MFMA chain per element, K ascending).
    const int bm = p.tokens >= 256 * 64 ? 64 : p.tokens >= 256 * 32 ? 32 : 16;
    const GemmShape shape{bm, 128, true};
    g.n_tiles = (p.n_experts + shape.bn - 1) / shape.bn;
    const int64_t mtiles = (p.tokens + shape.bm - 1) / shape.bm;
    e = launch_gemm(g, kind, EPI_PLAIN, shape, mtiles, 0, stream, first);
  }
  if (e != hipSuccess) return e;
  dim3 grid(static_cast<unsigned>((p.tokens + 3) / 4));
  return launch_k(route_select_kernel, grid, dim3(256), stream, Timing{nullptr, t.stop}, p);
}

}  // namespace moe
