// route.hip -- router logits and grouped top-k selection, one kernel.
//
// Layer statement: baseRT issue "Requesting converter + runtime support for
// the Nemotron-H architecture", section "Architecture (config.json)" (128
// experts, 6 per token, n_groups=8, topk_group=1, routed_scaling_factor=2.5,
// norm_topk_prob); the fp32 correction bias: auto-round PR "feat: support
// Nemotron-H / Nemotron-Cascade-2", discussion.  Sigmoid scoring, the top-2
// group score and selection-only use of the bias are this library's reading.
//
// One workgroup (4 waves) owns 16 tokens.  Logits l[16][E] come from MFMA
// (bf16 16x16x32, or four f32 16x16x4 steps) with both operands read straight
// from global memory into registers: x rows and gate rows are K-contiguous,
// so every lane loads 16 contiguous bytes and no LDS staging is needed.  Each
// wave owns E/64 of the 16-expert column blocks.  The logits then go through
// LDS to the selection phase, where each wave takes four tokens and does the
// grouped top-k with wave-wide reductions.
#include "internal.hpp"

namespace moe {

namespace {

constexpr int RT_TOK = 16;   // tokens per workgroup
constexpr int RT_MAXE = 256; // experts supported
constexpr int RT_EPL = RT_MAXE / WAVE;

template <int KIND>
__device__ __forceinline__ void router_logits(const RouteArgs& p, int64_t t0, float* lds_logit) {
  const int lane = lane_id();
  const int wave = threadIdx.x / WAVE;
  const int row = lane & 15;
  const int grp = lane >> 4;
  const int64_t t = min<int64_t>(t0 + row, p.tokens - 1);  // tail rows read the last token
  const int d = p.hidden;
  const int row_bytes = d * (KIND == K_F32 ? 4 : 2);
  const char* xrow = static_cast<const char*>(p.x) + t * row_bytes;
  const int nblk = p.n_experts / 16;
  for (int nb = wave; nb < nblk; nb += 4) {
    const char* grow = static_cast<const char*>(p.w_gate) + int64_t(nb * 16 + row) * row_bytes;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // 64-byte K step per MFMA group; unrolled by 4 to keep loads in flight
    const int steps = row_bytes / 64;
    int s = 0;
    for (; s + 4 <= steps; s += 4) {
      i32x4_t a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = *reinterpret_cast<const i32x4_t*>(xrow + (s + u) * 64 + grp * 16);
        b[u] = *reinterpret_cast<const i32x4_t*>(grow + (s + u) * 64 + grp * 16);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc = KIND == K_F32 ? mfma_f32x4(a[u], b[u], acc) : mfma_bf16(a[u], b[u], acc);
    }
    for (; s < steps; ++s) {
      i32x4_t a = *reinterpret_cast<const i32x4_t*>(xrow + s * 64 + grp * 16);
      i32x4_t b = *reinterpret_cast<const i32x4_t*>(grow + s * 64 + grp * 16);
      acc = KIND == K_F32 ? mfma_f32x4(a, b, acc) : mfma_bf16(a, b, acc);
    }
    // lane holds expert nb*16 + row, tokens 4*grp .. 4*grp+3
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_logit[(4 * grp + i) * (RT_MAXE + 1) + nb * 16 + row] = acc[i];
  }
}

__device__ void select_one(const RouteArgs& p, const float* logit, int64_t t, float* sc,
                           float* gsc) {
  const int lane = lane_id();
  const int E = p.n_experts, G = p.n_group, Eg = E / G;
  float s[RT_EPL], c[RT_EPL];
  // expert e = lane + 64 * j
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    const int e = lane + WAVE * j;
    if (e < E) {
      float l = logit[e];
      s[j] = 1.0f / (1.0f + expf(-l));
      c[j] = s[j] + p.e_bias[e];
      sc[e] = c[j];
    } else {
      s[j] = 0.f;
      c[j] = -INFINITY;
    }
  }
  wave_lds_sync();
  // group scores: lane g sums the two largest c of its group
  float gs = -INFINITY;
  if (lane < G) {
    float b1 = -INFINITY, b2 = -INFINITY;
    for (int e = lane * Eg; e < (lane + 1) * Eg; ++e) {
      float v = sc[e];
      if (v > b1) {
        b2 = b1;
        b1 = v;
      } else if (v > b2) {
        b2 = v;
      }
    }
    gs = Eg == 1 ? b1 : b1 + b2;
  }
  // keep topk_group groups
  uint64_t gmask = 0;
  for (int r = 0; r < p.topk_group; ++r) {
    float v = ((gmask >> lane) & 1) || lane >= G ? -INFINITY : gs;
    int i = lane < G && !((gmask >> lane) & 1) ? lane : 0x7FFFFFFF;
    wave_argmax(v, i);
    if (i < G) gmask |= uint64_t(1) << i;
  }
  // keep top_k experts inside the kept groups
  bool sel[RT_EPL];
  bool elig[RT_EPL];
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    const int e = lane + WAVE * j;
    sel[j] = false;
    elig[j] = e < E && ((gmask >> (e / Eg)) & 1);
  }
  for (int r = 0; r < p.top_k; ++r) {
    float v = -INFINITY;
    int i = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < RT_EPL; ++j) {
      const int e = lane + WAVE * j;
      if (elig[j] && !sel[j] && (c[j] > v || (c[j] == v && e < i))) {
        v = c[j];
        i = e;
      }
    }
    wave_argmax(v, i);
#pragma unroll
    for (int j = 0; j < RT_EPL; ++j)
      if (lane + WAVE * j == i) sel[j] = true;
  }
  // ascending expert ids: rank = selected experts with a smaller id
  int base = 0;
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    uint64_t bj = ballot(sel[j]);
    if (sel[j]) {
      int rank = base + __popcll(bj & lanemask_lt());
      gsc[rank] = s[j];
      p.topk_idx[t * p.top_k + rank] = lane + WAVE * j;
    }
    base += __popcll(bj);
  }
  wave_lds_sync();
  if (lane < p.top_k) {
    float w = gsc[lane];
    if (p.norm_topk_prob) {
      float denom = 0.f;
      for (int r = 0; r < p.top_k; ++r) denom += gsc[r];
      w = p.scale * (w / denom);
    } else {
      w = p.scale * w;
    }
    p.topk_w[t * p.top_k + lane] = w;
  }
  wave_lds_sync();
}

template <int KIND>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs p) {
  __shared__ float lds_logit[RT_TOK * (RT_MAXE + 1)];
  __shared__ float lds_c[4][RT_MAXE];
  __shared__ float lds_s[4][64];
  const int64_t t0 = int64_t(blockIdx.x) * RT_TOK;
  router_logits<KIND>(p, t0, lds_logit);
  __syncthreads();
  const int wave = threadIdx.x / WAVE;
  for (int i = wave; i < RT_TOK; i += 4) {
    const int64_t t = t0 + i;
    if (t >= p.tokens) break;
    select_one(p, lds_logit + i * (RT_MAXE + 1), t, lds_c[wave], lds_s[wave]);
  }
}

}  // namespace

hipError_t launch_route(const RouteArgs& p, int kind, hipStream_t stream, Timing t) {
  dim3 grid(static_cast<unsigned>((p.tokens + RT_TOK - 1) / RT_TOK));
  if (kind == K_F32) return launch_k(route_kernel<K_F32>, grid, dim3(256), stream, t, p);
  return launch_k(route_kernel<K_BF16>, grid, dim3(256), stream, t, p);
}

}  // namespace moe
