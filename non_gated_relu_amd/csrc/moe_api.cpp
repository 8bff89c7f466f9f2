// moe_api.cpp -- the C ABI of libmoe: argument checks, workspace layout, and
// the stream-ordered launch sequence of the Nemotron-H MoE layer forward.
//
// The layer and its configuration fields follow the exo commit "Add support
// for Nemotron sharding" (ModelArgs: moe_intermediate_size,
// moe_shared_expert_intermediate_size, n_group, n_routed_experts,
// topk_group, num_experts_per_tok, norm_topk_prob, routed_scaling_factor;
// NemotronHMoE = switch_mlp + shared_experts) and the baseRT issue
// "Requesting converter + runtime support for the Nemotron-H architecture"
// (section "Architecture (config.json)").  Unsupported layers are refused up
// front, as the exo sharding code refuses models it cannot handle.
//
// Launch sequence of moe_forward (one stream, no host synchronisation):
//   route (1 kernel, or 2 for few tokens) -> permute (1 kernel for at most
//   PM_SMALL_MAX slots, else 3; it also writes the GEMM tile schedule) ->
//   [fp8: quantise x] -> up GEMM + relu^2 -> [fp8: quantise h] -> down GEMM
//   -> combine.  When the shared expert's weights have the routed experts'
//   type it rides in the same two GEMM launches as one extra group; with fp8
//   routed experts it gets its own two bf16 launches.
#include <cmath>
#include <cstring>
#include <mutex>

#include "moe.h"
#include "internal.hpp"

using namespace moe;

namespace {

constexpr int64_t ROUTE_WAVES_MAX_TOKENS = 64;     // up to here: one wave per logit block
constexpr int64_t ROUTE_DIRECT_MAX_TOKENS = 2048;  // beyond: router logits as a GEMM
// up to here moe_forward selects and permutes in one launch (each of its 16
// waves selects at most one token; beyond, two launches are faster)
constexpr int64_t SELECT_PERMUTE_MAX_TOKENS = 16;
constexpr size_t ALIGN = 256;

size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int kind_of(int32_t dt) {
  return dt == MOE_F32 ? K_F32 : dt == MOE_BF16 ? K_BF16 : dt == MOE_FP8_E4M3 ? K_FP8 : K_FP4;
}

size_t esize(int32_t dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->hidden <= 0 || c->n_experts <= 0 || c->n_group <= 0 || c->inter <= 0 ||
      c->shared_inter < 0)
    return MOE_ERR_INVALID_ARG;
  if (c->n_experts % c->n_group != 0) return MOE_ERR_INVALID_ARG;
  if (c->topk_group < 1 || c->topk_group > c->n_group) return MOE_ERR_INVALID_ARG;
  const int eg = c->n_experts / c->n_group;
  if (c->top_k < 1 || c->top_k > c->topk_group * eg) return MOE_ERR_INVALID_ARG;
  if (c->norm_topk_prob != 0 && c->norm_topk_prob != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->routed_scaling_factor)) return MOE_ERR_INVALID_ARG;
  const bool dt_ok = ((c->act_dtype == MOE_F32 && c->expert_dtype == MOE_F32) ||
                      (c->act_dtype == MOE_BF16 &&
                       (c->expert_dtype == MOE_BF16 || c->expert_dtype == MOE_FP8_E4M3 ||
                        c->expert_dtype == MOE_FP4_E2M1))) &&
                     (c->shared_dtype == c->act_dtype ||
                      (c->shared_dtype == MOE_FP4_E2M1 && c->expert_dtype == MOE_FP4_E2M1));
  auto known = [](int32_t dt) { return dt >= MOE_F32 && dt <= MOE_FP4_E2M1; };
  if (!known(c->act_dtype) || !known(c->expert_dtype) || !known(c->shared_dtype))
    return MOE_ERR_INVALID_ARG;
  if (!dt_ok) return MOE_ERR_UNSUPPORTED;
  if (c->hidden % 64 || c->inter % 64 || c->shared_inter % 64) return MOE_ERR_UNSUPPORTED;
  if (c->n_experts % 16 || c->n_experts > 256 || c->n_group > 64 || c->top_k > 32)
    return MOE_ERR_UNSUPPORTED;
  if (c->expert_dtype == MOE_FP4_E2M1 && (c->hidden > F4_MAX_K || c->inter > F4_MAX_K))
    return MOE_ERR_UNSUPPORTED;
  if (c->shared_dtype == MOE_FP4_E2M1 && c->shared_inter > F4_MAX_K) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// fp4 weights: the GEMM addresses its activation and h rows with 32-bit
// buffer offsets, so [a_rows, K] bf16 operands must stay below 2 GiB.
bool fp4_rows_fit(int64_t a_rows, int64_t a_cols, int64_t h_rows, int64_t h_cols) {
  constexpr int64_t LIM = 0x7fffffff;
  return a_rows * a_cols * 2 <= LIM && h_rows * h_cols * 2 <= LIM;
}

moe_status check_tokens(const moe_config* c, int64_t tokens) {
  if (tokens < 0) return MOE_ERR_INVALID_ARG;
  if (tokens * c->top_k >= (int64_t(1) << 31) - 1) return MOE_ERR_UNSUPPORTED;
  if (c->expert_dtype == MOE_FP4_E2M1 &&
      !fp4_rows_fit(tokens, c->hidden, tokens * c->top_k, c->inter))
    return MOE_ERR_UNSUPPORTED;
  if (c->shared_dtype == MOE_FP4_E2M1 && !fp4_rows_fit(tokens, c->hidden, tokens, c->shared_inter))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Carves a workspace into aligned pieces (or only measures it when base is null).
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <typename T>
  T* take(size_t bytes) {
    size_t at = used;
    used = align_up(used + bytes);
    return base ? reinterpret_cast<T*>(base + at) : nullptr;
  }
};

Timing slot(void* const* ev, int i) {
  if (!ev) return Timing{};
  return Timing{static_cast<hipEvent_t>(ev[2 * i]), static_cast<hipEvent_t>(ev[2 * i + 1])};
}

// ------------------------------------------------------- grouped expert MLP

// One family of expert MLPs: n_mats matrix pairs over grouped rows.
struct Mlp {
  int n_mats = 0;
  int inter = 0;
  int32_t w_dtype = MOE_BF16;
  int64_t a_rows = 0;
  const void* a = nullptr;
  int64_t rows = 0;
  const int32_t* offsets = nullptr;  // null: one group over all rows
  const int32_t* row_index = nullptr;
  int index_div = 1;
  const void* w_up = nullptr;
  const void* up_scale = nullptr;  // fp8: fp32 per row; fp4: E8M0 per 32 elements
  const void* w_down = nullptr;
  const void* down_scale = nullptr;
  float* out = nullptr;
  // workspace
  void* h = nullptr;        // [rows, inter]: bf16 (bf16, fp4) / fp32 (fp8: fp32 staging)
  uint8_t* hq = nullptr;    // fp8 codes of h
  float* hs = nullptr;      // fp8 row scales of h
  uint8_t* aq = nullptr;    // fp8 codes of a
  float* as = nullptr;      // fp8 row scales of a
};

// Shape and tile bound of a launch over `main` (+ `extra_rows` of a second
// single-group problem).
struct FfnPlan {
  GemmShape shape;  // both projections
  int64_t mtiles_first;   // bound of the routed (or only) family's M tiles
  int64_t mtiles_extra;   // M tiles of the extra single-group family
  int64_t mtiles() const { return mtiles_first + mtiles_extra; }
};

FfnPlan plan_ffn(int32_t w_dtype, int64_t rows, int n_mats, int64_t extra_rows) {
  FfnPlan f;
  f.shape = pick_gemm_shape(kind_of(w_dtype), rows, n_mats);
  f.mtiles_first = max_mtiles(rows, n_mats, f.shape.bm);
  f.mtiles_extra = extra_rows > 0 ? (extra_rows + f.shape.bm - 1) / f.shape.bm : 0;
  return f;
}

void carve_mlp_buffers(Carver& cv, Mlp& m, int hidden) {
  const size_t hsz = m.w_dtype == MOE_BF16 || m.w_dtype == MOE_FP4_E2M1 ? 2 : 4;
  m.h = cv.take<void>(size_t(m.rows) * m.inter * hsz);
  if (m.w_dtype == MOE_FP8_E4M3) {
    m.hq = cv.take<uint8_t>(size_t(m.rows) * m.inter);
    m.hs = cv.take<float>(sizeof(float) * size_t(m.rows));
    m.aq = cv.take<uint8_t>(size_t(m.a_rows) * hidden);
    m.as = cv.take<float>(sizeof(float) * size_t(m.a_rows));
  }
}

GemmProblem up_problem(const Mlp& m, int hidden) {
  GemmProblem p{};
  const bool fp8 = m.w_dtype == MOE_FP8_E4M3;
  p.a = fp8 ? static_cast<const void*>(m.aq) : m.a;
  p.a_scale = fp8 ? m.as : nullptr;
  p.row_index = m.row_index;
  p.w = m.w_up;
  p.w_scale = fp8 ? static_cast<const float*>(m.up_scale) : nullptr;
  p.w_bscale = m.w_dtype == MOE_FP4_E2M1 ? static_cast<const uint8_t*>(m.up_scale) : nullptr;
  p.offsets = m.offsets;
  p.out = m.h;
  p.a_rows = m.a_rows;
  p.rows = m.rows;
  p.n = m.inter;
  p.k = hidden;
  p.index_div = m.index_div;
  p.out_bf16 = m.w_dtype == MOE_BF16 || m.w_dtype == MOE_FP4_E2M1;
  return p;
}

GemmProblem down_problem(const Mlp& m, int hidden) {
  GemmProblem p{};
  const bool fp8 = m.w_dtype == MOE_FP8_E4M3;
  p.a = fp8 ? static_cast<const void*>(m.hq) : m.h;
  p.a_scale = fp8 ? m.hs : nullptr;
  p.row_index = nullptr;
  p.w = m.w_down;
  p.w_scale = fp8 ? static_cast<const float*>(m.down_scale) : nullptr;
  p.w_bscale = m.w_dtype == MOE_FP4_E2M1 ? static_cast<const uint8_t*>(m.down_scale) : nullptr;
  p.offsets = m.offsets;
  p.out = m.out;
  p.a_rows = m.rows;
  p.rows = m.rows;
  p.n = hidden;
  p.k = m.inter;
  p.index_div = 1;
  p.out_bf16 = 0;
  return p;
}

struct FfnTiming {
  Timing qa, up, qh, down;
};

// Runs `m` (and `extra`, a single-group family of the same weight type, in
// the same launches).  `sched` holds the schedule already when `have_sched`.
moe_status run_mlps(int hidden, const Mlp& m, const Mlp* extra, int32_t* sched, bool have_sched,
                    hipStream_t s, const FfnTiming& tm) {
  const int64_t extra_rows = extra ? extra->rows : 0;
  if (m.rows == 0 && extra_rows == 0) return MOE_OK;
  const FfnPlan f = plan_ffn(m.w_dtype, m.rows, m.n_mats, extra_rows);
  if (!have_sched) {
    ScheduleArgs sp{m.offsets, m.rows, m.n_mats,
                    ScheduleSpec{sched, extra_rows, f.shape.bm, static_cast<int>(f.mtiles())}};
    if (launch_schedule(sp, s) != hipSuccess) return MOE_ERR_HIP;
  }
  const int kind = kind_of(m.w_dtype);
  if (kind == K_FP8) {
    QuantArgs q{m.a, m.aq, m.as, m.a_rows, hidden, 1};
    if (launch_quant(q, s, tm.qa) != hipSuccess) return MOE_ERR_HIP;
  }
  GemmArgs up{};
  up.prob[0] = up_problem(m, hidden);
  if (extra) up.prob[1] = up_problem(*extra, hidden);
  up.sched = sched;
  up.n_groups = m.n_mats;
  up.n_tiles = (m.inter + f.shape.bn - 1) / f.shape.bn;
  up.n_tiles2 = extra ? (extra->inter + f.shape.bn - 1) / f.shape.bn : 0;
  up.second_first = f.shape.bm == 16;  // decode tiles
  if (launch_gemm(up, kind, EPI_RELU2, f.shape, f.mtiles_first, f.mtiles_extra, s, tm.up) !=
      hipSuccess)
    return MOE_ERR_HIP;
  if (kind == K_FP8) {
    QuantArgs q{m.h, m.hq, m.hs, m.rows, m.inter, 0};
    if (launch_quant(q, s, tm.qh) != hipSuccess) return MOE_ERR_HIP;
  }
  GemmArgs dn{};
  dn.prob[0] = down_problem(m, hidden);
  if (extra) dn.prob[1] = down_problem(*extra, hidden);
  dn.sched = sched;
  dn.n_groups = m.n_mats;
  dn.n_tiles = (hidden + f.shape.bn - 1) / f.shape.bn;
  dn.n_tiles2 = extra ? dn.n_tiles : 0;
  dn.second_first = up.second_first;
  if (launch_gemm(dn, kind, EPI_PLAIN, f.shape, f.mtiles_first, f.mtiles_extra, s, tm.down) !=
      hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

// ---------------------------------------------------------- forward layout

struct Forward {
  int64_t T = 0, S = 0;
  bool fused_shared = false;
  float* logits = nullptr;  // router logits (many tokens)
  int32_t* block_counts = nullptr;
  int32_t* topk_idx = nullptr;
  float* topk_w = nullptr;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* sorted_slot = nullptr;
  int32_t* slot_pos = nullptr;
  int32_t* sched = nullptr;
  int32_t* shared_sched = nullptr;
  FfnPlan plan{};
  Mlp routed, shared;
};

int permute_chunks(int64_t slots) {
  if (slots <= PM_SMALL_MAX) return 1;
  return static_cast<int>((slots + PM_CHUNK - 1) / PM_CHUNK);
}

// Router path for T tokens given room for the logits (all give the same bits).
int route_mode(int64_t T) {
  if (T <= ROUTE_WAVES_MAX_TOKENS) return ROUTE_WAVES;
  if (T > ROUTE_DIRECT_MAX_TOKENS) return ROUTE_GEMM;
  return ROUTE_ONE_KERNEL;
}

size_t route_logit_bytes(const moe_config& c, int64_t T) {
  return sizeof(float) * size_t(T) * c.n_experts;
}

// Whether the shared expert runs as one more group of the routed experts'
// launches: always when it has their weight type; with fp8 experts and a bf16
// shared expert when both take the 256 x 256 ring kernels (many rows per
// expert), whose mixed form runs each tile in its own type, and their rows
// fit its 32-bit fp8 offsets.
bool shared_fused(const moe_config& c, int64_t T) {
  if (c.shared_inter <= 0) return false;
  if (c.expert_dtype == c.shared_dtype) return true;
  if (c.expert_dtype != MOE_FP8_E4M3 || c.shared_dtype != MOE_BF16) return false;
  const int64_t S = T * c.top_k;
  const int64_t lim = int64_t(1) << 32;
  return pick_gemm_shape(K_FP8, S, c.n_experts).bm == 256 && T * c.hidden < lim &&
         S * c.inter < lim && T * c.shared_inter < lim && int64_t(c.inter) * c.hidden < lim &&
         int64_t(c.shared_inter) * c.hidden < lim;
}

Forward carve_forward(Carver& cv, const moe_config& c, int64_t T) {
  Forward f;
  f.T = T;
  f.S = T * c.top_k;
  f.fused_shared = shared_fused(c, T);
  if (route_mode(T) != ROUTE_ONE_KERNEL) f.logits = cv.take<float>(route_logit_bytes(c, T));
  f.block_counts = cv.take<int32_t>(sizeof(int32_t) * size_t(permute_chunks(f.S)) * c.n_experts);
  f.topk_idx = cv.take<int32_t>(sizeof(int32_t) * size_t(f.S));
  f.topk_w = cv.take<float>(sizeof(float) * size_t(f.S));
  f.counts = cv.take<int32_t>(sizeof(int32_t) * c.n_experts);
  f.offsets = cv.take<int32_t>(sizeof(int32_t) * (c.n_experts + 1));
  f.sorted_slot = cv.take<int32_t>(sizeof(int32_t) * size_t(f.S));
  f.slot_pos = cv.take<int32_t>(sizeof(int32_t) * size_t(f.S));

  Mlp& r = f.routed;
  r.n_mats = c.n_experts;
  r.inter = c.inter;
  r.w_dtype = c.expert_dtype;
  r.a_rows = T;
  r.rows = f.S;
  r.offsets = f.offsets;
  r.row_index = f.sorted_slot;
  r.index_div = c.top_k;
  r.out = cv.take<float>(sizeof(float) * size_t(f.S) * c.hidden);  // y_perm
  carve_mlp_buffers(cv, r, c.hidden);
  if (c.shared_inter > 0) {
    Mlp& sh = f.shared;
    sh.n_mats = 1;
    sh.inter = c.shared_inter;
    sh.w_dtype = c.shared_dtype;
    sh.a_rows = T;
    sh.rows = T;
    sh.out = cv.take<float>(sizeof(float) * size_t(T) * c.hidden);
    carve_mlp_buffers(cv, sh, c.hidden);
  }
  f.plan = plan_ffn(r.w_dtype, r.rows, r.n_mats, f.fused_shared ? T : 0);
  f.sched = cv.take<int32_t>(sizeof(int32_t) * (2 + 2 * size_t(f.plan.mtiles())));
  if (c.shared_inter > 0 && !f.fused_shared) {
    const FfnPlan ps = plan_ffn(c.shared_dtype, T, 1, 0);
    f.shared_sched = cv.take<int32_t>(sizeof(int32_t) * (2 + 2 * size_t(ps.mtiles())));
  }
  return f;
}

RouteArgs route_args(const moe_config& c, int64_t T, const void* x, const void* w_gate,
                     const float* e_bias, int32_t* topk_idx, float* topk_w, float* logits) {
  return RouteArgs{x, w_gate, e_bias, topk_idx, topk_w, logits, T, c.hidden, c.n_experts,
                   c.n_group, c.topk_group, c.top_k, c.norm_topk_prob, c.routed_scaling_factor};
}

moe_status do_permute(const moe_config& c, int64_t T, const int32_t* topk_idx, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                      int32_t* block_counts, ScheduleSpec spec, hipStream_t s, Timing t = {}) {
  const int64_t S = T * c.top_k;
  PermuteArgs p{topk_idx, counts, offsets, sorted_slot, slot_pos, block_counts, S,
                permute_chunks(S), c.n_experts, spec};
  return hip_status(launch_permute(p, s, t));
}

Mlp standalone_mlp(int32_t n_mats, int32_t inter, int32_t w_dtype, int64_t a_rows,
                   const void* a, int64_t rows, const int32_t* row_offsets,
                   const int32_t* row_index, int32_t index_div) {
  Mlp m;
  m.n_mats = n_mats;
  m.inter = inter;
  m.w_dtype = w_dtype;
  m.a_rows = a_rows;
  m.a = a;
  m.rows = rows;
  m.offsets = row_offsets;
  m.row_index = row_index;
  m.index_div = index_div;
  return m;
}

size_t carve_standalone(Carver& cv, Mlp& m, int hidden, int32_t** sched) {
  const FfnPlan f = plan_ffn(m.w_dtype, m.rows, m.n_mats, 0);
  *sched = cv.take<int32_t>(sizeof(int32_t) * (2 + 2 * size_t(f.mtiles())));
  carve_mlp_buffers(cv, m, hidden);
  return cv.used;
}

struct LayerWeights {
  const void* w_gate;
  const float* e_bias;
  const void *w_up, *w_up_scale, *w_down, *w_down_scale;
  const void *ws_up, *ws_up_scale, *ws_down, *ws_down_scale;
};

// The stages moe_forward runs for a positive token count (bit i: stage i of
// the MOE_T_* enumeration).
uint32_t forward_stage_mask(const moe_config& c, int64_t T) {
  uint32_t m = (1u << MOE_T_ROUTE) | (1u << MOE_T_PERMUTE) | (1u << MOE_T_ROUTED_UP) |
               (1u << MOE_T_ROUTED_DOWN);
  if (c.expert_dtype == MOE_FP8_E4M3) m |= (1u << MOE_T_QUANT_X) | (1u << MOE_T_QUANT_H);
  const bool own_shared = c.shared_inter > 0 && !shared_fused(c, T);
  if (own_shared) m |= (1u << MOE_T_SHARED_UP) | (1u << MOE_T_SHARED_DOWN);
  return m | (1u << MOE_T_COMBINE);
}

// Bytes of the block's normalised rows in the workspace.
size_t norm_bytes(const moe_config& c, int64_t T) { return size_t(T) * c.hidden * esize(c.act_dtype); }

// The layer on x (norm_weight null), or the block x + layer(RMSNorm(x)): the
// norm's rows go to the workspace after the layer's own part, the layer runs
// on them, and the combine adds x before its rounding.
moe_status run_forward(const moe_config* cfg, int64_t tokens, const void* x,
                       const void* norm_weight, float eps, const LayerWeights& w, void* y,
                       int32_t* topk_idx, float* topk_w, int32_t* expert_counts, void* workspace,
                       size_t workspace_bytes, void* stream, void* const* ev) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  const moe_config& c = *cfg;
  const bool block = norm_weight != nullptr;
  const void* ptrs[] = {x, w.w_gate, w.e_bias, w.w_up, w.w_down, y};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (c.shared_inter > 0 &&
      (!w.ws_up || !w.ws_down || !aligned16(w.ws_up) || !aligned16(w.ws_down)))
    return MOE_ERR_INVALID_ARG;
  if ((c.expert_dtype == MOE_FP8_E4M3 || c.expert_dtype == MOE_FP4_E2M1) &&
      (!w.w_up_scale || !w.w_down_scale || !aligned16(w.w_up_scale) ||
       !aligned16(w.w_down_scale)))
    return MOE_ERR_INVALID_ARG;
  if (c.shared_inter > 0 && c.shared_dtype == MOE_FP4_E2M1 &&
      (!w.ws_up_scale || !w.ws_down_scale || !aligned16(w.ws_up_scale) ||
       !aligned16(w.ws_down_scale)))
    return MOE_ERR_INVALID_ARG;
  const void* outs[] = {topk_idx, topk_w, expert_counts};
  for (const void* p : outs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  Carver measure(nullptr);
  carve_forward(measure, c, tokens);
  if (block) measure.take<char>(norm_bytes(c, tokens));
  if (!workspace || workspace_bytes < measure.used || !aligned16(workspace))
    return MOE_ERR_WORKSPACE;
  Carver cv(workspace);
  Forward f = carve_forward(cv, c, tokens);
  void* xn = block ? cv.take<char>(norm_bytes(c, tokens)) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : f.topk_idx;
  float* wts = topk_w ? topk_w : f.topk_w;
  int32_t* cnt = expert_counts ? expert_counts : f.counts;
  if (block) {
    NormArgs na{x, norm_weight, xn, tokens, c.hidden, eps};
    if (launch_rmsnorm(na, c.act_dtype == MOE_BF16, s, slot(ev, MOE_T_NORM)) != hipSuccess)
      return MOE_ERR_HIP;
  }
  const void* xl = block ? xn : x;  // the layer's input rows
  f.routed.a = xl;
  f.routed.w_up = w.w_up;
  f.routed.up_scale = w.w_up_scale;
  f.routed.w_down = w.w_down;
  f.routed.down_scale = w.w_down_scale;
  f.shared.a = xl;
  f.shared.w_up = w.ws_up;
  f.shared.up_scale = c.shared_dtype == MOE_FP4_E2M1 ? w.ws_up_scale : nullptr;
  f.shared.w_down = w.ws_down;
  f.shared.down_scale = c.shared_dtype == MOE_FP4_E2M1 ? w.ws_down_scale : nullptr;

  const RouteArgs ra = route_args(c, tokens, xl, w.w_gate, w.e_bias, idx, wts, f.logits);
  const ScheduleSpec spec{f.sched, f.fused_shared ? tokens : 0, f.plan.shape.bm,
                          static_cast<int>(f.plan.mtiles())};
  if (tokens <= SELECT_PERMUTE_MAX_TOKENS && route_mode(tokens) == ROUTE_WAVES &&
      permute_chunks(f.S) == 1 && tokens * c.n_experts <= SP_MAX_LOGITS) {
    // decode: the logits, then the selection and the permute in one launch
    // (the permute stage's events time both)
    const PermuteArgs pa{idx, cnt, f.offsets, f.sorted_slot, f.slot_pos, f.block_counts, f.S, 1,
                         c.n_experts, spec};
    if (launch_route_logits_waves(ra, kind_of(c.act_dtype), s, slot(ev, MOE_T_ROUTE)) !=
            hipSuccess ||
        launch_select_permute(ra, pa, s, slot(ev, MOE_T_PERMUTE)) != hipSuccess)
      return MOE_ERR_HIP;
  } else {
    if (launch_route(ra, kind_of(c.act_dtype), route_mode(tokens), s, slot(ev, MOE_T_ROUTE)) !=
        hipSuccess)
      return MOE_ERR_HIP;
    if ((st = do_permute(c, tokens, idx, cnt, f.offsets, f.sorted_slot, f.slot_pos,
                         f.block_counts, spec, s, slot(ev, MOE_T_PERMUTE))) != MOE_OK)
      return st;
  }
  FfnTiming rt{slot(ev, MOE_T_QUANT_X), slot(ev, MOE_T_ROUTED_UP), slot(ev, MOE_T_QUANT_H),
               slot(ev, MOE_T_ROUTED_DOWN)};
  if ((st = run_mlps(c.hidden, f.routed, f.fused_shared ? &f.shared : nullptr, f.sched, true, s,
                     rt)) != MOE_OK)
    return st;
  if (c.shared_inter > 0 && !f.fused_shared) {
    FfnTiming sh{Timing{}, slot(ev, MOE_T_SHARED_UP), Timing{}, slot(ev, MOE_T_SHARED_DOWN)};
    if ((st = run_mlps(c.hidden, f.shared, nullptr, f.shared_sched, false, s, sh)) != MOE_OK)
      return st;
  }
  CombineArgs p{f.slot_pos, wts, f.routed.out, c.shared_inter > 0 ? f.shared.out : nullptr,
                block ? x : nullptr, y, tokens, c.hidden, c.top_k};
  return hip_status(launch_combine(p, c.act_dtype == MOE_BF16, s, slot(ev, MOE_T_COMBINE)));
}

// ----------------------------------------------- static scratch (no allocation)
//
// moe_forward_static's workspace: one file-scope device array, which every
// GPU the library runs on holds (at its own address) until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory, so
// the device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is ever handed to kernels.
// Nothing in the forward's workspace needs to start at zero (every buffer is
// written before it is read), so the array is never cleared.
constexpr size_t STATIC_SCRATCH_BYTES = size_t(MOE_STATIC_SCRATCH_BYTES);
static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The device address of the current device's scratch (resolved on the first
// call on that device).
moe_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= MAX_DEVICES) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 6; }

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

moe_status moe_forward_stage_mask(const moe_config* cfg, int64_t tokens, uint32_t* mask) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (!mask) return MOE_ERR_INVALID_ARG;
  *mask = tokens > 0 ? forward_stage_mask(*cfg, tokens) : 0u;
  return MOE_OK;
}

moe_status moe_workspace_size(const moe_config* cfg, int64_t tokens, size_t* bytes) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  Carver cv(nullptr);
  carve_forward(cv, *cfg, tokens);
  *bytes = cv.used;
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, int64_t tokens, const void* x, const void* w_gate,
                     const float* e_bias, int32_t* topk_idx, float* topk_w, void* workspace,
                     size_t workspace_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  const void* ptrs[] = {x, w_gate, e_bias, topk_idx, topk_w};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  // every router path gives the same bits; all but one need room for the logits
  int mode = route_mode(tokens);
  float* logits = nullptr;
  if (mode != ROUTE_ONE_KERNEL && workspace && aligned16(workspace) &&
      workspace_bytes >= route_logit_bytes(*cfg, tokens))
    logits = static_cast<float*>(workspace);
  if (!logits) mode = ROUTE_ONE_KERNEL;
  const RouteArgs ra = route_args(*cfg, tokens, x, w_gate, e_bias, topk_idx, topk_w, logits);
  return hip_status(launch_route(ra, kind_of(cfg->act_dtype), mode,
                                 static_cast<hipStream_t>(stream)));
}

moe_status moe_permute(const moe_config* cfg, int64_t tokens, const int32_t* topk_idx,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slot,
                       int32_t* slot_pos, const void* x, void* x_perm, void* workspace,
                       size_t workspace_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  const void* ptrs[] = {topk_idx, expert_counts, expert_offsets, sorted_slot, slot_pos};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARG;
  if (x && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_INVALID_ARG;
  const int64_t S = tokens * cfg->top_k;
  const size_t need = align_up(sizeof(int32_t) * size_t(permute_chunks(S)) * cfg->n_experts);
  if (permute_chunks(S) > 1 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = do_permute(*cfg, tokens, topk_idx, expert_counts, expert_offsets, sorted_slot, slot_pos,
                  static_cast<int32_t*>(workspace), ScheduleSpec{}, s);
  if (st != MOE_OK || !x) return st;
  GatherArgs g{x, x_perm, sorted_slot, S, static_cast<int>(cfg->hidden * esize(cfg->act_dtype)),
               cfg->top_k};
  return hip_status(launch_gather(g, s));
}


moe_status moe_expert_ffn_workspace_size(const moe_config* cfg, int32_t n_mats, int32_t inter,
                                         int32_t w_dtype, int64_t a_rows, int64_t rows,
                                         size_t* bytes) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (!bytes || n_mats < 1 || inter <= 0 || a_rows < 0 || rows < 0) return MOE_ERR_INVALID_ARG;
  if (w_dtype < MOE_F32 || w_dtype > MOE_FP4_E2M1) return MOE_ERR_INVALID_ARG;
  if (w_dtype == MOE_FP4_E2M1 && inter > F4_MAX_K) return MOE_ERR_UNSUPPORTED;
  Carver cv(nullptr);
  Mlp m = standalone_mlp(n_mats, inter, w_dtype, a_rows, nullptr, rows, nullptr, nullptr, 1);
  int32_t* sched;
  *bytes = carve_standalone(cv, m, cfg->hidden, &sched);
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* cfg, int32_t n_mats, int32_t inter, int32_t w_dtype,
                          int64_t a_rows, const void* a, int64_t rows,
                          const int32_t* row_offsets, const int32_t* row_index,
                          int32_t index_div, const void* w_up, const void* w_up_scale,
                          const void* w_down, const void* w_down_scale, float* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (n_mats < 1 || inter <= 0 || a_rows < 0 || rows < 0 || index_div < 1)
    return MOE_ERR_INVALID_ARG;
  if (w_dtype < MOE_F32 || w_dtype > MOE_FP4_E2M1) return MOE_ERR_INVALID_ARG;
  if (inter % 64) return MOE_ERR_UNSUPPORTED;
  if (w_dtype == MOE_FP4_E2M1 &&
      (inter > F4_MAX_K || !fp4_rows_fit(a_rows, cfg->hidden, rows, inter)))
    return MOE_ERR_UNSUPPORTED;
  // fp8 and fp4 weights take bf16 activations; fp32 weights take fp32; bf16 takes bf16
  const bool combo = (w_dtype == MOE_F32 && cfg->act_dtype == MOE_F32) ||
                     (w_dtype != MOE_F32 && cfg->act_dtype == MOE_BF16);
  if (!combo) return MOE_ERR_UNSUPPORTED;
  if (rows >= (int64_t(1) << 31) - 1 || a_rows >= (int64_t(1) << 31) - 1)
    return MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (a_rows == 0) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {a, row_offsets, w_up, w_down, out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (row_index && !aligned16(row_index)) return MOE_ERR_INVALID_ARG;
  if (w_dtype == MOE_FP8_E4M3 || w_dtype == MOE_FP4_E2M1) {
    if (!w_up_scale || !w_down_scale || !aligned16(w_up_scale) || !aligned16(w_down_scale))
      return MOE_ERR_INVALID_ARG;
  }
  Mlp m = standalone_mlp(n_mats, inter, w_dtype, a_rows, a, rows, row_offsets, row_index,
                         index_div);
  m.w_up = w_up;
  m.up_scale = w_up_scale;
  m.w_down = w_down;
  m.down_scale = w_down_scale;
  m.out = out;
  Carver measure(nullptr);
  int32_t* sched;
  Mlp probe = m;
  const size_t need = carve_standalone(measure, probe, cfg->hidden, &sched);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  Carver cv(workspace);
  carve_standalone(cv, m, cfg->hidden, &sched);
  return run_mlps(cfg->hidden, m, nullptr, sched, false, static_cast<hipStream_t>(stream),
                  FfnTiming{});
}

moe_status moe_combine(const moe_config* cfg, int64_t tokens, const int32_t* slot_pos,
                       const float* topk_w, const float* y_perm, const float* shared_out,
                       void* y, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  const void* ptrs[] = {slot_pos, topk_w, y_perm, y};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (shared_out && !aligned16(shared_out)) return MOE_ERR_INVALID_ARG;
  CombineArgs p{slot_pos, topk_w, y_perm, shared_out, nullptr, y, tokens, cfg->hidden,
                cfg->top_k};
  return hip_status(launch_combine(p, cfg->act_dtype == MOE_BF16, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward_timed(const moe_config* cfg, int64_t tokens, const void* x,
                             const void* w_gate, const float* e_bias, const void* w_up,
                             const void* w_up_scale, const void* w_down,
                             const void* w_down_scale, const void* ws_up,
                             const void* ws_up_scale, const void* ws_down,
                             const void* ws_down_scale, void* y, int32_t* topk_idx,
                             float* topk_w, int32_t* expert_counts,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* ev) {
  const LayerWeights w{w_gate, e_bias, w_up, w_up_scale, w_down, w_down_scale,
                       ws_up, ws_up_scale, ws_down, ws_down_scale};
  return run_forward(cfg, tokens, x, nullptr, 0.0f, w, y, topk_idx, topk_w, expert_counts,
                     workspace, workspace_bytes, stream, ev);
}

moe_status moe_forward(const moe_config* cfg, int64_t tokens, const void* x, const void* w_gate,
                       const float* e_bias, const void* w_up, const void* w_up_scale,
                       const void* w_down, const void* w_down_scale, const void* ws_up,
                       const void* ws_up_scale, const void* ws_down, const void* ws_down_scale,
                       void* y, int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return moe_forward_timed(cfg, tokens, x, w_gate, e_bias, w_up, w_up_scale, w_down, w_down_scale,
                           ws_up, ws_up_scale, ws_down, ws_down_scale, y, topk_idx, topk_w,
                           expert_counts, workspace, workspace_bytes, stream, nullptr);
}

moe_status moe_forward_static(const moe_config* cfg, int64_t tokens, const void* x,
                              const void* w_gate, const float* e_bias, const void* w_up,
                              const void* w_up_scale, const void* w_down,
                              const void* w_down_scale, const void* ws_up,
                              const void* ws_up_scale, const void* ws_down,
                              const void* ws_down_scale, void* y, int32_t* topk_idx,
                              float* topk_w, int32_t* expert_counts, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  // sizes beyond the scratch are refused before anything is resolved or enqueued
  Carver measure(nullptr);
  carve_forward(measure, *cfg, tokens);
  if (measure.used > STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != MOE_OK) return st;
  const LayerWeights w{w_gate, e_bias, w_up, w_up_scale, w_down, w_down_scale,
                       ws_up, ws_up_scale, ws_down, ws_down_scale};
  return run_forward(cfg, tokens, x, nullptr, 0.0f, w, y, topk_idx, topk_w, expert_counts, ws,
                     STATIC_SCRATCH_BYTES, stream, nullptr);
}

moe_status moe_quantize_rows(int32_t in_dtype, int64_t rows, int32_t cols, const void* in,
                             uint8_t* q, float* scale, void* stream) {
  if (in_dtype != MOE_F32 && in_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (rows < 0 || cols <= 0 || cols % 8) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  const void* ptrs[] = {in, q, scale};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  QuantArgs a{in, q, scale, rows, cols, in_dtype == MOE_BF16 ? 1 : 0};
  return hip_status(launch_quant(a, static_cast<hipStream_t>(stream)));
}

moe_status moe_rmsnorm(const moe_config* cfg, int64_t tokens, const void* x, const void* weight,
                       float eps, void* out, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (tokens < 0 || !std::isfinite(eps) || eps < 0.0f) return MOE_ERR_INVALID_ARG;
  if (tokens == 0) return MOE_OK;
  const void* ptrs[] = {x, weight, out};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  NormArgs a{x, weight, out, tokens, cfg->hidden, eps};
  return hip_status(
      launch_rmsnorm(a, cfg->act_dtype == MOE_BF16, static_cast<hipStream_t>(stream)));
}

moe_status moe_block_workspace_size(const moe_config* cfg, int64_t tokens, size_t* bytes) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (!bytes) return MOE_ERR_INVALID_ARG;
  Carver cv(nullptr);
  carve_forward(cv, *cfg, tokens);
  cv.take<char>(norm_bytes(*cfg, tokens));
  *bytes = cv.used;
  return MOE_OK;
}

moe_status moe_block_forward_timed(const moe_config* cfg, int64_t tokens, const void* x,
                                   const void* norm_weight, float eps, const void* w_gate,
                                   const float* e_bias, const void* w_up,
                                   const void* w_up_scale, const void* w_down,
                                   const void* w_down_scale, const void* ws_up,
                                   const void* ws_up_scale, const void* ws_down,
                                   const void* ws_down_scale, void* out, int32_t* topk_idx,
                                   float* topk_w, int32_t* expert_counts, void* workspace,
                                   size_t workspace_bytes, void* stream, void* const* ev) {
  if (!norm_weight || !aligned16(norm_weight) || !std::isfinite(eps) || eps < 0.0f)
    return MOE_ERR_INVALID_ARG;
  const LayerWeights w{w_gate, e_bias, w_up, w_up_scale, w_down, w_down_scale,
                       ws_up, ws_up_scale, ws_down, ws_down_scale};
  return run_forward(cfg, tokens, x, norm_weight, eps, w, out, topk_idx, topk_w, expert_counts,
                     workspace, workspace_bytes, stream, ev);
}

moe_status moe_block_forward(const moe_config* cfg, int64_t tokens, const void* x,
                             const void* norm_weight, float eps, const void* w_gate,
                             const float* e_bias, const void* w_up, const void* w_up_scale,
                             const void* w_down, const void* w_down_scale, const void* ws_up,
                             const void* ws_up_scale, const void* ws_down,
                             const void* ws_down_scale, void* out, int32_t* topk_idx,
                             float* topk_w, int32_t* expert_counts, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return moe_block_forward_timed(cfg, tokens, x, norm_weight, eps, w_gate, e_bias, w_up,
                                 w_up_scale, w_down, w_down_scale, ws_up, ws_up_scale, ws_down,
                                 ws_down_scale, out, topk_idx, topk_w, expert_counts, workspace,
                                 workspace_bytes, stream, nullptr);
}

}  // extern "C"
