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
#include <cmath>
#include <cstring>

#include "../../include/moe.h"
#include "internal.hpp"

using namespace moe;

namespace {

constexpr int64_t PERMUTE_CHUNK = 4096;
constexpr size_t ALIGN = 256;

size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int kind_of(int32_t dt) { return dt == MOE_F32 ? K_F32 : dt == MOE_BF16 ? K_BF16 : K_FP8; }

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
  const bool dt_ok = (c->act_dtype == MOE_F32 && c->expert_dtype == MOE_F32) ||
                     (c->act_dtype == MOE_BF16 &&
                      (c->expert_dtype == MOE_BF16 || c->expert_dtype == MOE_FP8_E4M3));
  const bool dt_known = (c->act_dtype >= 0 && c->act_dtype <= 2) &&
                        (c->expert_dtype >= 0 && c->expert_dtype <= 2);
  if (!dt_known) return MOE_ERR_INVALID_ARG;
  if (!dt_ok) return MOE_ERR_UNSUPPORTED;
  if (c->hidden % 64 || c->inter % 64 || c->shared_inter % 64) return MOE_ERR_UNSUPPORTED;
  if (c->n_experts % 16 || c->n_experts > 256 || c->n_group > 64 || c->top_k > 32)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_tokens(const moe_config* c, int64_t tokens) {
  if (tokens < 0) return MOE_ERR_INVALID_ARG;
  if (tokens * c->top_k >= (int64_t(1) << 31) - 1) return MOE_ERR_UNSUPPORTED;
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

// ------------------------------------------------------- grouped expert MLP

struct FfnPlan {
  GemmShape shape;
  int64_t mtiles;
};

FfnPlan plan_ffn(int32_t w_dtype, int64_t rows, int n_mats) {
  FfnPlan f;
  f.shape = pick_gemm_shape(kind_of(w_dtype), rows, n_mats);
  f.mtiles = max_mtiles(rows, n_mats, f.shape.bm);
  return f;
}

struct FfnBuffers {
  int32_t* sched;
  void* h;        // [rows, inter]: bf16 / fp32 (fp8: fp32 staging)
  uint8_t* hq;    // fp8 codes of h
  float* hs;      // fp8 row scales of h
  uint8_t* aq;    // fp8 codes of a
  float* as;      // fp8 row scales of a
};

FfnBuffers carve_ffn(Carver& cv, int32_t w_dtype, int inter, int hidden, int64_t a_rows,
                     int64_t rows, int n_mats) {
  FfnPlan f = plan_ffn(w_dtype, rows, n_mats);
  FfnBuffers b{};
  b.sched = cv.take<int32_t>(sizeof(int32_t) * (2 + 2 * size_t(f.mtiles)));
  const size_t hsz = w_dtype == MOE_BF16 ? 2 : 4;
  b.h = cv.take<void>(size_t(rows) * inter * hsz);
  if (w_dtype == MOE_FP8_E4M3) {
    b.hq = cv.take<uint8_t>(size_t(rows) * inter);
    b.hs = cv.take<float>(sizeof(float) * size_t(rows));
    b.aq = cv.take<uint8_t>(size_t(a_rows) * hidden);
    b.as = cv.take<float>(sizeof(float) * size_t(a_rows));
  }
  return b;
}

// Timing slots of one grouped MLP: quantise a, up GEMM, quantise h, down GEMM.
struct FfnTiming {
  Timing qa, up, qh, down;
};

moe_status run_ffn(const moe_config& c, int n_mats, int inter, int32_t w_dtype, int64_t a_rows,
                   const void* a, int64_t rows, const int32_t* offsets, const int32_t* row_index,
                   int index_div, const void* w_up, const float* up_scale, const void* w_down,
                   const float* down_scale, float* out, const FfnBuffers& b, hipStream_t s,
                   const FfnTiming& tm = FfnTiming{}) {
  if (rows == 0) return MOE_OK;
  const FfnPlan f = plan_ffn(w_dtype, rows, n_mats);
  hipError_t e;
  ScheduleArgs sp{offsets, b.sched, rows, n_mats, f.shape.bm, static_cast<int>(f.mtiles)};
  if ((e = launch_schedule(sp, s)) != hipSuccess) return MOE_ERR_HIP;
  const int kind = kind_of(w_dtype);
  const void* a_op = a;
  const float* a_sc = nullptr;
  if (kind == K_FP8) {
    QuantArgs q{a, b.aq, b.as, a_rows, c.hidden, 1, nullptr};
    if ((e = launch_quant(q, s, tm.qa)) != hipSuccess) return MOE_ERR_HIP;
    a_op = b.aq;
    a_sc = b.as;
  }
  GemmArgs up{};
  up.a = a_op;
  up.a_scale = a_sc;
  up.row_index = row_index;
  up.w = w_up;
  up.w_scale = up_scale;
  up.offsets = offsets;
  up.sched = b.sched;
  up.out = b.h;
  up.a_rows = a_rows;
  up.rows = rows;
  up.n = inter;
  up.k = c.hidden;
  up.index_div = index_div;
  up.n_tiles = (inter + f.shape.bn - 1) / f.shape.bn;
  up.out_bf16 = w_dtype == MOE_BF16;
  if ((e = launch_gemm(up, kind, EPI_RELU2, f.shape, f.mtiles, s, tm.up)) != hipSuccess)
    return MOE_ERR_HIP;
  const void* h_op = b.h;
  const float* h_sc = nullptr;
  if (kind == K_FP8) {
    QuantArgs q{b.h, b.hq, b.hs, rows, inter, 0, nullptr};
    if ((e = launch_quant(q, s, tm.qh)) != hipSuccess) return MOE_ERR_HIP;
    h_op = b.hq;
    h_sc = b.hs;
  }
  GemmArgs dn{};
  dn.a = h_op;
  dn.a_scale = h_sc;
  dn.row_index = nullptr;
  dn.w = w_down;
  dn.w_scale = down_scale;
  dn.offsets = offsets;
  dn.sched = b.sched;
  dn.out = out;
  dn.a_rows = rows;
  dn.rows = rows;
  dn.n = c.hidden;
  dn.k = inter;
  dn.index_div = 1;
  dn.n_tiles = (c.hidden + f.shape.bn - 1) / f.shape.bn;
  dn.out_bf16 = 0;
  if ((e = launch_gemm(dn, kind, EPI_PLAIN, f.shape, f.mtiles, s, tm.down)) != hipSuccess)
    return MOE_ERR_HIP;
  return MOE_OK;
}

// ---------------------------------------------------------- forward layout

struct FwdBuffers {
  int32_t* block_counts;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_slot;
  int32_t* slot_pos;
  float* y_perm;
  float* shared_out;
  FfnBuffers routed;
  FfnBuffers shared;
};

int permute_chunks(int64_t slots) {
  return static_cast<int>((slots + PERMUTE_CHUNK - 1) / PERMUTE_CHUNK);
}

FwdBuffers carve_forward(Carver& cv, const moe_config& c, int64_t T) {
  FwdBuffers b{};
  const int64_t S = T * c.top_k;
  b.block_counts = cv.take<int32_t>(sizeof(int32_t) * size_t(permute_chunks(S)) * c.n_experts);
  b.topk_idx = cv.take<int32_t>(sizeof(int32_t) * size_t(S));
  b.topk_w = cv.take<float>(sizeof(float) * size_t(S));
  b.counts = cv.take<int32_t>(sizeof(int32_t) * c.n_experts);
  b.offsets = cv.take<int32_t>(sizeof(int32_t) * (c.n_experts + 1));
  b.sorted_slot = cv.take<int32_t>(sizeof(int32_t) * size_t(S));
  b.slot_pos = cv.take<int32_t>(sizeof(int32_t) * size_t(S));
  b.y_perm = cv.take<float>(sizeof(float) * size_t(S) * c.hidden);
  b.routed = carve_ffn(cv, c.expert_dtype, c.inter, c.hidden, T, S, c.n_experts);
  if (c.shared_inter > 0) {
    b.shared_out = cv.take<float>(sizeof(float) * size_t(T) * c.hidden);
    b.shared = carve_ffn(cv, c.act_dtype, c.shared_inter, c.hidden, T, T, 1);
  }
  return b;
}

moe_status do_route(const moe_config& c, int64_t T, const void* x, const void* w_gate,
                    const float* e_bias, int32_t* topk_idx, float* topk_w, hipStream_t s,
                    Timing t = {}) {
  RouteArgs p{x, w_gate, e_bias, topk_idx, topk_w, T, c.hidden, c.n_experts, c.n_group,
              c.topk_group, c.top_k, c.norm_topk_prob, c.routed_scaling_factor};
  return hip_status(launch_route(p, kind_of(c.act_dtype), s, t));
}

moe_status do_permute(const moe_config& c, int64_t T, const int32_t* topk_idx, int32_t* counts,
                      int32_t* offsets, int32_t* sorted_slot, int32_t* slot_pos,
                      int32_t* block_counts, hipStream_t s, Timing t = {}) {
  const int64_t S = T * c.top_k;
  PermuteArgs p{topk_idx, counts, offsets, sorted_slot, slot_pos, block_counts, S,
                PERMUTE_CHUNK, permute_chunks(S), c.n_experts};
  return hip_status(launch_permute(p, s, t));
}

Timing slot(void* const* ev, int i) {
  if (!ev) return Timing{};
  return Timing{static_cast<hipEvent_t>(ev[2 * i]), static_cast<hipEvent_t>(ev[2 * i + 1])};
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return 1; }

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
  (void)workspace;
  (void)workspace_bytes;
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  const void* ptrs[] = {x, w_gate, e_bias, topk_idx, topk_w};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  return do_route(*cfg, tokens, x, w_gate, e_bias, topk_idx, topk_w,
                  static_cast<hipStream_t>(stream));
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
                  static_cast<int32_t*>(workspace), s);
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
  if (w_dtype < 0 || w_dtype > 2) return MOE_ERR_INVALID_ARG;
  Carver cv(nullptr);
  carve_ffn(cv, w_dtype, inter, cfg->hidden, a_rows, rows, n_mats);
  *bytes = cv.used;
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_config* cfg, int32_t n_mats, int32_t inter, int32_t w_dtype,
                          int64_t a_rows, const void* a, int64_t rows,
                          const int32_t* row_offsets, const int32_t* row_index,
                          int32_t index_div, const void* w_up, const float* w_up_scale,
                          const void* w_down, const float* w_down_scale, float* out,
                          void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if (n_mats < 1 || inter <= 0 || a_rows < 0 || rows < 0 || index_div < 1)
    return MOE_ERR_INVALID_ARG;
  if (w_dtype < 0 || w_dtype > 2) return MOE_ERR_INVALID_ARG;
  if (inter % 64) return MOE_ERR_UNSUPPORTED;
  // fp8 weights take bf16 activations; fp32 weights take fp32; bf16 takes bf16
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
  if (w_dtype == MOE_FP8_E4M3) {
    if (!w_up_scale || !w_down_scale || !aligned16(w_up_scale) || !aligned16(w_down_scale))
      return MOE_ERR_INVALID_ARG;
  }
  Carver measure(nullptr);
  carve_ffn(measure, w_dtype, inter, cfg->hidden, a_rows, rows, n_mats);
  if (!workspace || workspace_bytes < measure.used || !aligned16(workspace))
    return MOE_ERR_WORKSPACE;
  Carver cv(workspace);
  FfnBuffers b = carve_ffn(cv, w_dtype, inter, cfg->hidden, a_rows, rows, n_mats);
  return run_ffn(*cfg, n_mats, inter, w_dtype, a_rows, a, rows, row_offsets, row_index, index_div,
                 w_up, w_up_scale, w_down, w_down_scale, out, b,
                 static_cast<hipStream_t>(stream));
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
  CombineArgs p{slot_pos, topk_w, y_perm, shared_out, y, tokens, cfg->hidden, cfg->top_k};
  return hip_status(launch_combine(p, cfg->act_dtype == MOE_BF16, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward_timed(const moe_config* cfg, int64_t tokens, const void* x,
                             const void* w_gate, const float* e_bias, const void* w_up,
                             const float* w_up_scale, const void* w_down,
                             const float* w_down_scale, const void* ws_up, const void* ws_down,
                             void* y, int32_t* topk_idx, float* topk_w, int32_t* expert_counts,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* ev) {
  moe_status st = check_config(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_tokens(cfg, tokens)) != MOE_OK) return st;
  if (tokens == 0) return MOE_OK;
  const moe_config& c = *cfg;
  const void* ptrs[] = {x, w_gate, e_bias, w_up, w_down, y};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARG;
  if (c.shared_inter > 0 && (!ws_up || !ws_down || !aligned16(ws_up) || !aligned16(ws_down)))
    return MOE_ERR_INVALID_ARG;
  if (c.expert_dtype == MOE_FP8_E4M3 &&
      (!w_up_scale || !w_down_scale || !aligned16(w_up_scale) || !aligned16(w_down_scale)))
    return MOE_ERR_INVALID_ARG;
  const void* outs[] = {topk_idx, topk_w, expert_counts};
  for (const void* p : outs)
    if (p && !aligned16(p)) return MOE_ERR_INVALID_ARG;
  Carver measure(nullptr);
  carve_forward(measure, c, tokens);
  if (!workspace || workspace_bytes < measure.used || !aligned16(workspace))
    return MOE_ERR_WORKSPACE;
  Carver cv(workspace);
  FwdBuffers b = carve_forward(cv, c, tokens);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* idx = topk_idx ? topk_idx : b.topk_idx;
  float* wts = topk_w ? topk_w : b.topk_w;
  int32_t* cnt = expert_counts ? expert_counts : b.counts;
  const int64_t S = tokens * c.top_k;

  if ((st = do_route(c, tokens, x, w_gate, e_bias, idx, wts, s, slot(ev, MOE_T_ROUTE))) != MOE_OK)
    return st;
  if ((st = do_permute(c, tokens, idx, cnt, b.offsets, b.sorted_slot, b.slot_pos, b.block_counts,
                       s, slot(ev, MOE_T_PERMUTE))) != MOE_OK)
    return st;
  FfnTiming rt{slot(ev, MOE_T_QUANT_X), slot(ev, MOE_T_ROUTED_UP), slot(ev, MOE_T_QUANT_H),
               slot(ev, MOE_T_ROUTED_DOWN)};
  if ((st = run_ffn(c, c.n_experts, c.inter, c.expert_dtype, tokens, x, S, b.offsets,
                    b.sorted_slot, c.top_k, w_up, w_up_scale, w_down, w_down_scale, b.y_perm,
                    b.routed, s, rt)) != MOE_OK)
    return st;
  if (c.shared_inter > 0) {
    FfnTiming sh{Timing{}, slot(ev, MOE_T_SHARED_UP), Timing{}, slot(ev, MOE_T_SHARED_DOWN)};
    if ((st = run_ffn(c, 1, c.shared_inter, c.act_dtype, tokens, x, tokens, nullptr, nullptr, 1,
                      ws_up, nullptr, ws_down, nullptr, b.shared_out, b.shared, s, sh)) != MOE_OK)
      return st;
  }
  CombineArgs p{b.slot_pos, wts, b.y_perm, c.shared_inter > 0 ? b.shared_out : nullptr, y,
                tokens, c.hidden, c.top_k};
  return hip_status(launch_combine(p, c.act_dtype == MOE_BF16, s, slot(ev, MOE_T_COMBINE)));
}

moe_status moe_forward(const moe_config* cfg, int64_t tokens, const void* x, const void* w_gate,
                       const float* e_bias, const void* w_up, const float* w_up_scale,
                       const void* w_down, const float* w_down_scale, const void* ws_up,
                       const void* ws_down, void* y, int32_t* topk_idx, float* topk_w,
                       int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                       void* stream) {
  return moe_forward_timed(cfg, tokens, x, w_gate, e_bias, w_up, w_up_scale, w_down, w_down_scale,
                           ws_up, ws_down, y, topk_idx, topk_w, expert_counts, workspace,
                           workspace_bytes, stream, nullptr);
}

}  // extern "C"
