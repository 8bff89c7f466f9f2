// internal.hpp -- argument blocks and launchers shared inside libmoe.
#pragma once

#include <hip/hip_ext.h>

#include "common.hpp"

namespace moe {

// Optional kernel timestamps: a launch given events records its own start
// and end (hipExtLaunchKernelGGL), adding no packets to the stream.
struct Timing {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename... KArgs, typename... Args>
inline hipError_t launch_k(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                           Timing t, Args... args) {
  if (t.start || t.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t.start, t.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

// launch_k with `shm` bytes of dynamic LDS.
template <typename... KArgs, typename... Args>
inline hipError_t launch_k_shm(void (*kernel)(KArgs...), dim3 grid, dim3 block, unsigned shm,
                               hipStream_t s, Timing t, Args... args) {
  if (t.start || t.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, shm, s, t.start, t.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, shm, s, args...);
  return hipGetLastError();
}

struct RouteArgs {
  const void* x;        // [tokens, d]
  const void* w_gate;   // [E, d]
  const float* e_bias;  // [E]
  int32_t* topk_idx;    // [tokens, k]
  float* topk_w;        // [tokens, k]
  float* logits;        // [tokens, E] workspace (GEMM path), or null (one-kernel path)
  int64_t tokens;
  int hidden, n_experts, n_group, topk_group, top_k, norm_topk_prob;
  float scale;
};

// M-tile schedule of a grouped GEMM: sched[0] = tile count, sched[1] = the
// tiles of the first problem's groups (they come first); entry i at
// sched[2+2i] = group | (rows of the tile << 16), sched[3+2i] = first problem
// row.  A tile's rows are min(bm, rows left in its group), so a GEMM knows
// where its tile's group ends without reading the group offsets.  Tiles of a
// group are consecutive and groups come in order; the optional extra group
// (index n_groups) covers rows [0, extra_rows) of the second problem.
// Groups are fewer than 2^16 and bm at most 2^15.
struct ScheduleSpec {
  int32_t* sched;      // [2 + 2*max_tiles], or null (no schedule wanted)
  int64_t extra_rows;  // rows of the extra group (0 = none)
  int bm;
  int max_tiles;
};

// How the router gets its logits (route.hip).
enum RouteMode : int { ROUTE_ONE_KERNEL = 0, ROUTE_WAVES = 1, ROUTE_GEMM = 2 };

// Routing slots the single-workgroup permute handles; beyond, the slots are
// split into chunks of PM_CHUNK, one workgroup each.
constexpr int PM_SMALL_MAX = 4096;
// Logits the fused selection and permute stages in LDS.
constexpr int SP_MAX_LOGITS = 8192;
constexpr int PM_CHUNK = 1024;

struct PermuteArgs {
  const int32_t* topk_idx;  // [slots]
  int32_t* expert_counts;   // [E]
  int32_t* expert_offsets;  // [E+1]
  int32_t* sorted_slot;     // [slots]
  int32_t* slot_pos;        // [slots]
  int32_t* block_counts;    // [n_chunks, E] workspace
  int64_t slots;
  int n_chunks;             // 1 (single workgroup), else ceil(slots / PM_CHUNK)
  int n_experts;
  ScheduleSpec sched;       // optional: schedule of the expert GEMMs
};

struct GatherArgs {
  const void* src;
  void* dst;
  const int32_t* sorted_slot;
  int64_t rows;
  int row_bytes;
  int div;
};

struct ScheduleArgs {
  const int32_t* offsets;  // [n_groups+1], or null: one group over all rows
  int64_t rows;
  int n_groups;
  ScheduleSpec spec;
};

struct CombineArgs {
  const int32_t* slot_pos;
  const float* topk_w;
  const float* y_perm;
  const float* shared;
  const void* residual;  // [tokens, hidden] in the output type, or null
  void* y;
  int64_t tokens;
  int hidden, top_k;
};

struct NormArgs {
  const void* x;       // [tokens, hidden] activation type
  const void* weight;  // [hidden] activation type
  void* out;           // [tokens, hidden] activation type
  int64_t tokens;
  int hidden;
  float eps;
};

enum Epilogue : int { EPI_RELU2 = 0, EPI_PLAIN = 1 };

// One grouped GEMM problem: out[r] = epi(a[src(r)] . W[g]^T) for the rows r
// of group g.
struct GemmProblem {
  const void* a;             // [a_rows, K] operand rows (KIND elements)
  const float* a_scale;      // fp8: scale per a row, else null
  const int32_t* row_index;  // problem row -> index (src = index / index_div), or null
  const void* w;             // [groups, N, K]
  const float* w_scale;      // fp8: [groups, N], else null
  const uint8_t* w_bscale;   // fp4: E8M0 [groups, N, K/32], else null (w is [groups, N, K/2])
  const int32_t* offsets;    // [groups+1] problem-row offsets, or null: one group
  void* out;                 // [rows, N]
  int64_t a_rows;
  int64_t rows;
  int n, k;                  // N and K in elements
  int index_div;
  int out_bf16;              // epilogue stores bf16 (else fp32)
};

// A launch: the groups of prob[0], plus (schedule group index n_groups) the
// single group of prob[1] when the schedule holds one.  Workgroups cover the
// M tiles of prob[0], n_tiles each, and those of prob[1], n_tiles2 each, so
// that no workgroup of a launch whose problems differ in N is left without a
// tile.  prob[0]'s come first, unless second_first: decode launches start
// the shared expert's tiles (the longest in K of a down projection) first,
// so that they do not make the tail of the launch.
struct GemmArgs {
  GemmProblem prob[2];
  const int32_t* sched;
  int n_groups;
  int n_tiles;               // N tiles of prob[0]
  int n_tiles2;              // N tiles of prob[1] (0: no second problem)
  int second_first;          // prob[1]'s tiles before prob[0]'s
};

struct QuantArgs {
  const void* in;   // [rows, cols] fp32 or bf16
  uint8_t* q;       // [rows, cols]
  float* scale;     // [rows]
  int64_t rows;
  int cols;
  int in_bf16;
};

// Block scales of one fp4 weight tile are staged in LDS: BN rows x K/32
// bytes must fit, which bounds K of fp4 weights (hidden, inter, shared_inter).
constexpr int F4_SCALE_LDS = 16384;
constexpr int F4_MAX_K = F4_SCALE_LDS * 32 / 64;

// Tile shape of a grouped GEMM launch.  `stream` asks for the DMA-ring
// kernel of thin tiles (bf16, bm = 16), which keeps more bytes in flight but
// reads rows in 64-byte slices: it wins for the router's logits, where every
// tile re-reads the small gate matrix from L2, and loses to the register-
// staged kernel's 128-byte reads when the tiles stream weights from HBM.
struct GemmShape {
  int bm, bn;
  bool stream = false;
};

// ROUTE_ONE_KERNEL computes logits and selects in one kernel; the other modes
// put the logits in p.logits and then run the selection kernel.
hipError_t launch_route(const RouteArgs& p, int kind, int mode, hipStream_t stream,
                        Timing t = {});
// The logits of the ROUTE_WAVES mode only (into p.logits), without selection.
hipError_t launch_route_logits_waves(const RouteArgs& p, int kind, hipStream_t stream,
                                     Timing t = {});
hipError_t launch_permute(const PermuteArgs& p, hipStream_t stream, Timing t = {});
// Selection from r.logits and the single-workgroup permute in one launch
// (p.n_chunks == 1; r and p describe the same tokens; r.tokens * E <=
// SP_MAX_LOGITS, E % 4 == 0).
hipError_t launch_select_permute(const RouteArgs& r, const PermuteArgs& p, hipStream_t stream,
                                 Timing t = {});
hipError_t launch_gather(const GatherArgs& p, hipStream_t stream);
hipError_t launch_schedule(const ScheduleArgs& p, hipStream_t stream, Timing t = {});
hipError_t launch_combine(const CombineArgs& p, bool bf16_out, hipStream_t stream, Timing t = {});
hipError_t launch_quant(const QuantArgs& p, hipStream_t stream, Timing t = {});
hipError_t launch_rmsnorm(const NormArgs& p, bool bf16, hipStream_t stream, Timing t = {});

// Pick the tile shape for a grouped GEMM with `rows` problem rows over
// `groups` matrices (the up and the down projection of an MLP use the same
// shape, so they share one M-tile schedule).
GemmShape pick_gemm_shape(int kind, int64_t rows, int groups);
// Upper bound of the M tiles a schedule of this shape can hold.
int64_t max_mtiles(int64_t rows, int groups, int bm);
// Launch one grouped GEMM (schedule already built for shape.bm): at most
// `mtiles_first` M tiles of prob[0] and `mtiles_second` of prob[1].
hipError_t launch_gemm(const GemmArgs& p, int kind, int epi, GemmShape shape, int64_t mtiles_first,
                       int64_t mtiles_second, hipStream_t stream, Timing t = {});

}  // namespace moe
