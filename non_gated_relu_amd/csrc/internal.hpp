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

struct RouteArgs {
  const void* x;        // [tokens, d]
  const void* w_gate;   // [E, d]
  const float* e_bias;  // [E]
  int32_t* topk_idx;    // [tokens, k]
  float* topk_w;        // [tokens, k]
  int64_t tokens;
  int hidden, n_experts, n_group, topk_group, top_k, norm_topk_prob;
  float scale;
};

struct PermuteArgs {
  const int32_t* topk_idx;  // [slots]
  int32_t* expert_counts;   // [E]
  int32_t* expert_offsets;  // [E+1]
  int32_t* sorted_slot;     // [slots]
  int32_t* slot_pos;        // [slots]
  int32_t* block_counts;    // [n_chunks, E] workspace
  int64_t slots;
  int64_t chunk;
  int n_chunks;
  int n_experts;
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
  const int32_t* offsets;  // [n_groups+1]
  int32_t* sched;          // [2 + 2*max_tiles]
  int64_t rows;
  int n_groups;
  int bm;
  int max_tiles;
};

struct CombineArgs {
  const int32_t* slot_pos;
  const float* topk_w;
  const float* y_perm;
  const float* shared;
  void* y;
  int64_t tokens;
  int hidden, top_k;
};

enum Epilogue : int { EPI_RELU2 = 0, EPI_PLAIN = 1 };

struct GemmArgs {
  const void* a;             // [a_rows, K] operand rows (KIND elements)
  const float* a_scale;      // fp8: scale per a row, else null
  const int32_t* row_index;  // problem row -> index, or null (identity)
  const void* w;             // [groups, N, K]
  const float* w_scale;      // fp8: [groups, N], else null
  const int32_t* offsets;    // [groups+1] problem-row offsets
  const int32_t* sched;      // M-tile schedule (see schedule_kernel)
  void* out;                 // [rows, N]
  int64_t a_rows;
  int64_t rows;
  int n, k;                  // N and K in elements
  int index_div;
  int n_tiles;               // N tiles of the launch
  int out_bf16;              // epilogue stores bf16 (else fp32)
};

struct QuantArgs {
  const void* in;   // [rows, cols] fp32 or bf16
  uint8_t* q;       // [rows, cols]
  float* scale;     // [rows]
  int64_t rows;
  int cols;
  int in_bf16;
  const int32_t* valid_rows;  // optional device count: rows >= *valid_rows are skipped
};

// Tile shape of a grouped GEMM launch.
struct GemmShape {
  int bm, bn;
};

hipError_t launch_route(const RouteArgs& p, int kind, hipStream_t stream, Timing t = {});
hipError_t launch_permute(const PermuteArgs& p, hipStream_t stream, Timing t = {});
hipError_t launch_gather(const GatherArgs& p, hipStream_t stream);
hipError_t launch_schedule(const ScheduleArgs& p, hipStream_t stream, Timing t = {});
hipError_t launch_combine(const CombineArgs& p, bool bf16_out, hipStream_t stream, Timing t = {});
hipError_t launch_quant(const QuantArgs& p, hipStream_t stream, Timing t = {});

// Pick the tile shape for a grouped GEMM with `rows` problem rows over
// `groups` matrices.
GemmShape pick_gemm_shape(int kind, int64_t rows, int groups);
// Upper bound of the M tiles a schedule of this shape can hold.
int64_t max_mtiles(int64_t rows, int groups, int bm);
// Launch one grouped GEMM (schedule already built for shape.bm).
hipError_t launch_gemm(const GemmArgs& p, int kind, int epi, GemmShape shape, int64_t mtiles_bound,
                       hipStream_t stream, Timing t = {});

}  // namespace moe
