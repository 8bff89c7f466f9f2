/*
 * moe.h -- C ABI of libmoe: the Nemotron-H MoE layer forward on MI355X (gfx950).
 *
 * The layer (baseRT issue "Requesting converter + runtime support for the
 * Nemotron-H architecture", section "Architecture (config.json)"; exo commit
 * "Add support for Nemotron sharding", typing stub of NemotronHMoE /
 * SwitchMLP / NemotronHMLP):
 *
 *   l = x Wg^T;  s = sigmoid(l);  c = s + e_bias       (bias selects only)
 *   groups: gs_g = sum of the two largest c in group g; keep topk_group groups,
 *           then the top_k experts of largest c inside them (ties: lower index)
 *   w_j = routed_scaling_factor * s_j / sum s    (norm_topk_prob; else scale * s_j)
 *   y = sum_j w_j Wdown[e_j] relu(Wup[e_j] x)^2  +  Ws_down relu(Ws_up x)^2
 *
 * Experts are non-gated up_proj -> relu^2 -> down_proj (vllm.cpp PR
 * "spec(MODEL-TEXT-nemotron-h)"), without biases (auto-round PR "feat:
 * support Nemotron-H / Nemotron-Cascade-2", quantisation log).
 *
 * Conventions shared by every entry point
 *  - Array arguments are DEVICE pointers unless marked (host); arrays are
 *    row-major and contiguous; every array pointer must be 16-byte aligned.
 *    bf16 arrays hold IEEE bfloat16 bit patterns; fp8 arrays hold OCP e4m3fn
 *    codes; fp4 arrays hold OCP MXFP4 data: e2m1 codes two per byte (the
 *    element of lower index in the low nibble) and, per 32 consecutive
 *    elements of a row, one E8M0 scale byte (the power of two 2^(code-127)).
 *  - The caller owns every buffer, including the workspace.  The library never
 *    allocates or frees memory, never synchronises, and keeps no state between
 *    calls; all work is enqueued on `stream` (a hipStream_t, NULL = the null
 *    stream) and the call returns at once.
 *  - Arguments are checked on the host before anything is enqueued; a failed
 *    check returns MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED /
 *    MOE_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *    MOE_ERR_HIP.  Faults during execution surface at the caller's next
 *    synchronisation.
 *  - tokens == 0 is valid: nothing is enqueued and MOE_OK is returned.
 *  - Calls on one stream with one workspace run in order; concurrent calls
 *    need distinct workspaces.
 *  - Inputs must be finite; routing of NaN/Inf scores is unspecified.
 *  - Results are deterministic: no floating-point atomics, fixed reduction
 *    orders, so reruns are bitwise identical.
 *
 * Deliberate departures from a plain statement of the five calls
 *  - moe_permute takes no row-scale output for its gathered rows: with fp8
 *    experts the activation rows are quantised inside moe_expert_ffn (one
 *    scale per row, before the up GEMM), not at the permute, and the permuted
 *    rows are gathered by the GEMM while loading rather than materialised.
 *  - moe_expert_ffn takes the weights' type (w_dtype) and a row-index divisor
 *    (index_div): one call then serves the routed experts (rows gathered
 *    through the sorted slots, slot / k = token) and the shared expert (the
 *    rows as they are), in bf16, fp32, fp8 or fp4 weights.
 *  - moe_forward takes the shared expert's block scales (ws_up_scale,
 *    ws_down_scale) for 4-bit shared-expert weights.
 */
#ifndef NGR_MOE_H
#define NGR_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, misalignment, inconsistent sizes   */
  MOE_ERR_UNSUPPORTED = 2, /* valid layer, but outside what the kernels cover  */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required       */
  MOE_ERR_HIP = 4          /* a HIP launch failed                              */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2, /* routed expert weights only, with fp32 per-row scales   */
  MOE_FP4_E2M1 = 3  /* routed expert weights only, MXFP4: E8M0 scale per 32
                       elements.  4-bit experts with 16-bit activations
                       (W4A16) are the decode configuration of the Nemotron-H
                       runtime support in vllm.cpp PR
                       "spec(MODEL-TEXT-nemotron-h)"; MXFP4 is this library's
                       choice of 4-bit format                               */
} moe_dtype;

/* Layer configuration; names follow the model config (exo commit "Add support
 * for Nemotron sharding", ModelArgs).  n_group is the ROUTING group count
 * (the config field n_group), not the Mamba n_groups. */
typedef struct moe_config {
  int32_t hidden;        /* d  (hidden_size), multiple of 64                        */
  int32_t n_experts;     /* E  (n_routed_experts), multiple of 16, <= 256            */
  int32_t n_group;       /* G  routing groups, divides E, <= 64                      */
  int32_t topk_group;    /* tg groups kept per token, 1..G                           */
  int32_t top_k;         /* k  (num_experts_per_tok), 1..min(tg*E/G, 32)             */
  int32_t inter;         /* I  (moe_intermediate_size), multiple of 64               */
  int32_t shared_inter;  /* Is (moe_shared_expert_intermediate_size), multiple of 64;
                            0 = no shared expert                                     */
  int32_t norm_topk_prob;/* 0 or 1                                                   */
  float routed_scaling_factor;
  int32_t act_dtype;     /* MOE_F32 or MOE_BF16: x, w_gate, y                        */
  int32_t expert_dtype;  /* routed weights: MOE_F32 (needs act F32), MOE_BF16,
                            MOE_FP8_E4M3 or MOE_FP4_E2M1 (these need act BF16;
                            fp4 also needs d and I <= 8192)                          */
  int32_t shared_dtype;  /* shared-expert weights: act_dtype, or MOE_FP4_E2M1 when
                            expert_dtype is MOE_FP4_E2M1 (the 4-bit checkpoint of
                            vllm.cpp PR "spec(MODEL-TEXT-nemotron-h)" quantises the
                            shared experts with the routed ones; fp4: Is <= 8192)   */
} moe_config;

/* Bytes of workspace moe_forward needs for `tokens` tokens (host output). The
 * same workspace also serves moe_route and moe_permute at that size. */
moe_status moe_workspace_size(const moe_config* cfg, int64_t tokens, size_t* bytes);

/* Router and grouped top-k selection (the first two lines of the layer above).
 *   x        [tokens, d]  act_dtype
 *   w_gate   [E, d]       act_dtype (the gate is never quantised: auto-round
 *                         log, predefined ignore_layers ``mixer.gate``)
 *   e_bias   [E]          fp32 correction bias, used only to select
 *   topk_idx [tokens, k]  int32 out, each row ascending by expert id
 *   topk_w   [tokens, k]  fp32 out, aligned with topk_idx
 *   workspace optional: with at least moe_workspace_size(cfg, tokens) bytes,
 *            large calls compute the logits as one GEMM into it; without, a
 *            single kernel does all.  Both give the same bits.
 * Logits accumulate in fp32, one MFMA per K step in ascending K; scores, group
 * sums and comparisons are fp32.  A token's routing does not depend on the
 * other tokens of the call. */
moe_status moe_route(const moe_config* cfg, int64_t tokens, const void* x, const void* w_gate,
                     const float* e_bias, int32_t* topk_idx, float* topk_w, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Stable grouping of the tokens*k routing slots (slot s = t*k + j) by expert.
 * The experts are applied as one stacked weight tensor per projection to the
 * rows routed to them (exo commit "Add support for Nemotron sharding": the
 * SwitchMLP typing stub, fc1 and fc2 called as switch_mlp(x, indices)); this
 * call produces that grouping, so each expert's rows are contiguous:
 *   expert_counts  [E]        int32 out
 *   expert_offsets [E+1]      int32 out, exclusive prefix sum of the counts
 *   sorted_slot    [tokens*k] int32 out, slot at each sorted position; within
 *                             one expert the slots ascend
 *   slot_pos       [tokens*k] int32 out, inverse of sorted_slot
 *   x, x_perm      optional (both NULL or both set): x_perm [tokens*k, d]
 *                  act_dtype receives x[sorted_slot[p] / k] at row p
 * topk_idx values must lie in [0, E). */
moe_status moe_permute(const moe_config* cfg, int64_t tokens, const int32_t* topk_idx,
                       int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_slot,
                       int32_t* slot_pos, const void* x, void* x_perm, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Workspace bytes moe_expert_ffn needs for one call (host output). */
moe_status moe_expert_ffn_workspace_size(const moe_config* cfg, int32_t n_mats, int32_t inter,
                                         int32_t w_dtype, int64_t a_rows, int64_t rows,
                                         size_t* bytes);

/* Grouped non-gated expert MLPs.  An expert is up_proj -> relu^2 -> down_proj
 * with no gate projection (vllm.cpp PR "spec(MODEL-TEXT-nemotron-h)", its
 * description of the expert MLP) and no bias (auto-round PR "feat: support
 * Nemotron-H / Nemotron-Cascade-2", quantisation log: Linear(2688 -> 1856)
 * and Linear(1856 -> 2688) with bias=False); the shared expert is the same
 * MLP at its own width (exo commit, NemotronHMLP stub).  For each matrix pair
 * m and each problem row r
 * in [row_offsets[m], row_offsets[m+1]):
 *     out[r] = Wdown[m] relu(Wup[m] a[src(r)])^2,  src(r) = row_index[r] / index_div
 *                                                  (or r when row_index is NULL)
 *   a            [a_rows, d] act_dtype
 *   row_offsets  [n_mats+1] int32, ascending, row_offsets[0] = 0,
 *                row_offsets[n_mats] = rows (values are clamped to [0, rows])
 *   row_index    [rows] int32 or NULL; index_div >= 1; sources clamp to a_rows-1
 *   w_up         [n_mats, inter, d], w_down [n_mats, d, inter], of w_dtype
 *                (fp4: [n_mats, inter, d/2] and [n_mats, d, inter/2] bytes)
 *   w_up_scale, w_down_scale
 *                MOE_FP8_E4M3: fp32 per-row scales [n_mats, inter] and [n_mats, d];
 *                MOE_FP4_E2M1: E8M0 block scales (uint8) [n_mats, inter, d/32]
 *                and [n_mats, d, inter/32], codes 1..252 (every weight a
 *                normal bf16 value); code 0 only for all-zero blocks.  fp4
 *                also needs a_rows*d*2 and rows*inter*2 below 2^31 and
 *                d, inter <= 8192 (else MOE_ERR_UNSUPPORTED)
 *                otherwise NULL (ignored)
 *   out          [rows, d] fp32
 * With fp8 weights each a row is quantised per row to e4m3 (scale amax/448,
 * nearest even, saturating) before the up GEMM and each h row likewise before
 * the down GEMM; both GEMMs run on fp8 MFMA with fp32 accumulation and the
 * scales applied in the epilogue.  fp4 weights are widened to bf16 (exact:
 * an e2m1 value times a power of two is a bf16 value, for scale codes down to
 * 2^-126) and multiply bf16 a and h on bf16 MFMA.  Otherwise, and for fp4, h
 * is rounded to bf16 (nearest even; fp32 for fp32 weights) and both GEMMs
 * accumulate in fp32.
 * The routed experts of the layer are the call (n_mats = E, a = x,
 * row_offsets = expert_offsets, row_index = sorted_slot, index_div = k); the
 * shared expert is (n_mats = 1, row_offsets = {0, tokens}, row_index = NULL). */
moe_status moe_expert_ffn(const moe_config* cfg, int32_t n_mats, int32_t inter, int32_t w_dtype,
                          int64_t a_rows, const void* a, int64_t rows,
                          const int32_t* row_offsets, const int32_t* row_index,
                          int32_t index_div, const void* w_up, const void* w_up_scale,
                          const void* w_down, const void* w_down_scale, float* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* The per-row quantiser of the fp8 expert path (moe_expert_ffn with
 * MOE_FP8_E4M3 weights applies it to the rows of a before the up GEMM and to
 * the fp32 rows of h before the down GEMM).  For each row r, in fp32:
 *     s_r = max_i |in[r,i]| / 448          (1 when the row is all zeros)
 *     q[r,i] = e4m3(in[r,i] / s_r)         (correctly rounded division; the
 *              OCP 8-bit floating point specification's E4M3 encoding,
 *              nearest even, saturating at +-448; a zero result is +0)
 * so that q[r,i] * s_r approximates in[r,i].
 *   in_dtype MOE_F32 or MOE_BF16; in [rows, cols] of in_dtype; q [rows, cols]
 *   uint8 out; scale [rows] fp32 out.  cols a positive multiple of 8.
 *   rows == 0 enqueues nothing. */
moe_status moe_quantize_rows(int32_t in_dtype, int64_t rows, int32_t cols, const void* in,
                             uint8_t* q, float* scale, void* stream);

/* Weighted combine (exo commit "Add support for Nemotron sharding": the shared
 * expert's output joins the routed sum before the mixer's single reduction):
 *     y[t] = sum_{j ascending} topk_w[t,j] * y_perm[slot_pos[t*k+j]] + shared_out[t]
 * summed in fp32 and rounded once to act_dtype (nearest even for bf16).
 *   slot_pos [tokens*k] int32, topk_w [tokens,k] fp32, y_perm [tokens*k, d] fp32,
 *   shared_out [tokens, d] fp32 or NULL, y [tokens, d] act_dtype out. */
moe_status moe_combine(const moe_config* cfg, int64_t tokens, const int32_t* slot_pos,
                       const float* topk_w, const float* y_perm, const float* shared_out,
                       void* y, void* stream);

/* The whole layer: route -> permute -> routed expert MLPs -> shared expert ->
 * combine, bit-identical to that composition of the entry points above.
 * When the shared expert's weights have the routed experts' type it runs in
 * the routed GEMM launches as one extra group (same arithmetic per element).
 *   x [tokens, d], w_gate [E, d], e_bias [E] fp32, w_up [E, I, d], w_down [E, d, I]
 *   (expert_dtype; packing and scales as in moe_expert_ffn), ws_up [Is, d], ws_down [d, Is]
 *   (shared_dtype; fp4: ws_up_scale [Is, d/32] and ws_down_scale [d, Is/32] E8M0,
 *   else NULL), y [tokens, d] act_dtype out.
 *   topk_idx [tokens,k], topk_w [tokens,k], expert_counts [E]: optional outputs
 *   (NULL = not wanted).
 *   workspace: at least moe_workspace_size(cfg, tokens) bytes. */
moe_status moe_forward(const moe_config* cfg, int64_t tokens, const void* x, const void* w_gate,
                       const float* e_bias, const void* w_up, const void* w_up_scale,
                       const void* w_down, const void* w_down_scale, const void* ws_up,
                       const void* ws_up_scale, const void* ws_down, const void* ws_down_scale,
                       void* y, int32_t* topk_idx, float* topk_w,
                       int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                       void* stream);

/* moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same launches and results, with the workspace taken from a static device
 * array of MOE_STATIC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on until the process ends.  The call allocates nothing; its first
 * call on a device resolves that device's copy of the array (the current
 * device: `stream` must belong to it).
 *   Sizes: calls whose moe_workspace_size(cfg, tokens) exceeds
 *   MOE_STATIC_SCRATCH_BYTES return MOE_ERR_WORKSPACE and enqueue nothing
 *   (bf16 layers of the Nemotron-H shape: up to about 600 tokens).
 *   Sharing: every call on one GPU uses the same array and leaves its
 *   contents there; calls that overlap in time on one GPU (other streams,
 *   other threads) race and give undefined results.  Calls on one stream run
 *   in order and are safe.  Nothing in it needs clearing between calls. */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
moe_status moe_forward_static(const moe_config* cfg, int64_t tokens, const void* x,
                              const void* w_gate, const float* e_bias, const void* w_up,
                              const void* w_up_scale, const void* w_down,
                              const void* w_down_scale, const void* ws_up,
                              const void* ws_up_scale, const void* ws_down,
                              const void* ws_down_scale, void* y, int32_t* topk_idx,
                              float* topk_w, int32_t* expert_counts, void* stream);

/* Measurement variant of moe_forward: the same launches and results.  When
 * `stage_events` is not NULL it holds 2 * MOE_T_SLOTS hipEvent_t created by
 * the caller (entries may be NULL); the kernels of stage i are launched with
 * stage_events[2i] recording the start of the stage's first kernel and
 * stage_events[2i+1] the end of its last one (hipExtLaunchKernelGGL), so
 * hipEventElapsedTime of the pair is the stage's device time.  Stages that do
 * not run for the configuration leave their events untouched. */
enum {
  MOE_T_ROUTE = 0,        /* router + grouped top-k (up to 16 tokens: the
                             logits only)                                  */
  MOE_T_PERMUTE = 1,      /* histogram, scan, stable placement (up to 16
                             tokens: with the grouped top-k, one launch)   */
  MOE_T_QUANT_X = 2,      /* fp8 experts: per-token e4m3 quantisation of x */
  MOE_T_ROUTED_UP = 3,    /* routed up GEMM + relu^2                      */
  MOE_T_QUANT_H = 4,      /* fp8 experts: per-row e4m3 quantisation of h  */
  MOE_T_ROUTED_DOWN = 5,  /* routed down GEMM                             */
  MOE_T_SHARED_UP = 6,    /* shared-expert up GEMM + relu^2 (its own
                             launch when its weight type differs from the
                             routed experts' and the call does not put
                             both in one launch: moe_forward_stage_mask) */
  MOE_T_SHARED_DOWN = 7,  /* shared-expert down GEMM (its own launch in
                             the same cases)                               */
  MOE_T_COMBINE = 8,      /* weighted combine + output rounding           */
  MOE_T_NORM = 9,         /* block only: the RMSNorm before the layer     */
  MOE_T_SLOTS = 10
};
/* Which stages moe_forward runs for `tokens` tokens (host output): bit i of
 * *mask is set when stage i of the enumeration above runs (0 for tokens ==
 * 0).  moe_block_forward runs the same stages and MOE_T_NORM.  Host-only: no
 * device is touched. */
moe_status moe_forward_stage_mask(const moe_config* cfg, int64_t tokens, uint32_t* mask);
moe_status moe_forward_timed(const moe_config* cfg, int64_t tokens, const void* x,
                             const void* w_gate, const float* e_bias, const void* w_up,
                             const void* w_up_scale, const void* w_down,
                             const void* w_down_scale, const void* ws_up,
                             const void* ws_up_scale, const void* ws_down,
                             const void* ws_down_scale, void* y, int32_t* topk_idx,
                             float* topk_w, int32_t* expert_counts,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* stage_events);

/* ------------------------------------------------------------------------
 * The block around the layer (exo commit "Add support for Nemotron
 * sharding": the NemotronHBlock stub holds a pre-mixer RMSNorm and the
 * mixer; the MLX RMSNorm stub: a weight and an additive eps):
 *     out = x + MoE(RMSNorm(x)),   RMSNorm(x)_i = x_i / sqrt(mean(x^2) + eps) * g_i
 * The norm's output is held in act_dtype, its weight's type (auto-round PR,
 * discussion of norm_dtype).  Precision of the norm: sum of squares in fp64;
 * var = fp32(ss / d); r = 1 / sqrt(var + eps) in fp32 (correctly rounded);
 * n_i = (x_i * r) * g_i in fp32, rounded once (nearest even) to act_dtype.
 * For bf16 rows (squares within a factor 2^37 of each other) the fp64 sum
 * is exact, so the normalised rows are the same bits in any implementation
 * of this rule.
 */

/* RMSNorm of rows: x [tokens, d], weight [d], out [tokens, d], all act_dtype.
 * eps finite and >= 0.  out may not alias x. */
moe_status moe_rmsnorm(const moe_config* cfg, int64_t tokens, const void* x, const void* weight,
                       float eps, void* out, void* stream);

/* Bytes of workspace moe_block_forward needs (host output): moe_forward's
 * plus the normalised rows. */
moe_status moe_block_workspace_size(const moe_config* cfg, int64_t tokens, size_t* bytes);

/* The block: out = x + MoE(RMSNorm(x)).  Arguments as moe_forward, plus the
 * norm's weight [d] act_dtype and eps.  The layer routes and runs on the
 * normalised rows; the combine adds the residual x to the fp32 sum before its
 * one rounding.  out may alias x (an in-place residual update).  Stage
 * events as moe_forward_timed, with MOE_T_NORM for the norm. */
moe_status moe_block_forward(const moe_config* cfg, int64_t tokens, const void* x,
                             const void* norm_weight, float eps, const void* w_gate,
                             const float* e_bias, const void* w_up, const void* w_up_scale,
                             const void* w_down, const void* w_down_scale, const void* ws_up,
                             const void* ws_up_scale, const void* ws_down,
                             const void* ws_down_scale, void* out, int32_t* topk_idx,
                             float* topk_w, int32_t* expert_counts, void* workspace,
                             size_t workspace_bytes, void* stream);
moe_status moe_block_forward_timed(const moe_config* cfg, int64_t tokens, const void* x,
                                   const void* norm_weight, float eps, const void* w_gate,
                                   const float* e_bias, const void* w_up,
                                   const void* w_up_scale, const void* w_down,
                                   const void* w_down_scale, const void* ws_up,
                                   const void* ws_up_scale, const void* ws_down,
                                   const void* ws_down_scale, void* out, int32_t* topk_idx,
                                   float* topk_w, int32_t* expert_counts, void* workspace,
                                   size_t workspace_bytes, void* stream,
                                   void* const* stage_events);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Version of this ABI (bumped on any signature or semantic change). */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NGR_MOE_H */
