// select.hpp -- grouped top-k selection of one token, one wave.
//
// Rule (baseRT issue "Requesting converter + runtime support for the
// Nemotron-H architecture", section "Architecture (config.json)": grouped
// top-k with n_groups and topk_group, norm_topk_prob, routed_scaling_factor;
// sigmoid scores, selection-only correction bias, top-2 group score and
// lowest-index tie break are this library's reading):
//   s = sigmoid(l), c = s + b; group score = sum of the two largest c of the
//   group; keep topk_group groups, then the top_k experts of largest c in
//   them; w_j = scale * s_j / sum s (or scale * s_j); ids ascend.
#pragma once

#include "internal.hpp"

namespace moe {

constexpr int RT_MAXE = 256;  // experts supported
constexpr int RT_EPL = RT_MAXE / WAVE;

// LDS scratch of one wave's selection.  Arrays are read four entries at a
// time (16-byte aligned, lengths padded), so loops cost one LDS round trip
// per four values.
struct __attribute__((aligned(16))) SelScratch {
  float c[RT_MAXE];       // biased scores
  float cv[RT_MAXE + 4];  // candidate biased scores, ascending expert id
  float cs[RT_MAXE + 4];  // candidate unbiased scores s
  int ci[RT_MAXE + 4];    // candidate expert ids
  float g[64 + 4];        // group scores, then the kept experts' s
};

// Selection for token t from its E fp32 logits (logit[e], LDS written by this
// wave) and the correction bias (bias[e], LDS or global).
//
// Top-n picks are made by rank, not by repeated arg-max: a candidate is kept
// when fewer than n candidates beat it, where b beats a when b's key is
// larger, or equal with a lower index.  That is a strict total order, so the
// kept set is the one repeated arg-max with lowest-index ties would pick, and
// every lane finds its own answer from LDS broadcast reads instead of chains
// of cross-lane shuffles.
__device__ inline void select_general(const RouteArgs& p, const float* logit, int64_t t,
                                      SelScratch& z, const float* bias) {
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
      c[j] = s[j] + bias[e];
      z.c[e] = c[j];
    } else {
      s[j] = 0.f;
      c[j] = -INFINITY;
    }
  }
  wave_lds_sync();

  // group scores: lane g sums the two largest c of its group.  b1 >= b2 are
  // the two largest values seen (a multiset: ties count twice), updated
  // branch-free so they stay in registers.
  float gs = -INFINITY;
  if (lane < G) {
    float b1 = -INFINITY, b2 = -INFINITY;
    const int e0 = lane * Eg;
    if ((Eg & 3) == 0) {
      for (int i = e0; i < e0 + Eg; i += 4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&z.c[i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          b2 = fmaxf(b2, fminf(b1, v[q]));
          b1 = fmaxf(b1, v[q]);
        }
      }
    } else {
      for (int i = e0; i < e0 + Eg; ++i) {
        b2 = fmaxf(b2, fminf(b1, z.c[i]));
        b1 = fmaxf(b1, z.c[i]);
      }
    }
    gs = Eg == 1 ? b1 : b1 + b2;
  }
  // padded to a multiple of 4 with entries that never win
  if (lane < ((G + 3) & ~3)) z.g[lane] = lane < G ? gs : -INFINITY;
  wave_lds_sync();

  // keep the topk_group groups
  int grank = 0;
  if (lane < G) {
    for (int i = 0; i < G; i += 4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&z.g[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        grank += (v[q] > gs || (v[q] == gs && i + q < lane)) ? 1 : 0;
    }
  }
  const uint64_t gmask = ballot(lane < G && grank < p.topk_group);

  // the eligible experts, compacted in ascending id order
  int n_el = 0;
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    const int e = lane + WAVE * j;
    const bool elig = e < E && ((gmask >> (e / Eg)) & 1);
    const uint64_t b = ballot(elig);
    if (elig) {
      const int at = n_el + __popcll(b & lanemask_lt());
      z.cv[at] = c[j];
      z.cs[at] = s[j];
      z.ci[at] = e;
    }
    n_el += __popcll(b);
  }
  if (lane < ((n_el + 3) & ~3) - n_el) {
    z.cv[n_el + lane] = -INFINITY;
    z.ci[n_el + lane] = 0x7FFFFFFF;
  }
  wave_lds_sync();

  // keep the top_k of them: one candidate per lane counts those that beat it;
  // kept candidates keep their (ascending id) order
  int kept_before = 0;
  for (int i0 = 0; i0 < n_el; i0 += WAVE) {
    const int i = i0 + lane;
    const bool have = i < n_el;
    const float my_c = have ? z.cv[i] : 0.f;
    const int my_e = have ? z.ci[i] : 0;
    int rank = 0;
    for (int m = 0; m < n_el; m += 4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&z.cv[m]);
      const i32x4_t id = *reinterpret_cast<const i32x4_t*>(&z.ci[m]);
#pragma unroll
      for (int q = 0; q < 4; ++q) rank += (v[q] > my_c || (v[q] == my_c && id[q] < my_e)) ? 1 : 0;
    }
    const bool keep = have && rank < p.top_k;
    const uint64_t b = ballot(keep);
    if (keep) {
      const int pos = kept_before + __popcll(b & lanemask_lt());
      if (pos < p.top_k) {  // holds for finite scores; guards the writes otherwise
        z.g[pos] = z.cs[i];
        p.topk_idx[t * p.top_k + pos] = my_e;
      }
    }
    kept_before += __popcll(b);
  }
  // zero padding up to a multiple of 4 (adding +0 after the terms changes no sum)
  if (lane >= p.top_k && lane < ((p.top_k + 3) & ~3)) z.g[lane] = 0.0f;
  wave_lds_sync();
  if (lane < p.top_k) {
    float w = z.g[lane];
    if (p.norm_topk_prob) {
      float denom = 0.f;  // ascending expert order
      for (int i = 0; i < p.top_k; i += 4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&z.g[i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) denom += v[q];
      }
      w = p.scale * (w / denom);
    } else {
      w = p.scale * w;
    }
    p.topk_w[t * p.top_k + lane] = w;
  }
  wave_lds_sync();
}


// The same selection, with fewer instructions and LDS round trips, when
// every group is a power-of-two run of at most 64 experts and the kept
// groups hold at most 64 experts (Nemotron-H: 16-expert groups, one kept).
// Expert e = lane + 64 j sits in lane e % 64, so a group is a run of Eg
// lanes, and its two largest c are found in registers by exchanges between
// disjoint halves of the run (DPP within 16 lanes, shuffles beyond); the
// largest two of a multiset do not depend on the order they are merged in,
// so the group scores are those of select_general.  The kept candidates are
// then ranked by one 64-bit key each: the order-preserving bits of c above
// the complement of the candidate's position in ascending expert order, so
// a larger key is a larger c, or an equal c with a lower expert id.  The
// weights are the same fp32 expressions, summed in the same order.
template <int CTRL>
__device__ __forceinline__ float sel_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ void sel_top2(float& b1, float& b2, float o1, float o2) {
  const float lo = fminf(b1, o1);
  b1 = fmaxf(b1, o1);
  b2 = fmaxf(lo, fmaxf(b2, o2));
}

__device__ __forceinline__ uint64_t sel_key(float c, int at) {
  const uint32_t b = __float_as_uint(c + 0.0f);  // -0 -> +0, as the float compare has them equal
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (uint64_t(o) << 32) | uint32_t(~at);
}

__device__ inline void select_fast(const RouteArgs& p, const float* logit, int64_t t,
                                   SelScratch& z, const float* bias, int lg_eg) {
  const int lane = lane_id();
  const int E = p.n_experts, G = p.n_group, Eg = 1 << lg_eg;
  float s[RT_EPL], c[RT_EPL], gsc[RT_EPL];
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    s[j] = 0.f;
    c[j] = -INFINITY;
    gsc[j] = -INFINITY;
    if (j * WAVE < E) {  // the same for the whole wave
      const int e = lane + WAVE * j;
      const bool ok = e < E;
      const float l = ok ? logit[e] : 0.0f;
      const float b = ok ? bias[e] : 0.0f;
      const float sv = 1.0f / (1.0f + expf(-l));
      s[j] = ok ? sv : 0.0f;
      c[j] = ok ? sv + b : -INFINITY;
      // the two largest c of the lane's group: each exchange merges two
      // disjoint halves of a run of lanes
      float b1 = c[j], b2 = -INFINITY;
      if (Eg >= 2) sel_top2(b1, b2, sel_dpp<0xB1>(b1), sel_dpp<0xB1>(b2));    // lane ^ 1
      if (Eg >= 4) sel_top2(b1, b2, sel_dpp<0x4E>(b1), sel_dpp<0x4E>(b2));    // lane ^ 2
      if (Eg >= 8) sel_top2(b1, b2, sel_dpp<0x141>(b1), sel_dpp<0x141>(b2));  // 7 - lane (in 8)
      if (Eg >= 16) sel_top2(b1, b2, sel_dpp<0x140>(b1), sel_dpp<0x140>(b2)); // 15 - lane (in 16)
      if (Eg >= 32) sel_top2(b1, b2, __shfl_xor(b1, 16), __shfl_xor(b2, 16));
      if (Eg >= 64) sel_top2(b1, b2, __shfl_xor(b1, 32), __shfl_xor(b2, 32));
      gsc[j] = Eg == 1 ? b1 : b1 + b2;
      if (ok && (lane & (Eg - 1)) == 0) z.g[e >> lg_eg] = gsc[j];
    }
  }
  if (lane >= G && lane < ((G + 3) & ~3)) z.g[lane] = -INFINITY;
  wave_lds_sync();

  // keep the topk_group groups (lane g ranks group g, as select_general)
  int grank = 0;
  if (lane < G) {
    const float gs = z.g[lane];
    for (int i = 0; i < G; i += 4) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&z.g[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        grank += (v[q] > gs || (v[q] == gs && i + q < lane)) ? 1 : 0;
    }
  }
  const uint64_t gmask = ballot(lane < G && grank < p.topk_group);

  // the candidates (experts of kept groups) in ascending id order: key, s, id
  uint64_t* key = reinterpret_cast<uint64_t*>(z.cv);
  int n_el = 0;
#pragma unroll
  for (int j = 0; j < RT_EPL; ++j) {
    if (j * WAVE < E) {
      const int e = lane + WAVE * j;
      const bool elig = e < E && ((gmask >> (e >> lg_eg)) & 1);
      const uint64_t bm = ballot(elig);
      if (elig) {
        const int at = n_el + __popcll(bm & lanemask_lt());
        key[at] = sel_key(c[j], at);
        z.cs[at] = s[j];
        z.ci[at] = e;
      }
      n_el += __popcll(bm);
    }
  }
  if (lane == 0 && (n_el & 1)) key[n_el] = 0;  // beats no candidate
  wave_lds_sync();

  // candidate `lane` counts the candidates with a larger key
  int rank = 0;
  uint64_t mine = 0;
  if (lane < n_el) {
    mine = key[lane];
    for (int m = 0; m < n_el; m += 2) {
      const i32x4_t v = *reinterpret_cast<const i32x4_t*>(&key[m]);
      const uint64_t k0 = (uint64_t(uint32_t(v[1])) << 32) | uint32_t(v[0]);
      const uint64_t k1 = (uint64_t(uint32_t(v[3])) << 32) | uint32_t(v[2]);
      rank += (k0 > mine ? 1 : 0) + (k1 > mine ? 1 : 0);
    }
  }
  const bool keep = lane < n_el && rank < p.top_k;
  const uint64_t kb = ballot(keep);
  if (keep) {
    const int pos = __popcll(kb & lanemask_lt());
    z.g[pos] = z.cs[lane];
    p.topk_idx[t * p.top_k + pos] = z.ci[lane];
  }
  if (lane >= p.top_k && lane < ((p.top_k + 3) & ~3)) z.g[lane] = 0.0f;
  wave_lds_sync();
  if (lane < p.top_k) {
    float w = z.g[lane];
    if (p.norm_topk_prob) {
      float denom = 0.f;  // ascending expert order
      for (int i = 0; i < p.top_k; i += 4) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&z.g[i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) denom += v[q];
      }
      w = p.scale * (w / denom);
    } else {
      w = p.scale * w;
    }
    p.topk_w[t * p.top_k + lane] = w;
  }
  wave_lds_sync();
}

// Grouped top-k of token t: select_fast where its shape conditions hold
// (decided once per call, the same for every wave), else select_general.
__device__ inline void select_one(const RouteArgs& p, const float* logit, int64_t t,
                                  SelScratch& z, const float* bias) {
  const int Eg = p.n_experts / p.n_group;
  if ((Eg & (Eg - 1)) == 0 && Eg <= 64 && p.topk_group * Eg <= 64)
    select_fast(p, logit, t, z, bias, __builtin_ctz(Eg));
  else
    select_general(p, logit, t, z, bias);
}

}  // namespace moe
