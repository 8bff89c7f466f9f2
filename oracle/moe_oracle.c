/*
 * moe_oracle.c -- plain fp64 CPU oracle of the Nemotron-H MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the HIP path.
 *
 * What it computes, per token (everything in fp64 unless said otherwise):
 *
 *   router (auto-round PR "feat: support Nemotron-H / Nemotron-Cascade-2",
 *   discussion: the router correction bias is one of the tensors kept fp32;
 *   ModelOpt page "nemotron_h_model_descriptor", class
 *   NemotronHExpertRemovalLayerDescriptor: the gate holds router weights and
 *   router biases; the quantisation log keeps ``mixer.gate`` unquantised)
 *     l_e  = sum_i x_i * Wg[e,i]                      (no linear bias)
 *     s_e  = 1 / (1 + exp(-l_e))                      (sigmoid, a reading)
 *     c_e  = s_e + b_e                                (bias used to select only)
 *
 *   grouped top-k (baseRT issue "Requesting converter + runtime support for
 *   the Nemotron-H architecture", section "Architecture (config.json)":
 *   128 experts, 6 per token, n_groups=8, topk_group=1,
 *   routed_scaling_factor=2.5, norm_topk_prob)
 *     group g = experts [g*Eg, (g+1)*Eg)               (contiguous, a reading)
 *     gs_g = sum of the two largest c_e in group g     (c_e itself if Eg == 1)
 *     keep the topk_group groups of largest gs_g, then the top_k experts of
 *     largest c_e inside them; equal keys go to the lower index.
 *     w_j = scale * s_j / sum_j' s_j'  (norm_topk_prob) else scale * s_j
 *     the chosen experts are reported in ascending expert id.
 *
 *   experts (vllm.cpp PR "spec(MODEL-TEXT-nemotron-h)": the MoE is non-gated,
 *   up_proj -> relu^2 -> down_proj; auto-round log: Linear(2688 -> 1856) and
 *   Linear(1856 -> 2688), bias=False)
 *     o = Wdown[e] * relu(Wup[e] * x)^2
 *   shared expert (exo commit "Add support for Nemotron sharding": the MoE
 *   mixer holds ``shared_experts``, an up/down MLP; baseRT issue: one shared
 *   expert, 3712 wide), added unscaled after the routed sum:
 *     y = sum_j w_j o_j  (j ascending)  +  Ws_down * relu(Ws_up * x)^2
 *
 * Precision modes.  Inputs are the stored values (fp32, bf16 bits, or fp8
 * e4m3 codes times an fp32 per-row scale) widened exactly to fp64.
 *   ORC_EXACT          h = relu(u)^2 is used unrounded.
 *   ORC_AS_CONFIGURED  h is held in the storage type of the GEMM that reads
 *                      it: rounded once from fp64 to bf16 (nearest even) for
 *                      bf16 weights, to fp32 for fp32 weights; for fp8 routed
 *                      weights h is rounded to fp32 and quantised per row
 *                      (below), and x is quantised per token before the
 *                      routed GEMMs.  The shared expert and the router keep
 *                      x as stored.
 *
 * 4-bit experts (vllm.cpp PR "spec(MODEL-TEXT-nemotron-h)": the published
 * checkpoint keeps its experts in a 4-bit W4A16 format; here the OCP MX
 * format MXFP4 stands in for it): a weight is an OCP e2m1 code (1 sign,
 * 2 exponent, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6) times the E8M0
 * scale 2^(X - 127) of its block of 32 along the input dimension.
 * Activations stay bf16 (W4A16): x is used as stored and h is held in bf16.
 * The same checkpoint holds its shared experts in that 4-bit format too, so
 * the shared expert may take fp4 weights (shared_dtype) like the routed ones.
 *
 * fp8 e4m3 per-row quantiser (OCP 8-bit floating point spec, E4M3 encoding:
 * bias 7, 3 mantissa bits, max 448, no infinities, S.1111.111 is NaN), all in
 * fp32 arithmetic: amax = max|v_i|; s = amax / 448 (0 -> 1); q_i = nearest
 * even e4m3 of v_i / s, magnitudes above 448 saturate to 448; value q_i * s.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_FP8 2
#define ORC_FP4 3

#define ORC_EXACT 0
#define ORC_AS_CONFIGURED 1

typedef struct {
  int32_t hidden;       /* d  */
  int32_t n_experts;    /* E  */
  int32_t n_group;      /* G  */
  int32_t topk_group;   /* tg */
  int32_t top_k;        /* k  */
  int32_t inter;        /* I  */
  int32_t shared_inter; /* Is, 0 = no shared expert */
  int32_t norm_topk_prob;
  double routed_scaling_factor;
  int32_t act_dtype;    /* x, w_gate, y */
  int32_t expert_dtype; /* routed weights */
  int32_t shared_dtype; /* shared-expert weights: act_dtype, or ORC_FP4 */
} orc_cfg;

#ifdef _OPENMP
#include <omp.h>
#endif

int orc_version(void) { return 6; }

/* Threads an OpenMP loop of the oracle uses. */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ codecs */

double orc_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Nearest-even rounding of a double to the 8-bit significand of bf16, in one
 * step (no detour through fp32, which would round twice). */
uint16_t orc_bf16_from_double(double v) {
  if (v == 0.0 || isnan(v) || isinf(v)) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
  }
  int e;
  frexp(fabs(v), &e);            /* |v| = m * 2^e, m in [0.5, 1) */
  int unb = e - 1;               /* |v| in [2^unb, 2^(unb+1)) */
  if (unb < -126) unb = -126;    /* bf16 subnormals share the lowest binade */
  double quantum = ldexp(1.0, unb - 7);
  double r = nearbyint(v / quantum) * quantum; /* default mode: ties to even */
  float f = (float)r;            /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

double orc_e4m3_to_double(uint8_t c) {
  int s = c >> 7, E = (c >> 3) & 15, M = c & 7;
  if (E == 15 && M == 7) return NAN;
  double mag = (E == 0) ? ldexp((double)M, -9) : ldexp(1.0 + M / 8.0, E - 7);
  return s ? -mag : mag;
}

/* OCP e2m1 (4 bits: sign, 2 exponent bits with bias 1, 1 mantissa bit) */
double orc_e2m1_to_double(uint8_t c) {
  int s = (c >> 3) & 1, E = (c >> 1) & 3, M = c & 1;
  double mag = (E == 0) ? 0.5 * M : ldexp(1.0 + 0.5 * M, E - 1);
  return s ? -mag : mag;
}
void orc_e2m1_to_double_array(const uint8_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e2m1_to_double(in[i]);
}
double orc_e8m0_to_double(uint8_t x);
void orc_e8m0_to_double_array(const uint8_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e8m0_to_double(in[i]);
}

uint8_t orc_e4m3_from_float(float vf) {
  double v = (double)vf;
  if (isnan(v)) return 0x7F;
  uint8_t sign = signbit(v) ? 0x80 : 0x00;
  double mag = fabs(v);
  int e;
  frexp(mag, &e);
  int unb = e - 1;
  if (unb < -6) unb = -6;        /* subnormal step 2^-9 */
  double quantum = ldexp(1.0, unb - 3);
  double r = nearbyint(mag / quantum) * quantum;
  if (r > 448.0) r = 448.0;      /* saturate */
  if (r == 0.0) return 0;        /* -0 encodes as +0 */
  uint8_t code;
  if (r < ldexp(1.0, -6)) {
    code = (uint8_t)nearbyint(r / ldexp(1.0, -9));
  } else {
    int re;
    frexp(r, &re);
    int E = re - 1 + 7;
    int M = (int)nearbyint((r / ldexp(1.0, re - 1) - 1.0) * 8.0);
    code = (uint8_t)((E << 3) | M);
  }
  return (uint8_t)(code | sign);
}

/* Per-row quantiser, fp32 arithmetic throughout. */
void orc_quantize_row(const float* v, int64_t n, uint8_t* q, float* scale) {
  float amax = 0.0f;
  for (int64_t i = 0; i < n; ++i) {
    float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  float s = amax / 448.0f;
  if (s == 0.0f) s = 1.0f;
  for (int64_t i = 0; i < n; ++i) q[i] = orc_e4m3_from_float(v[i] / s);
  *scale = s;
}

void orc_bf16_from_double_array(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(in[i]);
}
void orc_e4m3_from_float_array(const float* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_from_float(in[i]);
}
void orc_e4m3_to_double_array(const uint8_t* in, double* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_to_double(in[i]);
}
void orc_quantize_rows(const float* v, int64_t rows, int64_t cols, uint8_t* q, float* s) {
  for (int64_t r = 0; r < rows; ++r) orc_quantize_row(v + r * cols, cols, q + r * cols, s + r);
}

/* --------------------------------------------------------- stored values */

/* OCP MX E8M0 scale: 2^(X - 127) (X = 255 is NaN) */
double orc_e8m0_to_double(uint8_t x) { return x == 255 ? NAN : ldexp(1.0, (int)x - 127); }

/* A stored weight matrix: elements of dtype `dt` at `w`; fp8 rows carry one
 * fp32 scale each (`row_scale`); fp4 rows hold two codes per byte (element
 * 2i in the low nibble of byte i) and one E8M0 scale per block of 32
 * elements (`bscale`, [rows, n / 32]). */
typedef struct {
  const void* w;
  int dt;
  const float* row_scale;
  const uint8_t* bscale;
} orc_mat;

static orc_mat plain_mat(const void* w, int dt) {
  orc_mat m = {w, dt, NULL, NULL};
  return m;
}

/* Widen row `row` (length n) of a stored matrix to fp64 (scales applied). */
static void widen_row(orc_mat m, int64_t row, int64_t n, double* out) {
  if (m.dt == ORC_F32) {
    const float* p = (const float*)m.w + row * n;
    for (int64_t i = 0; i < n; ++i) out[i] = (double)p[i];
  } else if (m.dt == ORC_BF16) {
    const uint16_t* p = (const uint16_t*)m.w + row * n;
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_double(p[i]);
  } else if (m.dt == ORC_FP8) {
    const uint8_t* p = (const uint8_t*)m.w + row * n;
    double s = (double)m.row_scale[row];
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_to_double(p[i]) * s;
  } else {
    const uint8_t* p = (const uint8_t*)m.w + row * (n / 2);
    const uint8_t* bs = m.bscale + row * (n / 32);
    for (int64_t i = 0; i < n; ++i) {
      uint8_t c = (i & 1) ? (p[i / 2] >> 4) : (p[i / 2] & 15);
      out[i] = orc_e2m1_to_double(c) * orc_e8m0_to_double(bs[i / 32]);
    }
  }
}

/* dot of an fp64 vector with row `row` of a stored matrix */
static double dot_row(const double* a, orc_mat m, int64_t row, int64_t n) {
  double acc = 0.0;
  if (m.dt == ORC_F32) {
    const float* p = (const float*)m.w + row * n;
    for (int64_t i = 0; i < n; ++i) acc += a[i] * (double)p[i];
  } else if (m.dt == ORC_BF16) {
    const uint16_t* p = (const uint16_t*)m.w + row * n;
    for (int64_t i = 0; i < n; ++i) {
      uint32_t u = (uint32_t)p[i] << 16;
      float f;
      memcpy(&f, &u, 4);
      acc += a[i] * (double)f;
    }
  } else if (m.dt == ORC_FP8) {
    const uint8_t* p = (const uint8_t*)m.w + row * n;
    double s = (double)m.row_scale[row];
    double part = 0.0;
    for (int64_t i = 0; i < n; ++i) part += a[i] * orc_e4m3_to_double(p[i]);
    acc = part * s; /* the row scale is a common factor of the row */
  } else {
    /* each block of 32 shares its E8M0 scale */
    const uint8_t* p = (const uint8_t*)m.w + row * (n / 2);
    const uint8_t* bs = m.bscale + row * (n / 32);
    for (int64_t b = 0; b < n / 32; ++b) {
      double part = 0.0;
      for (int64_t i = b * 32; i < b * 32 + 32; ++i) {
        uint8_t c = (i & 1) ? (p[i / 2] >> 4) : (p[i / 2] & 15);
        part += a[i] * orc_e2m1_to_double(c);
      }
      acc += part * orc_e8m0_to_double(bs[b]);
    }
  }
  return acc;
}

/* ------------------------------------------------------------ block norm */

/* The block around the layer (exo commit "Add support for Nemotron sharding":
 * the NemotronHBlock stub holds a pre-mixer RMSNorm and the mixer; the MLX
 * RMSNorm stub: a weight over the feature dimension and an additive eps):
 *   block(x) = x + MoE(RMSNorm(x)),   RMSNorm(x)_i = x_i / sqrt(mean_i(x^2) + eps) * g_i
 * The norm's output takes the type of its weight, the layer's activation type
 * (auto-round PR, discussion of norm_dtype).  Precision (this library's
 * reading, fixed so that every implementation rounds x_norm the same way):
 * the sum of squares in fp64 (exact, so its order does not matter, while the
 * squares lie within a factor 2^37 of each other: a bf16 square has 16
 * significant bits, fp64 keeps 53); var = fp32(ss / d);
 * r = 1 / sqrt(var + eps) in fp32; n_i = (x_i * r) * g_i in fp32, rounded
 * once to the storage type (nearest even).  Rows [T, d] of dtype dt (fp32 or
 * bf16 bits); g [d] of the same dtype. */
void orc_rmsnorm(const void* x, int dt, const void* g, float eps, int64_t T, int64_t d,
                 void* out) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t i = 0; i < d; ++i) {
      double v = dt == ORC_F32 ? (double)((const float*)x)[t * d + i]
                               : orc_bf16_to_double(((const uint16_t*)x)[t * d + i]);
      ss += v * v;
    }
    float var = (float)(ss / (double)d);
    float r = 1.0f / sqrtf(var + eps);
    for (int64_t i = 0; i < d; ++i) {
      float xi, gi;
      if (dt == ORC_F32) {
        xi = ((const float*)x)[t * d + i];
        gi = ((const float*)g)[i];
      } else {
        xi = (float)orc_bf16_to_double(((const uint16_t*)x)[t * d + i]);
        gi = (float)orc_bf16_to_double(((const uint16_t*)g)[i]);
      }
      float n = (xi * r) * gi;
      if (dt == ORC_F32)
        ((float*)out)[t * d + i] = n;
      else
        ((uint16_t*)out)[t * d + i] = orc_bf16_from_double((double)n);
    }
  }
}

/* ---------------------------------------------------------------- router */

/* Selection for one token from its fp64 logits.  Writes k ascending expert
 * ids, their weights, and the smallest decision margin (how far the last
 * chosen group / expert lies above the best one left out; +inf if nothing
 * was left out). */
static void select_token(const orc_cfg* cfg, const double* logit, const float* bias,
                         int32_t* idx, double* w, double* margin, double* s, double* c,
                         double* gs, char* gsel, char* esel) {
  const int E = cfg->n_experts, G = cfg->n_group, Eg = E / G;
  const int tg = cfg->topk_group, k = cfg->top_k;
  for (int e = 0; e < E; ++e) {
    s[e] = 1.0 / (1.0 + exp(-logit[e]));
    c[e] = s[e] + (double)bias[e];
  }
  for (int g = 0; g < G; ++g) {
    if (Eg == 1) {
      gs[g] = c[g];
    } else {
      double b1 = -INFINITY, b2 = -INFINITY;
      for (int e = g * Eg; e < (g + 1) * Eg; ++e) {
        if (c[e] > b1) {
          b2 = b1;
          b1 = c[e];
        } else if (c[e] > b2) {
          b2 = c[e];
        }
      }
      gs[g] = b1 + b2;
    }
    gsel[g] = 0;
  }
  double m = INFINITY;
  double last_group = INFINITY;
  for (int r = 0; r < tg; ++r) {
    int best = -1;
    for (int g = 0; g < G; ++g)
      if (!gsel[g] && (best < 0 || gs[g] > gs[best])) best = g; /* '>' keeps the lower index */
    gsel[best] = 1;
    last_group = gs[best];
  }
  for (int g = 0; g < G; ++g)
    if (!gsel[g] && last_group - gs[g] < m) m = last_group - gs[g];

  for (int e = 0; e < E; ++e) esel[e] = 0;
  double last_expert = INFINITY;
  for (int r = 0; r < k; ++r) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (!gsel[e / Eg] || esel[e]) continue;
      if (best < 0 || c[e] > c[best]) best = e;
    }
    esel[best] = 1;
    last_expert = c[best];
  }
  for (int e = 0; e < E; ++e)
    if (gsel[e / Eg] && !esel[e] && last_expert - c[e] < m) m = last_expert - c[e];

  int j = 0;
  double denom = 0.0;
  for (int e = 0; e < E; ++e)
    if (esel[e]) {
      idx[j++] = e;
      denom += s[e];
    }
  for (j = 0; j < k; ++j) {
    double sj = s[idx[j]];
    w[j] = cfg->norm_topk_prob ? cfg->routed_scaling_factor * (sj / denom)
                               : cfg->routed_scaling_factor * sj;
  }
  *margin = m;
}

/* Routing for T tokens: topk_idx [T,k] int32, topk_w [T,k] fp64, margin [T],
 * and optionally the fp64 logits [T,E]. */
int orc_route(const orc_cfg* cfg, int64_t T, const void* x, const void* w_gate,
              const float* e_bias, int32_t* topk_idx, double* topk_w, double* margin,
              double* logits_out) {
  const int E = cfg->n_experts, d = cfg->hidden, G = cfg->n_group;
  if (G <= 0 || E % G || cfg->topk_group < 1 || cfg->topk_group > G || cfg->top_k < 1 ||
      cfg->top_k > cfg->topk_group * (E / G))
    return -1;
#pragma omp parallel
  {
    double* xa = (double*)malloc(sizeof(double) * d);
    double* l = (double*)malloc(sizeof(double) * E * 4 + sizeof(double) * G);
    char* flags = (char*)malloc(G + E);
#pragma omp for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
      widen_row(plain_mat(x, cfg->act_dtype), t, d, xa);
      for (int e = 0; e < E; ++e) l[e] = dot_row(xa, plain_mat(w_gate, cfg->act_dtype), e, d);
      if (logits_out)
        for (int e = 0; e < E; ++e) logits_out[t * E + e] = l[e];
      select_token(cfg, l, e_bias, topk_idx + t * cfg->top_k, topk_w + t * cfg->top_k,
                   margin + t, l + E, l + 2 * E, l + 3 * E, flags, flags + G);
    }
    free(xa);
    free(l);
    free(flags);
  }
  return 0;
}

/* -------------------------------------------------------------- one FFN */

/* h = relu(u)^2 held as the GEMM that reads it holds it (see modes above).
 * `hf` is fp32 scratch of length 2 * inter. */
static void hold_h(double* h, int64_t inter, int w_dtype, int mode, float* hf) {
  if (mode == ORC_EXACT) return;
  if (w_dtype == ORC_BF16 || w_dtype == ORC_FP4) {
    for (int64_t n = 0; n < inter; ++n) h[n] = orc_bf16_to_double(orc_bf16_from_double(h[n]));
  } else if (w_dtype == ORC_F32) {
    for (int64_t n = 0; n < inter; ++n) h[n] = (double)(float)h[n];
  } else {
    uint8_t* q = (uint8_t*)(hf + inter);
    float s;
    for (int64_t n = 0; n < inter; ++n) hf[n] = (float)h[n];
    orc_quantize_row(hf, inter, q, &s);
    for (int64_t n = 0; n < inter; ++n) h[n] = orc_e4m3_to_double(q[n]) * (double)s;
  }
}

/* out[c] = sum_n Wdown[c,n] * hold(relu(sum_i a_i Wup[n,i])^2), c < d */
static void ffn_one(const double* a, int64_t d, int64_t inter, orc_mat up, orc_mat down,
                    int mode, double* h, float* hf, double* out) {
  for (int64_t n = 0; n < inter; ++n) {
    double u = dot_row(a, up, n, d);
    double r = u > 0.0 ? u : 0.0;
    h[n] = r * r;
  }
  hold_h(h, inter, up.dt, mode, hf);
  for (int64_t c = 0; c < d; ++c) out[c] = dot_row(h, down, c, inter);
}

/* Matrix e of a stack of [rows, cols] matrices of dtype dt.  fp8: `scale`
 * holds one fp32 scale per row ([n_mats, rows]).  fp4: `bscale` holds the
 * E8M0 block scales ([n_mats, rows, cols / 32]). */
static orc_mat stack_mat(const void* w, int dt, const float* scale, const uint8_t* bscale,
                         int64_t e, int64_t rows, int64_t cols) {
  orc_mat m = plain_mat(w, dt);
  if (dt == ORC_FP4) {
    m.w = (const char*)w + (size_t)e * rows * (cols / 2);
    m.bscale = bscale + (size_t)e * rows * (cols / 32);
  } else {
    size_t esz = dt == ORC_F32 ? 4 : dt == ORC_BF16 ? 2 : 1;
    m.w = (const char*)w + (size_t)e * rows * cols * esz;
    if (dt == ORC_FP8) m.row_scale = scale + e * rows;
  }
  return m;
}

/* The activation row the routed GEMMs read: x as stored, or (fp8 routed
 * weights, as-configured mode) x quantised per token. */
static void routed_input(const orc_cfg* cfg, const void* x, int64_t t, int mode, double* xa,
                         double* xr, float* tmpf) {
  int64_t d = cfg->hidden;
  if (cfg->expert_dtype == ORC_FP8 && mode == ORC_AS_CONFIGURED) {
    uint8_t* q = (uint8_t*)(tmpf + d);
    float s;
    for (int64_t i = 0; i < d; ++i) tmpf[i] = (float)xa[i]; /* exact: x is bf16/fp32 */
    orc_quantize_row(tmpf, d, q, &s);
    for (int64_t i = 0; i < d; ++i) xr[i] = orc_e4m3_to_double(q[i]) * (double)s;
  } else {
    memcpy(xr, xa, sizeof(double) * d);
  }
  (void)x;
  (void)t;
}

/* FFN outputs for explicit (row, matrix) pairs: out[p] = FFN_{mat[p]}(a[row[p]]).
 * `a` is [a_rows, d] of dtype a_dtype; matrices are stacked [n_mats, inter, d]
 * and [n_mats, d, inter] of dtype w_dtype with their scales as stack_mat
 * reads them.  quant_a quantises each a row to e4m3 before the GEMMs. */
int orc_ffn_rows(int64_t d, int64_t inter, const void* a, int a_dtype, int64_t n_pairs,
                 const int32_t* row, const int32_t* mat, const void* w_up,
                 const float* w_up_scale, const uint8_t* w_up_bscale, const void* w_down,
                 const float* w_down_scale, const uint8_t* w_down_bscale, int w_dtype,
                 int quant_a, int mode, double* out) {
#pragma omp parallel
  {
    double* xa = (double*)malloc(sizeof(double) * d);
    double* xr = (double*)malloc(sizeof(double) * d);
    double* h = (double*)malloc(sizeof(double) * inter);
    float* hf = (float*)malloc(sizeof(float) * (inter + d) * 2 + 64);
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < n_pairs; ++p) {
      int64_t e = mat[p];
      widen_row(plain_mat(a, a_dtype), row[p], d, xa);
      if (quant_a) {
        uint8_t* q = (uint8_t*)(hf + d);
        float s;
        for (int64_t i = 0; i < d; ++i) hf[i] = (float)xa[i];
        orc_quantize_row(hf, d, q, &s);
        for (int64_t i = 0; i < d; ++i) xr[i] = orc_e4m3_to_double(q[i]) * (double)s;
      } else {
        memcpy(xr, xa, sizeof(double) * d);
      }
      ffn_one(xr, d, inter, stack_mat(w_up, w_dtype, w_up_scale, w_up_bscale, e, inter, d),
              stack_mat(w_down, w_dtype, w_down_scale, w_down_bscale, e, d, inter), mode, h, hf,
              out + p * d);
    }
    free(xa);
    free(xr);
    free(h);
    free(hf);
  }
  return 0;
}

/* ---------------------------------------------------------- whole layer */

/* y for the tokens listed in `tokens` (n_tok of them): y [n_tok, d] fp64,
 * plus their routing (topk_idx [n_tok,k], topk_w [n_tok,k], margin [n_tok]). */
int orc_forward(const orc_cfg* cfg, int64_t n_tok, const int64_t* tokens, const void* x,
                const void* w_gate, const float* e_bias, const void* w_up,
                const float* w_up_scale, const uint8_t* w_up_bscale, const void* w_down,
                const float* w_down_scale, const uint8_t* w_down_bscale, const void* ws_up,
                const uint8_t* ws_up_bscale, const void* ws_down, const uint8_t* ws_down_bscale,
                int mode, double* y, int32_t* topk_idx, double* topk_w, double* margin) {
  const int E = cfg->n_experts, G = cfg->n_group, k = cfg->top_k;
  const int64_t d = cfg->hidden, I = cfg->inter, Is = cfg->shared_inter;
  if (G <= 0 || E % G || cfg->topk_group < 1 || cfg->topk_group > G || k < 1 ||
      k > cfg->topk_group * (E / G))
    return -1;
  int64_t hmax = I > Is ? I : Is;
#pragma omp parallel
  {
    double* xa = (double*)malloc(sizeof(double) * d);
    double* xr = (double*)malloc(sizeof(double) * d);
    double* o = (double*)malloc(sizeof(double) * d);
    double* h = (double*)malloc(sizeof(double) * hmax);
    float* hf = (float*)malloc(sizeof(float) * (hmax + d) * 2 + 64);
    double* l = (double*)malloc(sizeof(double) * (E * 4 + G));
    char* flags = (char*)malloc(G + E);
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < n_tok; ++p) {
      int64_t t = tokens[p];
      double* yt = y + p * d;
      int32_t* it = topk_idx + p * k;
      double* wt = topk_w + p * k;
      widen_row(plain_mat(x, cfg->act_dtype), t, d, xa);
      for (int e = 0; e < E; ++e) l[e] = dot_row(xa, plain_mat(w_gate, cfg->act_dtype), e, d);
      select_token(cfg, l, e_bias, it, wt, margin + p, l + E, l + 2 * E, l + 3 * E, flags,
                   flags + G);
      routed_input(cfg, x, t, mode, xa, xr, hf);
      for (int64_t c = 0; c < d; ++c) yt[c] = 0.0;
      for (int j = 0; j < k; ++j) {
        int64_t e = it[j];
        const int dt = cfg->expert_dtype;
        ffn_one(xr, d, I, stack_mat(w_up, dt, w_up_scale, w_up_bscale, e, I, d),
                stack_mat(w_down, dt, w_down_scale, w_down_bscale, e, d, I), mode, h, hf, o);
        for (int64_t c = 0; c < d; ++c) yt[c] += wt[j] * o[c];
      }
      if (Is > 0) {
        const int sdt = cfg->shared_dtype;
        ffn_one(xa, d, Is, stack_mat(ws_up, sdt, NULL, ws_up_bscale, 0, Is, d),
                stack_mat(ws_down, sdt, NULL, ws_down_bscale, 0, d, Is), mode, h, hf, o);
        for (int64_t c = 0; c < d; ++c) yt[c] += o[c];
      }
    }
    free(xa);
    free(xr);
    free(o);
    free(h);
    free(hf);
    free(l);
    free(flags);
  }
  return 0;
}
