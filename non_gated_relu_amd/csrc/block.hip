// block.hip -- the RMSNorm before the layer in its block.
//
// The block around the MoE mixer (exo commit "Add support for Nemotron
// sharding": the NemotronHBlock stub holds a pre-mixer RMSNorm and the
// mixer; the MLX RMSNorm stub: a weight over the feature dimension and an
// additive eps) computes block(x) = x + MoE(RMSNorm(x)).  The norm's output
// takes its weight's type, the layer's activation type (auto-round PR
// "feat: support Nemotron-H / Nemotron-Cascade-2", discussion of
// norm_dtype).  The residual add happens in the combine kernel, before its
// single rounding.
//
// Precision, fixed so that every implementation rounds the normalised rows
// the same way: the sum of squares in fp64 (exact for bf16 rows, whose
// squares have 16 significant bits, while they lie within a factor 2^37 of
// each other: then the order of the sum does not matter); var = fp32(ss / d);
// r = 1 / sqrt(var + eps) in fp32 with correctly rounded division and square
// root; n_i = (x_i * r) * g_i in fp32, rounded once (nearest even) to the
// activation type.
#include "internal.hpp"

namespace moe {

namespace {

constexpr int NORM_WAVES = 4;  // rows per workgroup, one wave each

// One wave per row; each lane takes 16-byte chunks c = lane, lane + 64, ...
template <bool BF16>
__global__ __launch_bounds__(NORM_WAVES * WAVE) void rmsnorm_kernel(NormArgs p) {
  const int64_t row = int64_t(blockIdx.x) * NORM_WAVES + threadIdx.x / WAVE;
  if (row >= p.tokens) return;
  const int lane = lane_id();
  constexpr int EPC = BF16 ? 8 : 4;  // elements per 16-byte chunk
  const int chunks = p.hidden / EPC;
  const char* xr = static_cast<const char*>(p.x) + row * int64_t(p.hidden) * (BF16 ? 2 : 4);
  auto widen = [&](const i32x4_t v, float (&f)[EPC]) {
    if constexpr (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f[2 * q] = __uint_as_float(uint32_t(v[q]) << 16);
        f[2 * q + 1] = __uint_as_float(uint32_t(v[q]) & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = __int_as_float(v[q]);
    }
  };
  double ss = 0.0;
  for (int c = lane; c < chunks; c += WAVE) {
    float f[EPC];
    widen(*reinterpret_cast<const i32x4_t*>(xr + c * 16), f);
#pragma unroll
    for (int q = 0; q < EPC; ++q) ss += double(f[q]) * double(f[q]);
  }
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  ss = __shfl(ss, 0);  // one value for every lane, also when the sum was not exact (fp32 rows)
  const float var = static_cast<float>(ss / double(p.hidden));
  const float r = 1.0f / sqrtf(var + p.eps);
  const char* gr = static_cast<const char*>(p.weight);
  char* orow = static_cast<char*>(p.out) + row * int64_t(p.hidden) * (BF16 ? 2 : 4);
  for (int c = lane; c < chunks; c += WAVE) {
    float f[EPC], g[EPC];
    widen(*reinterpret_cast<const i32x4_t*>(xr + c * 16), f);
    widen(*reinterpret_cast<const i32x4_t*>(gr + c * 16), g);
    i32x4_t o;
    if constexpr (BF16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = (f[2 * q] * r) * g[2 * q];
        const float hi = (f[2 * q + 1] * r) * g[2 * q + 1];
        o[q] = int(pack_bf16x2(lo, hi));
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = __float_as_int((f[q] * r) * g[q]);
    }
    *reinterpret_cast<i32x4_t*>(orow + c * 16) = o;
  }
}

}  // namespace

hipError_t launch_rmsnorm(const NormArgs& p, bool bf16, hipStream_t stream, Timing t) {
  if (p.tokens <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((p.tokens + NORM_WAVES - 1) / NORM_WAVES));
  const dim3 block(NORM_WAVES * WAVE);
  if (bf16) return launch_k(rmsnorm_kernel<true>, grid, block, stream, t, p);
  return launch_k(rmsnorm_kernel<false>, grid, block, stream, t, p);
}

}  // namespace moe
