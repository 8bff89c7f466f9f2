// common.hpp -- device helpers shared by the gfx950 kernels of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

enum Kind : int { K_F32 = 0, K_BF16 = 1, K_FP8 = 2, K_FP4 = 3 };

constexpr int WAVE = 64;

// ---------------------------------------------------------------- numbers

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two IEEE binary32 values -> two bfloat16 (a in the low half), each rounded
// to nearest, ties to even: one v_cvt_pk_bf16_f32 (gfx950's conversion rounds
// as the mode register says, nearest even by default).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// IEEE binary32 -> bfloat16, round to nearest, ties to even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f));
}

// ---------------------------------------------------------------- waves

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << lane_id()) - 1;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Order LDS writes before later LDS reads of other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave-wide arg-max: larger value wins, equal values go to the smaller index.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) {
    float ov = __shfl_xor(v, off);
    int oi = __shfl_xor(i, off);
    if (ov > v || (ov == v && oi < i)) {
      v = ov;
      i = oi;
    }
  }
}

// ---------------------------------------------------------------- MFMA

// D += A * B over one 16x16 output block.  A and B fragments: lane l holds
// row/column l % 16 and a contiguous run of K for the lane group l / 16
// (bf16: 8 values, f32: 4 values used by four 16x16x4 steps, fp8: 32 values).
// D: lane l holds column l % 16, rows 4 * (l / 16) .. +3.
__device__ __forceinline__ f32x4_t mfma_bf16(const i32x4_t a, const i32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32x4(const i32x4_t a, const i32x4_t b, f32x4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[0]), __int_as_float(b[0]), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[1]), __int_as_float(b[1]), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[2]), __int_as_float(b[2]), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[3]), __int_as_float(b[3]), c, 0, 0, 0);
  return c;
}

// fp8 e4m3 x e4m3 (format selectors 0, 0), no block scaling.
__device__ __forceinline__ f32x4_t mfma_fp8(const i32x8_t a, const i32x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

}  // namespace moe
