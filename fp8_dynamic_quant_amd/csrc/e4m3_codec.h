// OCP E4M3 encoding of bf16 data with one scale per row, shared by the quantization kernels.
// The arithmetic and its exactness argument are described in quantize.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace dq {
namespace codec {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr float kE4M3Max = 448.0f;
constexpr float kFltMinNormal = 1.17549435082228750797e-38f;
constexpr float kTinyAmax = 0x1p-60f;  // rows below this work on x 2^64 and scale 2^64

__device__ __forceinline__ uint32_t absmax_pk(uint32_t acc, uint32_t w) {
  u16x2 a = __builtin_bit_cast(u16x2, acc);
  u16x2 b = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ uint32_t absmax4(uint32_t acc, uint4 v) {
  acc = absmax_pk(acc, v.x);
  acc = absmax_pk(acc, v.y);
  acc = absmax_pk(acc, v.z);
  return absmax_pk(acc, v.w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two dwords of bf16 (4 values) -> four E4M3 codes in one dword.
//   kind 0: Markstein quotient (y = fl32(1 / ss), ss = scale k, k = 1 or 2^64, xs = x k);
//   kind 1: IEEE division by a subnormal scale, clamped to +-448.
template <int kKind, bool kScaled>
__device__ __forceinline__ uint32_t encode4(uint32_t w0, uint32_t w1, float ss, float y) {
  float v[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (kKind == 0) {
      const float xs = kScaled ? __fmul_rn(v[i], 0x1p64f) : v[i];
      const float q = __fmul_rn(xs, y);
      const float r = __builtin_fmaf(-q, ss, xs);
      // the chain is odd in x except at x = -0 (it gives +0): take the sign from x
      v[i] = __builtin_copysignf(__builtin_fmaf(r, y, q), v[i]);
    } else {
      v[i] = fminf(fmaxf(v[i] / ss, -kE4M3Max), kE4M3Max);
    }
  }
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], r, true);
  return (uint32_t)r;
}

// Codes of an all-zero row: the sign bit of each bf16 moved to bit 7 of its byte.
__device__ __forceinline__ uint32_t signs4(uint32_t w0, uint32_t w1) {
  return ((w0 >> 8) & 0x80u) | ((w0 >> 16) & 0x8000u) | ((w1 << 8) & 0x800000u) |
         (w1 & 0x80000000u);
}

template <int kKind, bool kScaled>
__device__ __forceinline__ uint2 encode8(uint4 v, float ss, float y) {
  return make_uint2(encode4<kKind, kScaled>(v.x, v.y, ss, y),
                    encode4<kKind, kScaled>(v.z, v.w, ss, y));
}

__device__ __forceinline__ uint2 signs8(uint4 v) {
  return make_uint2(signs4(v.x, v.y), signs4(v.z, v.w));
}

}  // namespace codec
}  // namespace dq
