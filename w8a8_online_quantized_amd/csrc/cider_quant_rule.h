// The element rule of the online symmetric quantizer, shared by the
// standalone quantization kernels and the GEMV kernel that quantizes its own
// activations (so both produce the same codes by construction).
//
// Rule (one group = a row, or gs consecutive elements of a row), after the
// Cider README, section "量化" (symmetric INT8 per-token activations):
//   s = max|v| / qmax              (fp32, one correctly rounded division)
//   q = clamp(rint(v / s), +-qmax) (v / s one correctly rounded fp32 division,
//                                   rint = ties to even); s == 0 -> q = 0.
// Each code is first formed from r = v * fl(1/s): |r - fl(v/s)| <= 3 * 2^-24 *
// 128 < 2.3e-5, so when r is at least 2^-13 away from every half-integer both
// round to the same integer; only the rare remaining elements take the exact
// division. The result is bit-identical to always dividing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cider {

constexpr float kNearHalf = 0.4998779296875f;   // 0.5 - 2^-13

// max |v| of 8 fp16 (or bf16) values as a 15-bit pattern: the magnitudes of
// both formats compare like their bit patterns (finite inputs).
__device__ __forceinline__ uint32_t abs_max_bits(uint4 v) {
  uint32_t m = 0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = w[i] & 0x7FFF7FFFu;
    m = max(m, max(a & 0xFFFFu, a >> 16));
  }
  return m;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)bits);
}

// The fp32 value of a 16-bit element (low 16 bits of `bits`): fp16, or bf16
// (the top half of an fp32 pattern). Exact either way.
template <bool BF>
__device__ __forceinline__ float elem_to_float(uint32_t bits) {
  if constexpr (BF) return __builtin_bit_cast(float, (bits & 0xFFFFu) << 16);
  else return half_bits_to_float(bits & 0xFFFFu);
}

// Code of one element given the group scale s (> 0) and inv = fl(1/s).
__device__ __forceinline__ int code_of(float v, float s, float inv, float qmax) {
  const float r = v * inv;
  float t = __builtin_rintf(r);
  if (__builtin_fabsf(r - t) > kNearHalf) t = __builtin_rintf(v / s);
  t = __builtin_fminf(__builtin_fmaxf(t, -qmax), qmax);
  return (int)t;
}

// 8 codes of one 16-byte chunk (8 fp16, or bf16 when BF, values).
template <bool BF = false>
__device__ __forceinline__ void codes_of_chunk(uint4 v, float s, float inv, float qmax, int q[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[2 * i] = code_of(elem_to_float<BF>(w[i]), s, inv, qmax);
    q[2 * i + 1] = code_of(elem_to_float<BF>(w[i] >> 16), s, inv, qmax);
  }
}

}  // namespace cider
