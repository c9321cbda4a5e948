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

// 8 codes of one 16-byte chunk (8 fp16, or bf16 when BF, values) as int8
// bytes, element j in byte j of the result, by the rule above.
// The integer is rounded by adding 1.5 * 2^23: for |r| < 2^22 the sum lands
// in [2^23, 2^24), where the fp32 spacing is 1, so the round-to-nearest-even
// addition yields rint(r) (ties to even, as the addend is even) in the low
// mantissa bits, and the low byte of the pattern is rint(r) as a two's
// complement byte. The near-half test runs per element but the exact-division
// path is entered once per chunk, only when some lane needs it.
// CLAMP: the scale may lie below max|v| / qmax (clipped scales), so r is
// clamped to +-qmax first (clamping to integer bounds commutes with rint).
// With min-max scales (s = fl(amax / qmax), amax = max|v| of the group)
// |v * fl(1/s)| <= qmax * (1 + 3 * 2^-24) < qmax + 1/2 and |fl(v / s)| <=
// qmax * (1 + 2^-24), so the clamp cannot act and is left out. A scale whose
// reciprocal is not finite (bf16 groups below ~3.7e-37) sends every element
// through the division.
template <bool BF, bool CLAMP>
__device__ __forceinline__ uint2 code_bytes_of_chunk(uint4 v, float s, float inv, float qmax) {
  constexpr float kMagic = 12582912.0f;   // 1.5 * 2^23
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float x[8], r[8], t[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = elem_to_float<BF>(w[i]);
    x[2 * i + 1] = elem_to_float<BF>(w[i] >> 16);
  }
  float worst = __builtin_isfinite(inv) ? 0.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    r[j] = x[j] * inv;
    if constexpr (CLAMP) r[j] = __builtin_fminf(__builtin_fmaxf(r[j], -qmax), qmax);
    t[j] = r[j] + kMagic;
    worst = __builtin_fmaxf(worst, __builtin_fabsf((t[j] - kMagic) - r[j]));
  }
  if (worst > kNearHalf) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (!(__builtin_fabsf((t[j] - kMagic) - r[j]) <= kNearHalf) || !__builtin_isfinite(inv))
        t[j] = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(x[j] / s), -qmax), qmax) + kMagic;
    }
  }
  uint32_t b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = __builtin_bit_cast(uint32_t, t[j]);
  uint2 o;
  o.x = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
  o.y = __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u) | __builtin_amdgcn_perm(b[7], b[6], 0x04000c0cu);
  return o;
}

}  // namespace cider
