// Online symmetric quantization of fp16 rows to int8 (or packed int4) codes.
//
// Follows the Cider README, section "架构 / Metal Kernel 流水线" (the first
// prefill step turns fp16 activations into int8 codes plus one scale per
// token) and section "量化" (symmetric INT8 per-token activations; symmetric
// INT8 or zero-point-8 INT4 weights). Per-group scales (section "W8A8 量化粒度",
// gs = 64 / 128) use the same rule on each run of gs elements along K.
//
// The element rule (scale, codes) is in cider_quant_rule.h.
//
// HBM-bound: 2 bytes read, 1 (or 0.5) byte written per element. One wave owns
// one row; each lane owns 16-byte chunks (8 fp16) at a 64-chunk stride, so a
// wave load instruction covers 1 KiB of contiguous row. The row stays in
// registers between the max pass and the code pass.
//
// The division v / s costs a ~10-instruction correctly rounded sequence; with
// 8 elements per chunk it would make the kernel ALU-bound, hence the
// reciprocal-first form of the rule's code_of.
#include "cider_internal.h"
#include "cider_quant_rule.h"

namespace cider {
namespace {

constexpr int kWaves = 4;                 // waves (rows) per workgroup

// Stores the 8 code bytes of one chunk (element j in byte j): as int8, or as
// int4 nibbles (code + 8, low nibble of byte b = even k, high = odd k).
__device__ __forceinline__ void store_codes(void* q, int64_t row, int64_t K, int chunk, bool pack4,
                                            uint2 c) {
  if (!pack4) {
    *reinterpret_cast<uint2*>(static_cast<int8_t*>(q) + row * K + (int64_t)chunk * 8) = c;
  } else {
    // the low nibble of a two's complement code in [-8, 7], xor 8, is code + 8
    uint32_t o = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) o |= ((((j < 4 ? c.x : c.y) >> (8 * (j & 3))) & 0xFu) ^ 0x8u) << (4 * j);
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(q) + row * (K / 2) + (int64_t)chunk * 4) = o;
  }
}

// Row held in registers: CPL = 16-byte chunks per lane. WPR = 1: one wave
// per row (kWaves rows per workgroup), lane L owning chunks L + 64i. WPR = 4:
// one workgroup of 4 waves per row segment (long rows), wave w owning chunks
// 64w + L + 256i, so each wave holds a quarter of the row in a quarter of the
// registers and more waves stay resident to overlap one row's loads with
// another's codes; the row max then goes through LDS.
// GS = 0 (one scale per row; the whole row, K <= 8 * 64 * WPR * CPL, is one
// segment) or 64 / 128 (groups never straddle a segment, so long rows are
// split into segments of kSegChunks chunks along gridDim.y; a group's chunks
// are consecutive lanes of one wave either way).
constexpr int kSegChunks = 64 * 32;
constexpr int kWgMinChunks = 256;   // K >= 2048

template <int CPL, int GS, bool BF, int WPR>
__global__ __launch_bounds__(64 * kWaves) void quant_rows_reg(const uint4* __restrict__ x, int64_t R,
                                                              int64_t K, float qmax, bool pack4,
                                                              void* __restrict__ q,
                                                              float* __restrict__ s) {
  static_assert(WPR == 1 || WPR == kWaves, "one row per wave or per workgroup");
  static_assert(64 * WPR * CPL <= kSegChunks, "a segment fits the registers");
  constexpr int kStride = 64 * WPR;                     // chunks between a lane's slots
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = WPR == 1 ? (int64_t)blockIdx.x * kWaves + wave : (int64_t)blockIdx.x;
  if (row >= R) return;                                 // uniform per workgroup when WPR > 1
  const int C = (int)(K / 8);
  const int c0 = (int)blockIdx.y * kSegChunks;          // first chunk of this segment
  const int cend = min(C, c0 + kSegChunks);
  const int cl = c0 + (WPR == 1 ? lane : 64 * wave + lane);   // this lane's first chunk
  const uint4* xr = x + row * C;

  uint4 v[CPL];
  uint32_t m[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = cl + kStride * i;
    v[i] = c < cend ? xr[c] : make_uint4(0, 0, 0, 0);
    m[i] = abs_max_bits(v[i]);
  }

  if constexpr (GS == 0) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < CPL; ++i) a = max(a, m[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off));
    if constexpr (WPR > 1) {
      __shared__ uint32_t red[WPR];
      if (lane == 0) red[wave] = a;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < WPR; ++w) a = max(a, red[w]);
    }
    const float amax = elem_to_float<BF>(a);
    const float sc = amax / qmax;
    if (threadIdx.x == 0 || (WPR == 1 && lane == 0)) s[row] = sc;
    const float inv = 1.0f / sc;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = cl + kStride * i;
      if (c < cend) {
        const uint2 cq = sc != 0.0f ? code_bytes_of_chunk<BF, false>(v[i], sc, inv, qmax) : make_uint2(0, 0);
        store_codes(q, row, K, c, pack4, cq);
      }
    }
  } else {
    constexpr int kCpg = GS / 8;   // chunks per group: 8 or 16 lanes
    const int G = (int)(K / GS);
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      uint32_t a = m[i];
#pragma unroll
      for (int off = kCpg / 2; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off));
      const int c = cl + kStride * i;
      if (c < cend) {
        const float amax = elem_to_float<BF>(a);
        const float sc = amax / qmax;
        if ((lane & (kCpg - 1)) == 0) s[row * G + c / kCpg] = sc;
        const float inv = 1.0f / sc;
        const uint2 cq = sc != 0.0f ? code_bytes_of_chunk<BF, false>(v[i], sc, inv, qmax) : make_uint2(0, 0);
        store_codes(q, row, K, c, pack4, cq);
      }
    }
  }
}

// Rows longer than the register path holds (per-row scale only): one
// workgroup per row reads the row twice, first for max|v|, then for codes.
template <bool BF>
__global__ __launch_bounds__(256) void quant_rows_two_pass(const uint4* __restrict__ x, int64_t K,
                                                           float qmax, bool pack4, void* __restrict__ q,
                                                           float* __restrict__ s) {
  __shared__ uint32_t red[4];
  const int64_t row = blockIdx.x;
  const int C = (int)(K / 8);
  const uint4* xr = x + row * C;
  uint32_t a = 0;
  for (int c = threadIdx.x; c < C; c += 256) a = max(a, abs_max_bits(xr[c]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = max(max(red[0], red[1]), max(red[2], red[3]));
  const float sc = elem_to_float<BF>(a) / qmax;
  if (threadIdx.x == 0) s[row] = sc;
  const float inv = 1.0f / sc;
  for (int c = threadIdx.x; c < C; c += 256) {
    const uint2 cq = sc != 0.0f ? code_bytes_of_chunk<BF, false>(xr[c], sc, inv, qmax) : make_uint2(0, 0);
    store_codes(q, row, K, c, pack4, cq);
  }
}

// Rows whose length is not a multiple of 8 elements (per-row scale, any
// K >= 1; even K for int4): a row then starts only 2-byte aligned, so its
// elements are loaded one at a time. One wave per row: the max pass, then
// 8-element chunks (padded with zeros past K, which give code 0 and are not
// stored) through the same element rule, stored byte by byte.
template <bool BF>
__global__ __launch_bounds__(64 * kWaves) void quant_rows_ragged(const uint16_t* __restrict__ x, int64_t R,
                                                                  int64_t K, float qmax, bool pack4,
                                                                  void* __restrict__ q, float* __restrict__ s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave;
  if (row >= R) return;
  const uint16_t* xr = x + row * K;
  uint32_t a = 0;
  for (int64_t k = lane; k < K; k += 64) a = max(a, (uint32_t)(xr[k] & 0x7FFFu));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off));
  const float sc = elem_to_float<BF>(a) / qmax;
  if (lane == 0) s[row] = sc;
  const float inv = 1.0f / sc;
  const int64_t C = (K + 7) / 8;
  for (int64_t c = lane; c < C; c += 64) {
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (8 * c + j < K) w[j >> 1] |= (uint32_t)xr[8 * c + j] << (16 * (j & 1));
    const uint2 cq =
        sc != 0.0f ? code_bytes_of_chunk<BF, false>(make_uint4(w[0], w[1], w[2], w[3]), sc, inv, qmax) : make_uint2(0, 0);
    if (!pack4) {
      int8_t* dst = static_cast<int8_t*>(q) + row * K + 8 * c;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (8 * c + j < K) dst[j] = (int8_t)(((j < 4 ? cq.x : cq.y) >> (8 * (j & 3))) & 0xFFu);
    } else {
      // byte b of the chunk holds codes 2b (low nibble) and 2b + 1, each + 8
      uint8_t* dst = static_cast<uint8_t*>(q) + row * (K / 2) + 4 * c;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (8 * c + 2 * b >= K) break;
        const uint32_t word = b < 2 ? cq.x : cq.y;
        const uint32_t lo = (word >> (16 * (b & 1))) & 0xFu, hi = (word >> (16 * (b & 1) + 8)) & 0xFu;
        dst[b] = (uint8_t)((lo ^ 0x8u) | ((hi ^ 0x8u) << 4));
      }
    }
  }
}

// Percentile-clipped scales (the README's notes section names a percentile
// rule, clip_percentile=99.9, beside the default min-max): one workgroup per
// group (a row, or gs elements of it). The clip threshold is the percentile of
// the group's magnitudes by linear interpolation between the order statistics
// i = floor(h) and j = min(i + 1, n - 1), h = (n - 1) * (percentile / 100):
// t = a_i + (h - i) * (a_j - a_i), each step one rounded fp64 operation, then
// rounded to fp32; s = t / qmax and the codes follow the element rule, so
// magnitudes above t saturate. a_i and a_j come from a two-level radix select
// over the 15-bit magnitude patterns of fp16 (which order like the values):
// a 256-bin histogram of the high 8 bits finds each rank's bucket, a 128-bin
// histogram of the low 7 bits inside it the exact pattern. The group is read
// three times (two histograms, then the codes); weight quantization is offline.
template <bool BF>
__global__ __launch_bounds__(256) void quant_rows_clip(const uint4* __restrict__ x, int64_t K, int n, int G,
                                                       double pfrac, float qmax, bool pack4,
                                                       void* __restrict__ q, float* __restrict__ s) {
  __shared__ uint32_t hist_hi[256];
  __shared__ uint32_t hist_lo[2][128];
  __shared__ int pick[4];        // bucket and rank within it, for ranks i and j
  __shared__ float scale;
  const int64_t row = blockIdx.x / G;
  const int g = (int)(blockIdx.x % G);
  const int C = n / 8;                                   // 16-byte chunks in the group
  const uint4* xg = x + (row * K + (int64_t)g * n) / 8;

  const double h = (double)(n - 1) * pfrac;
  const int i = (int)__builtin_floor(h);
  const int j = min(i + 1, n - 1);

  for (int b = threadIdx.x; b < 256; b += 256) hist_hi[b] = 0;
  if (threadIdx.x < 128) hist_lo[0][threadIdx.x] = hist_lo[1][threadIdx.x] = 0;
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += 256) {
    const uint4 v = xg[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) atomicAdd(&hist_hi[((w[e >> 1] >> (16 * (e & 1))) & 0x7FFFu) >> 7], 1u);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t cum = 0;
    int bi = -1, bj = -1;
    for (int b = 0; b < 256; ++b) {
      const uint32_t next = cum + hist_hi[b];
      if (bi < 0 && (uint32_t)i < next) { bi = b; pick[1] = i - (int)cum; }
      if (bj < 0 && (uint32_t)j < next) { bj = b; pick[3] = j - (int)cum; }
      cum = next;
    }
    pick[0] = bi;
    pick[2] = bj;
  }
  __syncthreads();
  const int bi = pick[0], bj = pick[2];
  for (int c = threadIdx.x; c < C; c += 256) {
    const uint4 v = xg[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t u = (w[e >> 1] >> (16 * (e & 1))) & 0x7FFFu;
      if ((int)(u >> 7) == bi) atomicAdd(&hist_lo[0][u & 127], 1u);
      if ((int)(u >> 7) == bj) atomicAdd(&hist_lo[1][u & 127], 1u);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t sel[2];
    for (int k = 0; k < 2; ++k) {
      const uint32_t rank = (uint32_t)pick[2 * k + 1];
      uint32_t cum = 0, lo = 0;
      for (int b = 0; b < 128; ++b) {
        const uint32_t next = cum + hist_lo[k][b];
        if (rank < next) { lo = (uint32_t)b; break; }
        cum = next;
      }
      sel[k] = ((uint32_t)pick[2 * k] << 7) | lo;
    }
    const double ai = (double)elem_to_float<BF>(sel[0]), aj = (double)elem_to_float<BF>(sel[1]);
    double prod = (h - (double)i) * (aj - ai);
    asm("" : "+v"(prod));                 // keep the product and the sum two roundings
    const float t = (float)(ai + prod);
    const float sc = t / qmax;
    s[row * G + g] = sc;
    scale = sc;
  }
  __syncthreads();
  const float sc = scale;
  const float inv = 1.0f / sc;
  for (int c = threadIdx.x; c < C; c += 256) {
    const uint2 cq = sc != 0.0f ? code_bytes_of_chunk<BF, true>(xg[c], sc, inv, qmax) : make_uint2(0, 0);
    store_codes(q, row, K, g * C + c, pack4, cq);
  }
}

template <int GS, bool BF, int WPR>
hipError_t launch_reg(int cpl, int segs, const uint4* x, int64_t R, int64_t K, float qmax, bool pack4,
                      void* q, float* s, hipStream_t st) {
  const int64_t blocks = WPR == 1 ? (R + kWaves - 1) / kWaves : R;
  const dim3 grid((unsigned)blocks, (unsigned)segs), block(64 * kWaves);
  switch (cpl) {
    case 1: quant_rows_reg<1, GS, BF, WPR><<<grid, block, 0, st>>>(x, R, K, qmax, pack4, q, s); break;
    case 2: quant_rows_reg<2, GS, BF, WPR><<<grid, block, 0, st>>>(x, R, K, qmax, pack4, q, s); break;
    case 3: quant_rows_reg<3, GS, BF, WPR><<<grid, block, 0, st>>>(x, R, K, qmax, pack4, q, s); break;
    case 4: quant_rows_reg<4, GS, BF, WPR><<<grid, block, 0, st>>>(x, R, K, qmax, pack4, q, s); break;
    case 5: quant_rows_reg<5, GS, BF, WPR><<<grid, block, 0, st>>>(x, R, K, qmax, pack4, q, s); break;
    case 8: quant_rows_reg<8, GS, BF, WPR><<<grid, block, 0, st>>>(x, R, K, qmax, pack4, q, s); break;
    case 16:
      if constexpr (WPR == 1) { quant_rows_reg<16, GS, BF, 1><<<grid, block, 0, st>>>(x, R, K, qmax, pack4, q, s); break; }
      [[fallthrough]];
    default:
      if constexpr (WPR == 1) quant_rows_reg<32, GS, BF, 1><<<grid, block, 0, st>>>(x, R, K, qmax, pack4, q, s);
      else return hipErrorInvalidValue;
      break;
  }
  return hipGetLastError();
}

template <bool BF>
hipError_t launch_quant_t(const void* x, int64_t R, int64_t K, int group_size, int qmax, void* q, float* s,
                          hipStream_t stream) {
  const uint4* xv = static_cast<const uint4*>(x);
  const bool pack4 = qmax == 7;
  const float fq = (float)qmax;
  if (K % 8 != 0) {   // per-row scales only (group sizes divide K)
    const dim3 grid((unsigned)((R + kWaves - 1) / kWaves)), block(64 * kWaves);
    quant_rows_ragged<BF><<<grid, block, 0, stream>>>(static_cast<const uint16_t*>(x), R, K, fq, pack4, q, s);
    return hipGetLastError();
  }
  const int64_t C = K / 8;
  if (group_size == 0 && C > kSegChunks) {
    quant_rows_two_pass<BF><<<dim3((unsigned)R), dim3(256), 0, stream>>>(xv, K, fq, pack4, q, s);
    return hipGetLastError();
  }
  const int64_t segs = (C + kSegChunks - 1) / kSegChunks;
  const int64_t per_seg = segs > 1 ? kSegChunks : C;
  // segments of >= kWgMinChunks chunks (K >= 2048): a workgroup per segment
  const bool wg = per_seg >= kWgMinChunks;
  const int lanes = wg ? 64 * kWaves : 64;
  // chunks per lane: the smallest of 1, 2, 3, 4, 5, 8, 16, 32 that covers the
  // segment (3 and 5 fit K = 6144 and 10240 exactly in a workgroup, so no
  // register slots sit idle)
  int cpl = 1;
  while (lanes * cpl < per_seg) cpl = cpl < 5 ? cpl + 1 : (cpl == 5 ? 8 : cpl * 2);
  switch (group_size) {
    case 0: return wg ? launch_reg<0, BF, kWaves>(cpl, 1, xv, R, K, fq, pack4, q, s, stream)
                      : launch_reg<0, BF, 1>(cpl, 1, xv, R, K, fq, pack4, q, s, stream);
    case 64: return wg ? launch_reg<64, BF, kWaves>(cpl, (int)segs, xv, R, K, fq, pack4, q, s, stream)
                       : launch_reg<64, BF, 1>(cpl, (int)segs, xv, R, K, fq, pack4, q, s, stream);
    default: return wg ? launch_reg<128, BF, kWaves>(cpl, (int)segs, xv, R, K, fq, pack4, q, s, stream)
                       : launch_reg<128, BF, 1>(cpl, (int)segs, xv, R, K, fq, pack4, q, s, stream);
  }
}

}  // namespace

hipError_t launch_quant_rows_clip(const void* x, int64_t R, int64_t K, int group_size, int qmax,
                                  double percentile, void* q, float* s, hipStream_t stream, bool bf16) {
  const int n = group_size ? group_size : (int)K;
  const int G = (int)(K / n);
  const dim3 grid((unsigned)(R * G)), block(256);
  const uint4* xv = static_cast<const uint4*>(x);
  if (bf16)
    quant_rows_clip<true><<<grid, block, 0, stream>>>(xv, K, n, G, percentile / 100.0, (float)qmax, qmax == 7, q, s);
  else
    quant_rows_clip<false><<<grid, block, 0, stream>>>(xv, K, n, G, percentile / 100.0, (float)qmax, qmax == 7, q, s);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* x, int64_t R, int64_t K, int group_size, int qmax, void* q,
                             float* s, hipStream_t stream, bool bf16) {
  return bf16 ? launch_quant_t<true>(x, R, K, group_size, qmax, q, s, stream)
              : launch_quant_t<false>(x, R, K, group_size, qmax, q, s, stream);
}

}  // namespace cider
