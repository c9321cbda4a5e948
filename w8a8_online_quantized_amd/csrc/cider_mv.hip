// Decode matrix-vector product: fp16 activations times int8 weights dequantized
// on the fly, with no activation quantization.
//
// Follows the Cider README, section "架构 / Metal Kernel 流水线": in decode
// (M = 1) the int8_mv kernel multiplies the activation vector by the int8
// weights, dequantizing them as it goes; the README's file list names a
// per-channel and a per-group MV kernel. Here:
//   y[m, n] = fp16( sum_k x[m, k] * w_q[n, k] * s_w[n, g(k)] ),  1 <= M <= 4,
// with per-channel (one s_w per row) or per-group (gs 64 / 128) scales.
//
// The weight stream is the whole cost (N*K bytes), so the kernel is shaped for
// HBM: a block owns RI = 8, 4 or 2 weight rows (chosen so that the grid
// covers the 256 CUs evenly); a wave instruction loads RI rows x (1024 / RI)
// contiguous bytes (lane L: 16 bytes of row L / (64 / RI)); the block's four
// waves take alternate steps of each row, a batch of steps in flight at a
// time, the next batch loading while the current one is consumed. The
// activations (and per-group, the block's scales) are DMA'd into LDS once per
// block before the first weight batch (when they fit in 64 KiB); otherwise
// each lane reads its activation chunks through the caches next to each
// weight chunk.
//
// Arithmetic: int8 codes become fp16 exactly (bias by 128, place the byte
// under the fp16 exponent of 1024 with v_perm_b32, subtract 1152 in packed
// fp16), and v_dot2_f32_f16 accumulates code * x pairs in fp32 (the products of
// an fp16 activation and an 8-bit code are exact in fp32). Per-channel keeps one
// fp32 sum per lane and applies s_w once at the end (fp32 product, then fp16);
// per-group forms each lane's 16-code partial and adds partial * s_w[n, g]
// (one group per partial: gs >= 16). The lanes of a row are summed by a
// fixed butterfly and the waves in wave order, so results are
// deterministic.
#include "cider_internal.h"

namespace cider {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mv_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: raw buffer, 32-bit data format (gfx9 family)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Four signed int8 codes (one dword, K order) -> two fp16 pairs (codes 0,1 and
// 2,3). u = code + 128 in [1, 255]; the fp16 with bits 0x64uu is 1024 + u.
__device__ __forceinline__ void codes_to_h2(uint32_t w, h2& lo, h2& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u);
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(h2, a) - bias;
  hi = __builtin_bit_cast(h2, b) - bias;
}

// fp16(fp32(t * s)): the product rounded to fp32 before the fp16 conversion
// (the empty asm keeps the backend from fusing the two into one rounding).
__device__ __forceinline__ _Float16 scale_to_f16(float t, float s) {
  float p = t * s;
  asm("" : "+v"(p));
  return (_Float16)p;
}

typedef __attribute__((address_space(3))) void lds_void;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS bytes of the staged activations [MT][Kpad] (whole rounds of the block's
// 16-byte DMA) and of the per-group scales [RI][G] (whole rounds of 4-byte DMA).
__host__ __device__ constexpr int64_t mv_x_lds(int64_t mt, int64_t kpad, int nwv) {
  return (mt * kpad / 8 + nwv * 64 - 1) / (nwv * 64) * (nwv * 64) * 16;
}
__host__ __device__ constexpr int64_t mv_s_lds(int64_t ri, int64_t g, int nwv) {
  return (ri * g + nwv * 64 - 1) / (nwv * 64) * (nwv * 64) * 4;
}

template <int MT, int GS, bool XL, int NWV, int RI>
__global__ void __launch_bounds__(NWV * 64)
mv_kernel(const _Float16* __restrict__ X, const int8_t* __restrict__ W, const float* __restrict__ SW,
          int M, int N, int K, _Float16* __restrict__ Y) {
  constexpr int kBatch = XL ? 8 : (MT == 1 ? 8 : (MT == 2 ? 4 : 2));   // steps in flight per wave
  constexpr int kStride = NWV * kBatch;                      // steps between a wave's batches
  constexpr int kLanesPerRow = 64 / RI;
  constexpr int kStep = 16 * kLanesPerRow;                   // codes (bytes) per row per step
  static_assert(GS == 0 || GS >= 16, "a lane's 16 codes must lie in one group");
  static_assert(RI == 8 || RI == 4 || RI == 2, "rows per block");
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * RI;
  const int row = lane / kLanesPerRow, sub = lane % kLanesPerRow;
  const int rows_w = min(RI, N - n0);
  const __amdgpu_buffer_rsrc_t rw = mv_rsrc(W + (int64_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);
  // rows of x past M, and codes past K, read as zero
  const __amdgpu_buffer_rsrc_t rx = mv_rsrc(X, (uint32_t)M * (uint32_t)K * 2u);
  const int steps = (K + kStep - 1) / kStep;
  const int G = GS ? K / GS : 1;
  const float* swr = SW + (int64_t)min(n0 + row, N - 1) * G;

  float acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0.0f;

  // XL: [MT][Kpad] activations, then (per-group) the block's [RI][G] scales
  extern __shared__ __attribute__((aligned(16))) _Float16 xs[];
  const int Kpad = steps * kStep;
  const float* scl = reinterpret_cast<const float*>(reinterpret_cast<const int8_t*>(xs) + mv_x_lds(MT, Kpad, NWV));
  struct Batch {
    v4i w[kBatch];
    v4i x[XL ? 1 : kBatch][XL ? 1 : MT][2];
    float s[kBatch];
  };
  auto load = [&](Batch& b, int base) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int st = base + NWV * i;
      const uint32_t kb = (uint32_t)st * kStep + 16u * (uint32_t)sub;   // code index of the lane's chunk
      const bool in = st < steps && kb < (uint32_t)K;
      b.w[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, in ? (uint32_t)row * (uint32_t)K + kb : 0x80000000u, 0, 0);
      if constexpr (!XL) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const uint32_t xo = in ? ((uint32_t)m * (uint32_t)K + kb) * 2u : 0x80000000u;
          b.x[i][m][0] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
          b.x[i][m][1] = __builtin_amdgcn_raw_buffer_load_b128(rx, in ? xo + 16u : 0x80000000u, 0, 0);
        }
      }
      if constexpr (GS != 0 && !XL) b.s[i] = in ? swr[kb / GS] : 0.0f;
    }
  };
  auto consume = [&](const Batch& b, int base) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (base + NWV * i >= steps) break;
      h2 c[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) codes_to_h2((uint32_t)b.w[i][d], c[2 * d], c[2 * d + 1]);
      const int kb = (base + NWV * i) * kStep + 16 * sub;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        float p = GS == 0 ? acc[m] : 0.0f;
        v4i xl[2];
        if constexpr (XL) {
          xl[0] = *reinterpret_cast<const v4i*>(xs + m * Kpad + kb);
          xl[1] = *reinterpret_cast<const v4i*>(xs + m * Kpad + kb + 8);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          // element first, then the bit cast: __builtin_bit_cast applied to a
          // vector-element subscript reads element 0 whatever the index
          const int xe = XL ? xl[j >> 2][j & 3] : b.x[XL ? 0 : i][XL ? 0 : m][j >> 2][j & 3];
          const h2 xv = __builtin_bit_cast(h2, xe);
          p = __builtin_amdgcn_fdot2(c[j], xv, p, false);
        }
        if constexpr (GS == 0) acc[m] = p;
        else acc[m] = __builtin_fmaf(p, XL ? scl[row * G + kb / GS] : b.s[i], acc[m]);
      }
    }
  };

  Batch ba, bb;
  if constexpr (XL) {
    // Activations (rows >= M and codes >= K as zero) and the block's scales
    // are DMA'd into LDS before any weight load, so waiting for them (vmcnt
    // counts in issue order) does not wait for the weight stream; every wave
    // issues the same number of DMA instructions (whole rounds of the block).
    const int chunks = MT * Kpad / 8, xr = (chunks + NWV * 64 - 1) / (NWV * 64);
    for (int j = 0; j < xr; ++j) {
      const int i = (j * NWV + wave) * 64 + lane;
      const int m = i / (Kpad / 8), c = i % (Kpad / 8);
      const uint32_t off = (i < chunks && m < M && c * 8 < K) ? ((uint32_t)m * (uint32_t)K + (uint32_t)c * 8) * 2u
                                                              : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(reinterpret_cast<int8_t*>(xs) + (j * NWV + wave) * 1024),
                                               16, off, 0, 0, 0);
    }
    if constexpr (GS != 0) {
      const __amdgpu_buffer_rsrc_t rs = mv_rsrc(SW + (int64_t)n0 * G, (uint32_t)rows_w * (uint32_t)G * 4u);
      const int sr = (RI * G + NWV * 64 - 1) / (NWV * 64);
      int8_t* sbase = reinterpret_cast<int8_t*>(xs) + mv_x_lds(MT, Kpad, NWV);
      for (int j = 0; j < sr; ++j) {
        const int i = (j * NWV + wave) * 64 + lane;   // scale (r = i / G, g = i % G) of the block
        const uint32_t off = i < RI * G ? (uint32_t)i * 4u : 0x80000000u;   // rows past N: past the range
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(sbase + (j * NWV + wave) * 256), 4, off, 0, 0, 0);
      }
    }
    load(ba, wave);
    wait_vmcnt<kBatch>();   // this wave's DMA landed (its weight batch may still fly)
    __syncthreads();        // everyone's
  } else {
    load(ba, wave);
  }
  for (int base = wave; base < steps; base += 2 * kStride) {
    if (base + kStride < steps) load(bb, base + kStride);
    consume(ba, base);
    if (base + kStride >= steps) break;
    if (base + 2 * kStride < steps) load(ba, base + 2 * kStride);
    consume(bb, base + kStride);
  }

  // the lanes of a row (fixed butterfly), then the waves in order
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int off = 1; off < kLanesPerRow; off <<= 1) acc[m] += __shfl_xor(acc[m], off);
  __shared__ float red[NWV][RI][MT];
  if (sub == 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m) red[wave][row][m] = acc[m];
  }
  __syncthreads();
  if (threadIdx.x >= RI * MT) return;
  const int r = threadIdx.x / MT, m = threadIdx.x % MT;
  const int n = n0 + r;
  if (m >= M || n >= N) return;
  float t = red[0][r][m];
#pragma unroll
  for (int w = 1; w < NWV; ++w) t += red[w][r][m];
  Y[(int64_t)m * N + n] = GS == 0 ? scale_to_f16(t, SW[n]) : (_Float16)t;
}

template <int MT, int GS, int NWV, int RI>
hipError_t launch_mv_w(const MvArgs& a, hipStream_t st) {
  constexpr int kStep = 16 * (64 / RI);
  const dim3 grid((unsigned)((a.N + RI - 1) / RI)), block(NWV * 64);
  const int64_t kpad = (a.K + kStep - 1) / kStep * kStep;
  const size_t lds = (size_t)(mv_x_lds(MT, kpad, NWV) + (GS ? mv_s_lds(RI, a.K / (GS ? GS : 1), NWV) : 0));
  if (lds <= 64 * 1024) {
    mv_kernel<MT, GS, true, NWV, RI><<<grid, block, lds, st>>>(static_cast<const _Float16*>(a.x), a.w, a.sw,
                                                               (int)a.M, (int)a.N, (int)a.K,
                                                               static_cast<_Float16*>(a.y));
  } else {
    mv_kernel<MT, GS, false, NWV, RI><<<grid, block, 0, st>>>(static_cast<const _Float16*>(a.x), a.w, a.sw,
                                                              (int)a.M, (int)a.N, (int)a.K,
                                                              static_cast<_Float16*>(a.y));
  }
  return hipGetLastError();
}

// Rows per block: 8 while that gives >= 1024 blocks (four per CU), else 4
// (also for more than two activation rows), else 2, so that small N still
// spreads over the 256 CUs; four waves per block.
template <int MT, int GS>
hipError_t launch_mv_t(const MvArgs& a, hipStream_t st) {
  if ((a.N + 7) / 8 >= 1024) return launch_mv_w<MT, GS, 4, 8>(a, st);
  if ((a.N + 3) / 4 >= 1024 || MT > 2) return launch_mv_w<MT, GS, 4, 4>(a, st);
  return launch_mv_w<MT, GS, 4, 2>(a, st);
}

template <int GS>
hipError_t launch_mv_gs(const MvArgs& a, hipStream_t st) {
  if (a.M == 1) return launch_mv_t<1, GS>(a, st);
  if (a.M == 2) return launch_mv_t<2, GS>(a, st);
  return launch_mv_t<4, GS>(a, st);
}

}  // namespace

hipError_t launch_mv(const MvArgs& a, hipStream_t st) {
  switch (a.group_size) {
    case 0: return launch_mv_gs<0>(a, st);
    case 64: return launch_mv_gs<64>(a, st);
    default: return launch_mv_gs<128>(a, st);
  }
}

}  // namespace cider
