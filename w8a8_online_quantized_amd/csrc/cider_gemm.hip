// INT8 x INT8 -> INT32 GEMMs with the dequant fused into the store stage, on
// CDNA4 matrix cores (v_mfma_i32_16x16x64_i8) and, for tiny M, v_dot4_i32_i8.
//
// Follows the Cider README: section "架构 / Metal Kernel 流水线"
// (matmul_fused_dequant: INT8 x INT8 -> INT32 -> FP16 with the scales applied
// in the store stage; for W4A8 the int4 weights are unpacked to int8 in the
// fragment load), section "量化" (INT32 accumulation; C_fp16 = C_int32 *
// s_act * s_weight per element) and section "W8A8 量化粒度" (per-channel or
// per-group gs = 128 / 64 scales). Section "架构 / Tile 配置" picks the tile by
// M and dispatches with an L2-friendly block order; here tiles are chosen by
// output-tile count for 64-wide waves and 256 CUs, and the block order is
// remapped so that each of the 8 XCDs (each with its own L2) works on a
// contiguous patch of output tiles.
//
// Operands: x codes [M, K] and w codes [N, K] are both K-contiguous, so each
// MFMA lane loads 16 consecutive K bytes of one row. The MFMA's first operand
// is the weight tile (output rows i = n) and its second the activation tile
// (output columns j = m); lane l then holds y[m = l%16][n = 4*(l/16) + r],
// r = 0..3 - four consecutive n of one output row - so the fp16 store is one
// 8-byte write per 16x16 sub-tile.
//
// Kernels in this file:
//   gemm_dma_kernel     per-channel / W4A8 / int32 test hook, M > 16: operands
//                       stream global -> LDS by buffer-load DMA, NS stages deep
//   gemm_dma_pg_kernel  per-group (gs 64 / 128), same pipeline plus group
//                       scales gathered into LDS
//   gemm_skinny_kernel  M <= 16: fragments buffer-loaded straight into MFMA
//                       registers, K split across the block's waves
//   gemm_gemv_kernel    M <= 4 per-channel / W4A8: full-cache-line weight
//                       stream with v_dot4_i32_i8
// W4A8 keeps the weights packed (in LDS or registers) and unpacks each lane's
// bytes into codes (nibble - 8) in the order 0,2,4,6 | 1,3,5,7 | ...; the
// activation bytes are permuted into the same order, so every MFMA / dot4
// pairs each activation code with its weight code.
#include <algorithm>
#include <type_traits>

#include "cider_internal.h"
#include "cider_quant_rule.h"

namespace cider {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4i zero4() { return v4i{0, 0, 0, 0}; }

// The lane index recomputed where it is used (mbcnt), so that no register
// holds it across a long loop.
__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Per-channel dequant of one element: fp16(fp32(fp32(acc) * s_a) * s_w), each
// product rounded to fp32 before the round-to-nearest-even fp16 conversion.
// The empty asm pins the second product as an fp32 register value: without it
// the backend fuses that multiply with the conversion into v_fma_mixlo_f16
// (even with contraction off), whose result differs from the two-step
// rounding in rare cases.
__device__ __forceinline__ _Float16 dequant1(int32_t acc, float sa, float sw) {
  float t = (float)acc * sa;
  t = t * sw;
  asm("" : "+v"(t));
  return (_Float16)t;
}

// fp16(fp32(t * s)): a finished fp32 sum times one scale (two roundings, as above).
__device__ __forceinline__ _Float16 scale1(float t, float s) {
  t = t * s;
  asm("" : "+v"(t));
  return (_Float16)t;
}

// Four consecutive outputs of one row (the same rounding as dequant1).
__device__ __forceinline__ h4 dequant4(v4i acc, float sa, float4 sw) {
  float4 t;
  t.x = ((float)acc.x * sa) * sw.x;
  t.y = ((float)acc.y * sa) * sw.y;
  t.z = ((float)acc.z * sa) * sw.z;
  t.w = ((float)acc.w * sa) * sw.w;
  asm("" : "+v"(t.x), "+v"(t.y), "+v"(t.z), "+v"(t.w));
  typedef float f4 __attribute__((ext_vector_type(4)));
  return __builtin_convertvector(f4{t.x, t.y, t.z, t.w}, h4);
}

// The same two fp32 roundings with a bfloat16 output (round to nearest even).
typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __bf16 dequant1_bf(int32_t acc, float sa, float sw) {
  float t = (float)acc * sa;
  t = t * sw;
  asm("" : "+v"(t));
  return (__bf16)t;
}

__device__ __forceinline__ bf4 dequant4_bf(v4i acc, float sa, float4 sw) {
  float4 t;
  t.x = ((float)acc.x * sa) * sw.x;
  t.y = ((float)acc.y * sa) * sw.y;
  t.z = ((float)acc.z * sa) * sw.z;
  t.w = ((float)acc.w * sa) * sw.w;
  asm("" : "+v"(t.x), "+v"(t.y), "+v"(t.z), "+v"(t.w));
  typedef float f4 __attribute__((ext_vector_type(4)));
  return __builtin_convertvector(f4{t.x, t.y, t.z, t.w}, bf4);
}

// A finished fp32 value to bfloat16.
__device__ __forceinline__ __bf16 to_bf16(float t) {
  asm("" : "+v"(t));
  return (__bf16)t;
}

// bf16(fp32(t * s)): a finished fp32 sum times one scale, two roundings.
__device__ __forceinline__ __bf16 scale1_bf(float t, float s) {
  t = t * s;
  asm("" : "+v"(t));
  return (__bf16)t;
}

// Reorder 16 activation codes (4 dwords, K order 0..15) into the order the
// unpacked int4 weights come in: 0,2,4,6 | 1,3,5,7 | 8,10,12,14 | 9,11,13,15.
__device__ __forceinline__ v4i even_odd_bytes(v4i v) {
  v4i o;
  o.x = (int)__builtin_amdgcn_perm((uint32_t)v.y, (uint32_t)v.x, 0x06040200u);
  o.y = (int)__builtin_amdgcn_perm((uint32_t)v.y, (uint32_t)v.x, 0x07050301u);
  o.z = (int)__builtin_amdgcn_perm((uint32_t)v.w, (uint32_t)v.z, 0x06040200u);
  o.w = (int)__builtin_amdgcn_perm((uint32_t)v.w, (uint32_t)v.z, 0x07050301u);
  return o;
}

// Nibbles u in [0, 15] of four bytes -> signed codes u - 8 in each byte,
// without carries between bytes: ((u | 0x80) - 8) ^ 0x80.
__device__ __forceinline__ uint32_t nib_to_code(uint32_t u) {
  return ((u | 0x80808080u) - 0x08080808u) ^ 0x80808080u;
}

__device__ __forceinline__ v4i unpack_int4(uint2 p) {
  v4i o;
  o.x = (int)nib_to_code(p.x & 0x0F0F0F0Fu);
  o.y = (int)nib_to_code((p.x >> 4) & 0x0F0F0F0Fu);
  o.z = (int)nib_to_code(p.y & 0x0F0F0F0Fu);
  o.w = (int)nib_to_code((p.y >> 4) & 0x0F0F0F0Fu);
  return o;
}

// ---------------------------------------------------------------------------
// Direct-to-LDS pipeline (per-channel and W4A8).
//
// Each stage moves BK codes of every tile row from global memory straight
// into LDS with buffer_load_dwordx4 ... lds (one wave instruction fills one
// contiguous KiB of LDS), NS stages deep, so the loads of stage k+NS-1 are in
// flight while the MFMAs of stage k run. The buffer descriptor covers exactly
// the valid rows of the tile; chunks past K get an out-of-range offset, so
// every out-of-bounds element arrives as 0 without a branch. Stage order is
// kept with s_waitcnt vmcnt (own loads) followed by s_barrier (everyone's).
// ---------------------------------------------------------------------------

// Physical 16-byte slot of logical chunk c in tile row r, for rows of RB bytes.
// Both XOR patterns were chosen by measurement on gfx950 (64 LDS banks): with
// them the MFMA fragment reads (16 consecutive rows per 16-lane group for the
// 16x16x64 shape, 32 rows per 32-lane group for 32x32x32) complete in 4
// cycles per ds_read_b128 with no bank-conflict cycles, while e.g. c ^ (r & 3)
// on 64-byte rows or c ^ (r & 7) on 128-byte rows take 8 for some of them.
template <int RB>
__device__ __forceinline__ int slot_of(int r, int c) {
  if constexpr (RB == 64) return c ^ ((r >> 1) & 3);
  else return c ^ ((r >> 1) & 7);
}

template <int RB>
__device__ __forceinline__ int tile_off(int r, int c) { return r * RB + (slot_of<RB>(r, c) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: raw buffer, 32-bit data format (gfx9 family)
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// DMA instructions each wave issues per stage for a ROWS x RB-byte tile.
template <int ROWS, int RB, int NW>
constexpr int dma_per_wave() {
  static_assert(ROWS * RB % 1024 == 0, "a stage tile is a whole number of 1 KiB blocks");
  return (ROWS * RB / 1024 + NW - 1) / NW;
}

// Issue the DMA loads of one stage of a ROWS x RB-byte operand tile. Block j
// of 1 KiB holds rows j*(1024/RB) ...; lane L writes LDS bytes L*16..L*16+15
// of its block, i.e. physical slot L % (RB/16) of block row L / (RB/16). When
// the blocks do not split evenly over the NW waves, a wave with no block left
// issues a zero-fill load (out-of-range offset) into the 1 KiB `pad`, so that
// every wave issues the same number of DMA instructions per stage and one
// s_waitcnt vmcnt count fits all waves. `wave` must be wave-uniform.
template <int ROWS, int RB, int NW>
__device__ __forceinline__ void dma_stage(__amdgpu_buffer_rsrc_t rsrc, int8_t* lds, int8_t* pad, int wave,
                                          int lane, uint32_t ld, int kb0, int kb_total) {
  constexpr int kBlocks = ROWS * RB / 1024;
  constexpr int kSlots = RB / 16;
  constexpr int kRowsPerBlock = 1024 / RB;
#pragma unroll
  for (int i = 0; i < dma_per_wave<ROWS, RB, NW>(); ++i) {
    const int j = wave + i * NW;
    const int r = j * kRowsPerBlock + lane / kSlots;
    const int p = lane % kSlots;
    const int c = slot_of<RB>(r, p);          // the XOR swizzle is an involution
    const int kb = kb0 + c * 16;
    uint32_t off = kb < kb_total ? (uint32_t)r * ld + (uint32_t)kb : 0x80000000u;
    int8_t* dst = lds + j * 1024;
    if constexpr (kBlocks % NW != 0) {
      if (j >= kBlocks) {
        off = 0x80000000u;
        dst = pad;
      }
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, off, 0, 0, 0);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// stage_barrier after this wave's LDS writes have landed (lgkmcnt(0)): the
// barrier alone does not wait for them
__device__ __forceinline__ void lds_write_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  stage_barrier();
}

// Address of output (m, n) in a column-split output: the part holding
// columns n .. n+3 (part widths are multiples of 4), as 16-bit elements.
__device__ __forceinline__ _Float16* split_dst(const OutSplit& osp, int m, int n) {
  const bool p1 = n >= osp.end[0], p2 = n >= osp.end[1], p3 = n >= osp.end[2];
  const int start = p3 ? osp.end[2] : p2 ? osp.end[1] : p1 ? osp.end[0] : 0;
  const int stop = p3 ? osp.end[3] : p2 ? osp.end[2] : p1 ? osp.end[1] : osp.end[0];
  _Float16* base = p3 ? osp.y[3] : p2 ? osp.y[2] : p1 ? osp.y[1] : osp.y[0];
  return base + (int64_t)m * (stop - start) + (n - start);
}

template <int BM, int BN, int WGM, int WGN, int BK, int NS, int WK, int EPI, bool SPLIT = false>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_dma_kernel(const int8_t* __restrict__ A, const float* __restrict__ SA, const void* __restrict__ Wv,
                const float* __restrict__ SW, int M, int N, int K, _Float16* __restrict__ Y,
                int32_t* __restrict__ ACC, int splits, OutSplit osp) {
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr bool kI4 = WK == kWeightI4;
  constexpr bool kF16 = EPI == kEpiF16 || EPI == kEpiF16Split || EPI == kEpiBF16 || EPI == kEpiBF16Split;
  constexpr bool kSplitOut = EPI == kEpiF16Split || EPI == kEpiBF16Split;
  constexpr int RBA = BK;                     // activation bytes per row per stage
  constexpr int RBW = kI4 ? BK / 2 : BK;      // weight bytes per row per stage
  constexpr int kStageBytes = BM * RBA + BN * RBW;
  constexpr int LPS = dma_per_wave<BM, RBA, NW>() + dma_per_wave<BN, RBW, NW>();   // per wave per stage
  static_assert(!kI4 || BK == 128, "int4 weights use 128-code stages (64-byte packed rows)");
  static_assert(BK == 64 || BK == 128, "stage depth");
  static_assert(TM * 16 == WTM && TN * 16 == WTN, "wave tile must be a multiple of the MFMA tile");

  // NS operand stages, the 1 KiB zero-fill pad when the DMA blocks do not
  // split evenly over the waves, then (fp16 store stage only) the tile's
  // scales: s_a of its BM rows followed by s_w of its BN columns, zero past M / N.
  constexpr bool kPad = (BM * RBA / 1024) % NW != 0 || (BN * RBW / 1024) % NW != 0;
  constexpr int kPadBytes = kPad ? 1024 : 0;
  constexpr int kScaleBytes = kF16 ? (BM + BN) * 4 : 0;
  __shared__ __attribute__((aligned(1024))) int8_t smem[NS * kStageBytes + kPadBytes + kScaleBytes];
  int8_t* const pad = smem + NS * kStageBytes;
  float* const lsc = reinterpret_cast<float*>(smem + NS * kStageBytes + kPadBytes);

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = (wave % WGM) * WTM, wn = (wave / WGM) * WTN;
  const int l16 = lane & 15, l4 = lane >> 4;

  // Work unit = (tile, K split); units are numbered tile-major and each of the
  // 8 XCDs (block b runs on XCD b % 8) takes a contiguous range of them, so
  // the splits of one tile share an L2. Tiles are then ordered in groups of 8
  // tile-rows of M (L2 reuse of the weight tiles).
  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int total = nbm * nbn;
  const int nsplit = SPLIT ? splits : 1;
  int tile, split;
  {
    const int units = total * nsplit;
    const int b = blockIdx.x, xcd = b & 7, idx = b >> 3;
    const int per = units >> 3, rem = units & 7;
    const int unit = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    tile = unit / nsplit;
    split = unit - tile * nsplit;
  }
  constexpr int kGroupM = 8;
  const int group = tile / (kGroupM * nbn);
  const int first_m = group * kGroupM;
  const int gsz = min(nbm - first_m, kGroupM);
  const int tm = first_m + (tile % (kGroupM * nbn)) % gsz;
  const int tn = (tile % (kGroupM * nbn)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;
  // this unit's codes [k0, k1): whole stages, the last split takes the rest
  const int kc = ((K + nsplit - 1) / nsplit + BK - 1) / BK * BK;
  const int k0 = split * kc, k1 = min(K, k0 + kc);

  const uint32_t lda = (uint32_t)K, ldw = kI4 ? (uint32_t)K / 2 : (uint32_t)K;
  const int rows_a = min(BM, M - m0), rows_w = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)m0 * K, (uint32_t)rows_a * lda);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(static_cast<const int8_t*>(Wv) + (int64_t)n0 * ldw, (uint32_t)rows_w * ldw);

  // Scale loads go out first: their latency overlaps the first stages' DMA,
  // and the store stage later reads them from LDS instead of global memory.
  constexpr int kScalesPerThread = (BM + BN + NW * 64 - 1) / (NW * 64);
  float scl[kScalesPerThread];
  if constexpr (kF16) {
#pragma unroll
    for (int i = 0; i < kScalesPerThread; ++i) {
      const int t = threadIdx.x + i * NW * 64;
      float v = 0.0f;
      if (t < BM) {
        if (t < rows_a) v = SA[m0 + t];
      } else if (t < BM + BN) {
        if (t - BM < rows_w) v = SW[n0 + t - BM];
      }
      scl[i] = v;
    }
  }

  v4i acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = zero4();

  const int KT = (k1 - k0 + BK - 1) / BK;
  const int kb1a = k1, kb1w = kI4 ? k1 / 2 : k1;
  // Each lane's DMA byte offsets at code 0, computed once per tile: a stage
  // that lies wholly inside [k0, k1) then needs one add per load and no range
  // checks (a uniform branch picks that path; the last stage of a ragged K
  // goes through dma_stage's per-lane checks).
  constexpr int kIA = dma_per_wave<BM, RBA, NW>(), kIW = dma_per_wave<BN, RBW, NW>();
  constexpr int kBA = BM * RBA / 1024, kBW = BN * RBW / 1024;
  uint32_t offa[kIA], offw[kIW];
#pragma unroll
  for (int i = 0; i < kIA; ++i) {
    const int r = (wave + i * NW) * (1024 / RBA) + lane / (RBA / 16);
    offa[i] = (uint32_t)r * lda + (uint32_t)(slot_of<RBA>(r, lane % (RBA / 16)) * 16);
  }
#pragma unroll
  for (int i = 0; i < kIW; ++i) {
    const int r = (wave + i * NW) * (1024 / RBW) + lane / (RBW / 16);
    offw[i] = (uint32_t)r * ldw + (uint32_t)(slot_of<RBW>(r, lane % (RBW / 16)) * 16);
  }
  auto issue = [&](int kt) {
    int8_t* st = smem + (kt % NS) * kStageBytes;
    const int kb = k0 + kt * BK;   // first code of stage kt
    if (kb + BK <= k1) {
#pragma unroll
      for (int i = 0; i < kIA; ++i) {
        const int j = wave + i * NW;
        int8_t* dst = st + j * 1024;
        uint32_t off = offa[i] + (uint32_t)kb;
        if (kBA % NW != 0 && j >= kBA) {
          dst = pad;
          off = 0x80000000u;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)dst, 16, off, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < kIW; ++i) {
        const int j = wave + i * NW;
        int8_t* dst = st + BM * RBA + j * 1024;
        uint32_t off = offw[i] + (uint32_t)(kI4 ? kb / 2 : kb);
        if (kBW % NW != 0 && j >= kBW) {
          dst = pad;
          off = 0x80000000u;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)dst, 16, off, 0, 0, 0);
      }
      return;
    }
    dma_stage<BM, RBA, NW>(ra, st, pad, wave, lane, lda, kb, kb1a);
    dma_stage<BN, RBW, NW>(rw, st + BM * RBA, pad, wave, lane, ldw, kI4 ? kb / 2 : kb, kb1w);
  };

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);

  if constexpr (kF16) {
#pragma unroll
    for (int i = 0; i < kScalesPerThread; ++i) {
      const int t = threadIdx.x + i * NW * 64;
      if (t < BM + BN) lsc[t] = scl[i];
    }
    // lgkmcnt(0): the scale writes land before the first stage barrier publishes them
    __builtin_amdgcn_s_waitcnt(0xC07F);
  }

  // Two-stage int8 pipeline for wave tiles under 160 accumulator registers:
  // the next stage's wait, barrier, DMA issue (two stages ahead) and first
  // fragment reads sit in the middle of the current stage's second 64-code
  // step, which runs from registers, so its remaining MFMAs cover the barrier
  // skew and the LDS read latency. (With 160 accumulators the extra live
  // fragments spill; those tiles keep the loop below.) Same-box A/B: M=1024
  // N=10240 K=2560 (256 x 192) 40.6 -> 39.9 us, M=4096 N=2560 K=10240
  // (256 x 192) 114.3 -> 111.4 us, M=1024 N=2560 K=10240 (128 x 320, split
  // K) 50.1 -> 48.8 us.
  if constexpr (!kI4 && BK == 128 && NS == 2 && TM * TN * 4 < 160) {
    v4i wf[TN], af[TM], nwf[TN], naf[TM];
    wait_vmcnt<0>();
    stage_barrier();
#pragma unroll
    for (int a = 0; a < TN; ++a)
      wf[a] = *reinterpret_cast<const v4i*>(smem + BM * RBA + tile_off<RBW>(wn + 16 * a + l16, l4));
#pragma unroll
    for (int b = 0; b < 2 && b < TM; ++b)
      af[b] = *reinterpret_cast<const v4i*>(smem + tile_off<RBA>(wm + 16 * b + l16, l4));
    __builtin_amdgcn_sched_barrier(0);
    issue(1);
    __builtin_amdgcn_sched_barrier(0);
    for (int kt = 0; kt < KT; ++kt) {
      const int8_t* sa_ = smem + (kt & 1) * kStageBytes;
      const int8_t* sw_ = sa_ + BM * RBA;
#pragma unroll
      for (int b = 0; b < TM; ++b) {
#pragma unroll
        for (int a = 0; a < TN; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[a], af[b], acc[a][b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (b + 2 < TM) af[b + 2] = *reinterpret_cast<const v4i*>(sa_ + tile_off<RBA>(wm + 16 * (b + 2) + l16, l4));
        naf[b] = *reinterpret_cast<const v4i*>(sa_ + tile_off<RBA>(wm + 16 * b + l16, 4 + l4));
        if (b < TN) nwf[b] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RBW>(wn + 16 * b + l16, 4 + l4));
        if (b == TM - 1) {
#pragma unroll
          for (int a = TM; a < TN; ++a)
            nwf[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RBW>(wn + 16 * a + l16, 4 + l4));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      constexpr int kHalf = TM / 2;
#pragma unroll
      for (int b = 0; b < kHalf; ++b)
#pragma unroll
        for (int a = 0; a < TN; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(nwf[a], naf[b], acc[a][b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < KT) {
        wait_vmcnt<0>();                        // stage kt+1 landed (own DMA)
        __builtin_amdgcn_s_waitcnt(0xC07F);     // own reads of stage kt returned
        stage_barrier();                        // everyone's: stage kt+1 ready, stage kt free
        issue(kt + 2);                          // into stage kt's buffer (past the end: zero fill)
        const int8_t* sb_ = smem + ((kt + 1) & 1) * kStageBytes;
#pragma unroll
        for (int a = 0; a < TN; ++a)
          wf[a] = *reinterpret_cast<const v4i*>(sb_ + BM * RBA + tile_off<RBW>(wn + 16 * a + l16, l4));
#pragma unroll
        for (int b = 0; b < 2 && b < TM; ++b)
          af[b] = *reinterpret_cast<const v4i*>(sb_ + tile_off<RBA>(wm + 16 * b + l16, l4));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = kHalf; b < TM; ++b)
#pragma unroll
        for (int a = 0; a < TN; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(nwf[a], naf[b], acc[a][b], 0, 0, 0);
    }
  } else
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmcnt<(NS - 2) * LPS>();
    stage_barrier();
    // the next stage's DMA (past the end: out-of-range offsets, zero fill,
    // never read); the 128-code int8 path issues it after its first reads
    if constexpr (kI4 || BK != 128) issue(kt + NS - 1);
    const int8_t* sa_ = smem + (kt % NS) * kStageBytes;
    const int8_t* sw_ = sa_ + BM * RBA;
    if constexpr (!kI4 && BK == 128) {
      // Two 64-code steps per stage. MFMAs run activation-fragment-major
      // (group b = the TN MFMAs of fragment b), and each group is followed
      // by reads issued ahead of use: step 0's fragment b+2, and step 1's
      // fragments b (into the register group b just freed) and the weight
      // fragment b. Step 1 then runs from registers, and a stage starts its
      // MFMAs after TN + 2 reads instead of TN + TM. (The order of the
      // MFMAs into one accumulator is unchanged: k ascending.)
      v4i wf[TN], af[TM], nwf[TN], naf[TM];
#pragma unroll
      for (int a = 0; a < TN; ++a)
        wf[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RBW>(wn + 16 * a + l16, l4));
#pragma unroll
      for (int b = 0; b < 2 && b < TM; ++b)
        af[b] = *reinterpret_cast<const v4i*>(sa_ + tile_off<RBA>(wm + 16 * b + l16, l4));
      __builtin_amdgcn_sched_barrier(0);
      issue(kt + NS - 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < TM; ++b) {
#pragma unroll
        for (int a = 0; a < TN; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[a], af[b], acc[a][b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (b + 2 < TM) af[b + 2] = *reinterpret_cast<const v4i*>(sa_ + tile_off<RBA>(wm + 16 * (b + 2) + l16, l4));
        naf[b] = *reinterpret_cast<const v4i*>(sa_ + tile_off<RBA>(wm + 16 * b + l16, 4 + l4));
        if (b < TN) nwf[b] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RBW>(wn + 16 * b + l16, 4 + l4));
        if (b == TM - 1) {
#pragma unroll
          for (int a = TM; a < TN; ++a)
            nwf[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RBW>(wn + 16 * a + l16, 4 + l4));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int b = 0; b < TM; ++b)
#pragma unroll
        for (int a = 0; a < TN; ++a)
          acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(nwf[a], naf[b], acc[a][b], 0, 0, 0);
    } else if constexpr (!kI4) {
#pragma unroll
      for (int ks = 0; ks < BK / 64; ++ks) {
        v4i wf[TN], af[TM];
#pragma unroll
        for (int a = 0; a < TN; ++a)
          wf[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RBW>(wn + 16 * a + l16, 4 * ks + l4));
#pragma unroll
        for (int b = 0; b < TM; ++b)
          af[b] = *reinterpret_cast<const v4i*>(sa_ + tile_off<RBA>(wm + 16 * b + l16, 4 * ks + l4));
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
          for (int b = 0; b < TM; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[a], af[b], acc[a][b], 0, 0, 0);
      }
    } else {
      // lane group g holds packed chunk g of its weight row: codes 32g .. 32g+31;
      // half h of it (8 bytes, 16 codes) pairs with activation chunk 2g + h.
      v4i wraw[TN];
#pragma unroll
      for (int a = 0; a < TN; ++a)
        wraw[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RBW>(wn + 16 * a + l16, l4));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4i wf[TN], af[TM];
#pragma unroll
        for (int a = 0; a < TN; ++a)
          wf[a] = unpack_int4(h ? make_uint2((uint32_t)wraw[a].z, (uint32_t)wraw[a].w)
                                : make_uint2((uint32_t)wraw[a].x, (uint32_t)wraw[a].y));
#pragma unroll
        for (int b = 0; b < TM; ++b)
          af[b] = even_odd_bytes(
              *reinterpret_cast<const v4i*>(sa_ + tile_off<RBA>(wm + 16 * b + l16, 2 * l4 + h)));
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
          for (int b = 0; b < TM; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[a], af[b], acc[a][b], 0, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();

  // Split-K (SPLIT, with the int32 epilogue): each unit stores its partial
  // sum over its K range to slab `split` of ACC ([splits][M][N]); a second
  // kernel adds the slabs and dequantizes, so no unit waits for another.
  static_assert(!SPLIT || EPI == kEpiAccI32, "split-K units store int32 partials");

  // ---- store stage: y = fp16((fp32(acc) * s_a[m]) * s_w[n]), or the raw int32.
  // Lane l holds column m = l % 16 of each 16x16 tile and the 4 consecutive
  // rows n = 4(l/16) .. +3, i.e. 4 consecutive outputs of one row of y.
  const bool vec_ok = (N & 3) == 0;
  const float* const lsa = lsc;
  const float* const lsw = lsc + BM;

  // fp16 / bf16 output with N % 8 == 0: the dequantized tile goes through LDS
  // (the operand stages are free once every wave is past its last MFMA) in
  // slabs of R rows, and is written back as whole 16-byte row chunks,
  // consecutive lanes on consecutive chunks, with nontemporal stores: every
  // store instruction fills whole 128-byte lines and the output stream does
  // not displace the operand panels from L2. Written straight from the
  // accumulator layout, each instruction covers 32 bytes of 16 rows. Same-box
  // A/B (outputs bit-identical): M=4096 N=10240 K=2560 102.9 -> 89.3 us,
  // M=8192 201.9 -> 176.3 us, M=1024 37.9 -> 32.4 us, M=1024 N=12288 K=2048
  // 32.8 -> 26.9 us; nontemporal stores straight from the accumulator layout
  // were slower (M=4096: 149 us).
  if constexpr (kF16) {
    if ((N & 7) == 0) {
      constexpr int kRowB = BN * 2 + 16;   // 16 bytes of padding spread the row starts over the banks
      constexpr int kAvail = NS * kStageBytes;
      constexpr int R = BM * kRowB <= kAvail ? BM : (BM / 2) * kRowB <= kAvail ? BM / 2 : BM / 4;
      static_assert(R % 16 == 0 && R * kRowB <= kAvail, "store slab fits the operand stages");
      constexpr int CPR = BN / 8;          // 16-byte chunks per tile row
      constexpr int kIt = (R * CPR + NW * 64 - 1) / (NW * 64);
      // Pass p takes the same TM / NP fragment rows of every wave, so all
      // waves (and all four SIMDs) share each pass's dequantization; slab
      // row (i, r) with i = wave % WGM, r < RB is tile row i * WTM + p * RB + r.
      constexpr int NP = BM / R, RB = 16 * TM / NP;
      static_assert(TM % NP == 0 && WGM * RB == R, "every wave writes RB rows per pass");
      stage_barrier();                     // every wave is done reading the operand stages
      // lane coordinates recomputed here rather than kept live across the loop
      const int s16 = lane_id() & 15, s4 = lane_id() >> 4;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int bl = 0; bl < TM / NP; ++bl) {
          const int b = p * (TM / NP) + bl;
          const int r0 = (wave % WGM) * RB + 16 * bl;   // wave-uniform slab row
          const float sam = lsa[wm + 16 * b + s16];
#pragma unroll
          for (int a = 0; a < TN; ++a) {
            const int nl = wn + 16 * a + 4 * s4;
            int8_t* d = smem + (r0 + s16) * kRowB + nl * 2;
            const float4 sw4 = *reinterpret_cast<const float4*>(lsw + nl);   // zero past N
            if constexpr (EPI == kEpiBF16 || EPI == kEpiBF16Split)
              *reinterpret_cast<bf4*>(d) = dequant4_bf(acc[a][b], sam, sw4);
            else
              *reinterpret_cast<h4*>(d) = dequant4(acc[a][b], sam, sw4);
          }
        }
        lds_write_barrier();
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
          const int f = (i * NW + wave) * 64 + lane_id();
          const int row = f / CPR, ch = f - row * CPR;
          const int m = m0 + (row / RB) * WTM + p * RB + row % RB, n = n0 + ch * 8;
          if (f < R * CPR && m < M && n < N) {
            const v4i v = *reinterpret_cast<const v4i*>(smem + row * kRowB + ch * 16);
            _Float16* dst = Y + (int64_t)m * N + n;
            if constexpr (kSplitOut) dst = split_dst(osp, m, n);   // parts are multiples of 16 wide
            __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(dst));
          }
        }
        if (p + 1 < NP) stage_barrier();   // the slab is rewritten by the next pass
      }
      return;
    }
  }
#pragma unroll
  for (int b = 0; b < TM; ++b) {
    const int ml = wm + 16 * b + l16;
    const int m = m0 + ml;
    if (m >= M) continue;
    float sam = 0.0f;
    if constexpr (kF16) sam = lsa[ml];
#pragma unroll
    for (int a = 0; a < TN; ++a) {
      const int nl = wn + 16 * a + 4 * l4;
      const int n = n0 + nl;
      if (n >= N) continue;
      if constexpr (!kF16) {
        int32_t* dst = ACC + (SPLIT ? (int64_t)split * M * N : 0) + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
          *reinterpret_cast<v4i*>(dst) = acc[a][b];
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = acc[a][b][r];
        }
      } else if constexpr (EPI == kEpiBF16 || EPI == kEpiBF16Split) {
        const bf4 o = dequant4_bf(acc[a][b], sam, *reinterpret_cast<const float4*>(lsw + nl));
        __bf16* dst = reinterpret_cast<__bf16*>(Y) + (int64_t)m * N + n;
        if constexpr (kSplitOut) dst = reinterpret_cast<__bf16*>(split_dst(osp, m, n));
        if (vec_ok && n + 3 < N) {
          *reinterpret_cast<bf4*>(dst) = o;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = o[r];
        }
      } else {
        const h4 o = dequant4(acc[a][b], sam, *reinterpret_cast<const float4*>(lsw + nl));   // s_w zero past N
        _Float16* dst = Y + (int64_t)m * N + n;
        if constexpr (kSplitOut) dst = split_dst(osp, m, n);
        if (vec_ok && n + 3 < N) {
          *reinterpret_cast<h4*>(dst) = o;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = o[r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent per-channel kernel for launches of more than one round of tiles
// (int8 weights, or packed int4 weights unpacked from LDS as in
// gemm_dma_kernel; fp16 / bf16 output, N % 8 == 0, K % 128 == 0: whole
// 128-code stages, two in flight). Each block walks its tiles one after another in the same
// XCD-contiguous order as gemm_dma_kernel, and the tiles overlap at the seam:
// the last stage of tile t already issues the DMA of tile t+1's first stage
// and of its scales (into the other of two scale buffers), and tile t's store
// stage - through LDS, whole 16-byte row chunks, nontemporal, as in
// gemm_dma_kernel, in slabs that fit the stage buffer nobody reads any more -
// then runs while that DMA lands, and its global stores drain while tile t+1
// computes. The waves split the memory work: the upper half issue every DMA
// and wait for it with s_waitcnt vmcnt, the lower half issue every global
// store and never wait on vmcnt. (vmcnt counts a wave's loads and stores in
// one in-order counter, so a wave that stored and then waited for a later
// load would wait for its stores to drain too.) Stores go through a buffer
// descriptor spanning the tile's valid rows; a masked lane gets an
// out-of-range offset, so every storing wave issues the same instructions.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int EPI, int WK = kWeightI8>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_persist_kernel(const int8_t* __restrict__ A, const float* __restrict__ SA, const int8_t* __restrict__ W,
                    const float* __restrict__ SW, int M, int N, int K, void* __restrict__ Y) {
  constexpr bool kI4 = WK == kWeightI4;
  constexpr int BK = 128, NW = WGM * WGN, NL = NW / 2;   // NL loader waves, NW - NL storer waves
  constexpr int RBW = kI4 ? BK / 2 : BK;                 // weight bytes per row per stage
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int kStageBytes = BM * BK + BN * RBW;
  constexpr int kBA = BM * BK / 1024, kBW = BN * RBW / 1024;    // 1 KiB DMA blocks per stage
  constexpr int kIA = kBA / NL, kIW = kBW / NL;                 // per loader wave
  constexpr int kRowStep = NL * (1024 / BK);                    // tile rows between a wave's blocks
  constexpr int kRowStepW = NL * (1024 / RBW);                  // the same for packed weight rows
  constexpr int kScInstr = (BM + BN) / 64;                      // 64 scales per 4-byte DMA instruction
  constexpr int kScPer = (kScInstr + NL - 1) / NL;
  constexpr int kScFloats = BM + BN;
  constexpr int kRowB = BN * 2 + 16;
  constexpr int R = BM * kRowB <= kStageBytes ? BM : (BM / 2) * kRowB <= kStageBytes ? BM / 2
                  : (BM / 4) * kRowB <= kStageBytes ? BM / 4 : BM / 8;
  constexpr int CPR = BN / 8;
  constexpr int kIt = (R * CPR + (NW - NL) * 64 - 1) / ((NW - NL) * 64);
  constexpr bool kBF = EPI == kEpiBF16;
  static_assert(EPI == kEpiF16 || EPI == kEpiBF16, "fp16 / bf16 output");
  static_assert(kBA % NL == 0 && kBW % NL == 0 && BM % 64 == 0 && BN % 64 == 0, "even DMA split");
  static_assert(TM * 16 == WTM && TN * 16 == WTN && TM >= 2, "wave tile");
  static_assert(R % 16 == 0 && R * kRowB <= kStageBytes, "store slab fits one stage");
  // pass p of the store stage takes the same TM / NP fragment rows of every
  // wave (all four SIMDs dequantize in every pass): slab row (i, r) with
  // i = wave % WGM, r < RB is tile row i * WTM + p * RB + r
  constexpr int NP = BM / R, RB = 16 * TM / NP;
  static_assert(TM % NP == 0 && WGM * RB == R, "every wave writes RB rows per pass");

  // two stages | two scale buffers ([BM] s_a then [BN] s_w) | 1 KiB landing pad for spare DMAs
  __shared__ __attribute__((aligned(1024))) int8_t smem[2 * kStageBytes + 2 * kScFloats * 4 + 1024];
  float* const lscb = reinterpret_cast<float*>(smem + 2 * kStageBytes);
  int8_t* const pad = smem + 2 * kStageBytes + 2 * kScFloats * 4;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = (wave % WGM) * WTM, wn = (wave / WGM) * WTN;
  const int l16 = lane & 15, l4 = lane >> 4;
  const bool loader = wave >= NL;
  const int lw = loader ? wave - NL : 0;

  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int units = nbm * nbn;
  const int KT = (K + BK - 1) / BK;
  const uint32_t ld = (uint32_t)K;
  const uint32_t ldw = kI4 ? ld / 2 : ld;

  // tile of virtual block vb (vb < units): XCD-contiguous ranges, then groups of 8 tile-rows
  auto tile_origin = [&](int vb, int& m0, int& n0) {
    const int xcd = vb & 7, idx = vb >> 3;
    const int per = units >> 3, rem = units & 7;
    const int tile = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    constexpr int kGroupM = 8;
    const int first_m = tile / (kGroupM * nbn) * kGroupM;
    const int gsz = min(nbm - first_m, kGroupM);
    m0 = (first_m + (tile % (kGroupM * nbn)) % gsz) * BM;
    n0 = (tile % (kGroupM * nbn)) / gsz * BN;
  };
  // descriptors spanning a tile's valid rows (passed by value: a descriptor
  // held in a struct member and handed to the DMA builtin left the kernel
  // without its host-side launch stub)
  auto rsrc_a = [&](int m0) { return make_rsrc(A + (int64_t)m0 * K, (uint32_t)min(BM, M - m0) * ld); };
  auto rsrc_w = [&](int n0) {
    return make_rsrc(W + (int64_t)n0 * (kI4 ? K / 2 : K), (uint32_t)min(BN, N - n0) * ldw);
  };
  auto rsrc_sa = [&](int m0) { return make_rsrc(SA + m0, (uint32_t)min(BM, M - m0) * 4); };
  auto rsrc_sw = [&](int n0) { return make_rsrc(SW + n0, (uint32_t)min(BN, N - n0) * 4); };

  // A loader lane's DMA byte offset at code 0 for its first block; block i of
  // the wave is kRowStep rows further, which keeps the row's swizzle slot
  // (kRowStep is a multiple of 16), so its offset is larger by i * kRowStep * K.
  const int r0 = lw * (1024 / BK) + lane / (BK / 16);
  const uint32_t off0 = (uint32_t)r0 * ld + (uint32_t)(slot_of<BK>(r0, lane % (BK / 16)) * 16);
  static_assert(kRowStep % 16 == 0, "uniform block step keeps the swizzle slot");
  // packed int4 weight rows (64 bytes per stage) have their own lane layout:
  // 16 rows of 4 chunks per 1 KiB block
  const int r0w = lw * (1024 / RBW) + lane / (RBW / 16);
  const uint32_t off0w = kI4 ? (uint32_t)r0w * ldw + (uint32_t)(slot_of<RBW>(r0w, lane % (RBW / 16)) * 16) : 0u;
  static_assert(kRowStepW % 16 == 0, "uniform block step keeps the swizzle slot");
  auto issue = [&](__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rw, int kt, int buf) {   // loader waves; K % BK == 0
    const int kb = kt * BK;
    {
      // The whole offset goes in the vector operand (the descriptor's range
      // check, which zero-fills past the tile's valid rows, applies to it).
      // `off` and `lbase` are opaque to the optimizer so that the per-block
      // offsets and LDS destinations are formed here, one add each, instead
      // of being hoisted out of the K loop as loop-invariant registers.
      // Block i of both operands sits at the same offset, and the offset of
      // block i+1 is one uniform step further: one running register and one
      // step register, instead of a loop-invariant register per block.
      uint32_t off = off0 + (uint32_t)kb;
      asm volatile("" : "+v"(off));
      uint32_t lbase = (uint32_t)buf * kStageBytes + (uint32_t)lw * 1024;
      asm volatile("" : "+s"(lbase));
      const uint32_t step = (uint32_t)kRowStep * ld;
      if constexpr (!kI4) {
#pragma unroll
        for (int i = 0; i < (kIA > kIW ? kIA : kIW); ++i) {
          if (i < kIA)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(smem + lbase + i * NL * 1024), 16, off, 0, 0, 0);
          if (i < kIW)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(smem + lbase + BM * BK + i * NL * 1024), 16,
                                                     off, 0, 0, 0);
          off += step;
        }
      } else {
        // the two operands' blocks differ in rows per block: a running
        // offset each
        uint32_t offw = off0w + (uint32_t)kb / 2;
        asm volatile("" : "+v"(offw));
        const uint32_t stepw = (uint32_t)kRowStepW * ldw;
#pragma unroll
        for (int i = 0; i < kIA; ++i) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(smem + lbase + i * NL * 1024), 16, off, 0, 0, 0);
          off += step;
        }
#pragma unroll
        for (int i = 0; i < kIW; ++i) {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(smem + lbase + BM * BK + i * NL * 1024), 16, offw,
                                                   0, 0, 0);
          offw += stepw;
        }
      }
    }
  };
  auto issue_scales = [&](__amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsw, int sb) {   // loader waves; rows past the tile load 0
    float* dst = lscb + sb * kScFloats;
    const uint32_t l4b = (uint32_t)lane_id() * 4;   // formed here, not kept across the K loop
#pragma unroll
    for (int i = 0; i < kScPer; ++i) {
      const int j = lw + i * NL;
      if (j >= kScInstr)   // spare: keeps every loader wave's vmcnt count equal
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void*)pad, 4, 0x80000000u, 0, 0, 0);
      else if (j < BM / 64)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)(dst + 64 * j), 4, 256u * j + l4b, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void*)(dst + BM + 64 * (j - BM / 64)), 4,
                                                 256u * (j - BM / 64) + l4b, 0, 0, 0);
    }
  };

  int vb = blockIdx.x;
  if (vb >= units) return;
  if (loader) {
    int m0, n0;
    tile_origin(vb, m0, n0);
    issue_scales(rsrc_sa(m0), rsrc_sw(n0), 0);
    issue(rsrc_a(m0), rsrc_w(n0), 0, 0);
  }
  int gs = 0;   // stages this block has consumed: stage kt of the current tile sits in buffer (gs + kt) & 1
  for (int it = 0;; ++it) {
    // the current tile's origin and descriptors, and the next tile's origin,
    // stay live through the K loop; the next tile's descriptors are built at
    // the last stage
    int m0, n0;
    tile_origin(vb, m0, n0);
    const __amdgpu_buffer_rsrc_t ra = rsrc_a(m0), rw = rsrc_w(n0);
    const int vbn = vb + (int)gridDim.x;
    const bool more = vbn < units;
    int m0n = 0, n0n = 0;   // the next tile's origin (its descriptors are built where used)
    if (more) tile_origin(vbn, m0n, n0n);

    v4i acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b) acc[a][b] = zero4();

    for (int kt = 0; kt < KT; ++kt) {
      if (loader) wait_vmcnt<0>();   // stage kt (and, at kt = 0, the tile's scales) landed
      stage_barrier();
      const int8_t* sa_ = smem + ((gs + kt) & 1) * kStageBytes;
      const int8_t* sw_ = sa_ + BM * BK;
      if constexpr (kI4) {
        // lane group g holds packed chunk g of its weight row (codes 32g ..
        // 32g + 31); half h of it pairs with activation chunk 2g + h, whose
        // bytes are reordered to the unpacked order (as in gemm_dma_kernel)
        v4i wraw[TN];
#pragma unroll
        for (int a = 0; a < TN; ++a)
          wraw[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RBW>(wn + 16 * a + l16, l4));
        __builtin_amdgcn_sched_barrier(0);
        if (loader) {
          if (kt + 1 < KT) {
            issue(ra, rw, kt + 1, (gs + kt + 1) & 1);
          } else if (more) {
            issue_scales(rsrc_sa(m0n), rsrc_sw(n0n), (it + 1) & 1);
            issue(rsrc_a(m0n), rsrc_w(n0n), 0, (gs + kt + 1) & 1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          v4i af[TM];
#pragma unroll
          for (int b = 0; b < TM; ++b)
            af[b] = even_odd_bytes(*reinterpret_cast<const v4i*>(sa_ + tile_off<BK>(wm + 16 * b + l16, 2 * l4 + h)));
#pragma unroll
          for (int a = 0; a < TN; ++a) {
            // unpacked just before its row of MFMAs: one weight fragment live
            const v4i wf = unpack_int4(h ? make_uint2((uint32_t)wraw[a].z, (uint32_t)wraw[a].w)
                                         : make_uint2((uint32_t)wraw[a].x, (uint32_t)wraw[a].y));
#pragma unroll
            for (int b = 0; b < TM; ++b)
              acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf, af[b], acc[a][b], 0, 0, 0);
          }
        }
      } else {
        // two 64-code steps, fragment reads issued ahead of use as in gemm_dma_kernel
        v4i wf[TN], af[TM], nwf[TN], naf[TM];
#pragma unroll
        for (int a = 0; a < TN; ++a)
          wf[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<BK>(wn + 16 * a + l16, l4));
#pragma unroll
        for (int b = 0; b < 2; ++b)
          af[b] = *reinterpret_cast<const v4i*>(sa_ + tile_off<BK>(wm + 16 * b + l16, l4));
        __builtin_amdgcn_sched_barrier(0);
        if (loader) {
          if (kt + 1 < KT) {
            issue(ra, rw, kt + 1, (gs + kt + 1) & 1);
          } else if (more) {
            issue_scales(rsrc_sa(m0n), rsrc_sw(n0n), (it + 1) & 1);
            issue(rsrc_a(m0n), rsrc_w(n0n), 0, (gs + kt + 1) & 1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < TM; ++b) {
#pragma unroll
          for (int a = 0; a < TN; ++a)
            acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[a], af[b], acc[a][b], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (b + 2 < TM) af[b + 2] = *reinterpret_cast<const v4i*>(sa_ + tile_off<BK>(wm + 16 * (b + 2) + l16, l4));
          naf[b] = *reinterpret_cast<const v4i*>(sa_ + tile_off<BK>(wm + 16 * b + l16, 4 + l4));
          if (b < TN) nwf[b] = *reinterpret_cast<const v4i*>(sw_ + tile_off<BK>(wn + 16 * b + l16, 4 + l4));
          if (b == TM - 1) {
#pragma unroll
            for (int a = TM; a < TN; ++a)
              nwf[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<BK>(wn + 16 * a + l16, 4 + l4));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
          for (int a = 0; a < TN; ++a)
            acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(nwf[a], naf[b], acc[a][b], 0, 0, 0);
      }
    }
    gs += KT;

    // ---- store stage: slabs of R rows in the buffer of the tile's last stage
    // (the next tile's first stage lands in the other one)
    stage_barrier();   // every wave is done reading that buffer
    int8_t* const slab = smem + ((gs - 1) & 1) * kStageBytes;
    const float* const lsa = lscb + (it & 1) * kScFloats;
    const float* const lsw = lsa + BM;
    const int rows_a = min(BM, M - m0);
    const __amdgpu_buffer_rsrc_t ry =
        make_rsrc(static_cast<int8_t*>(Y) + (int64_t)m0 * N * 2, (uint32_t)rows_a * (uint32_t)N * 2);
    const int s16 = lane_id() & 15, s4 = lane_id() >> 4;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
      for (int bl = 0; bl < TM / NP; ++bl) {
        const int b = p * (TM / NP) + bl;
        const int rr = (wave % WGM) * RB + 16 * bl;   // wave-uniform slab row
        const float sam = lsa[wm + 16 * b + s16];
#pragma unroll
        for (int a = 0; a < TN; ++a) {
          const int nl = wn + 16 * a + 4 * s4;
          int8_t* d = slab + (rr + s16) * kRowB + nl * 2;
          const float4 sw4 = *reinterpret_cast<const float4*>(lsw + nl);   // zero past N
          if constexpr (kBF)
            *reinterpret_cast<bf4*>(d) = dequant4_bf(acc[a][b], sam, sw4);
          else
            *reinterpret_cast<h4*>(d) = dequant4(acc[a][b], sam, sw4);
        }
      }
      lds_write_barrier();
      if (!loader) {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
          const int f = (i * (NW - NL) + wave) * 64 + lane_id();
          const int row = min(f / CPR, R - 1), ch = f - (f / CPR) * CPR;
          const int trow = (row / RB) * WTM + p * RB + row % RB;   // tile row
          const int n = n0 + ch * 8;
          const bool ok = f < R * CPR && trow < rows_a && n < N;
          const v4i v = *reinterpret_cast<const v4i*>(slab + row * kRowB + ch * 16);
          const uint32_t off = ok ? ((uint32_t)trow * (uint32_t)N + (uint32_t)n) * 2 : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, 2 /* nontemporal */);
        }
      }
      if (p + 1 < NP) stage_barrier();   // the slab is rewritten by the next pass
    }
    if (!more) break;
    vb = vbn;
  }
}

// ---------------------------------------------------------------------------
// Skinny path, M <= 16 (decode-sized batches): the weight stream dominates, so
// nothing is staged in LDS. A block owns 16 weight rows; its S waves split K
// into units of U codes (unit u goes to wave u % S) and each wave feeds its
// weight and activation fragments straight from buffer loads into
// v_mfma_i32_16x16x64_i8 (activation rows >= M and chunks past K load as
// zero). The S int32 partial sums are added through LDS in wave order, which
// is exact; per-group partial fp32 sums are added in the same fixed order.
// ---------------------------------------------------------------------------
template <int S, int WK, int GS, int EPI>
__global__ void __launch_bounds__(S * 64)
gemm_skinny_kernel(const int8_t* __restrict__ X, const float* __restrict__ SA, const void* __restrict__ Wv,
                   const float* __restrict__ SW, int M, int N, int K, _Float16* __restrict__ Y,
                   int32_t* __restrict__ ACC) {
  constexpr bool kI4 = WK == kWeightI4;
  constexpr int U = GS == 128 ? 128 : 64;      // codes per unit: one group for per-group
  constexpr int kMf = U / 64;                  // MFMAs per unit
  constexpr int kBatch = 8;                    // units in flight per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int rows_w = min(16, N - n0);
  const uint32_t ldw = kI4 ? (uint32_t)K / 2 : (uint32_t)K;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)M * (uint32_t)K);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(static_cast<const int8_t*>(Wv) + (int64_t)n0 * ldw, (uint32_t)rows_w * ldw);
  const int KU = (K + U - 1) / U;
  const int G = GS == 0 ? 1 : K / (GS == 0 ? 1 : GS);

  v4i acc = zero4();
  float facc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int base = wave; base < KU; base += kBatch * S) {
    v4i wf[kBatch][kMf], xf[kBatch][kMf];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int u = base + i * S;
#pragma unroll
      for (int j = 0; j < kMf; ++j) {
        const int k = u * U + 64 * j + 16 * l4;    // first code of this lane's chunk
        const bool in = u < KU && k < K;
        const uint32_t xo = in ? (uint32_t)l16 * (uint32_t)K + (uint32_t)k : 0x80000000u;
        xf[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rx, xo, 0, 0);
        if constexpr (kI4) {
          const uint32_t wo = in ? (uint32_t)l16 * ldw + (uint32_t)k / 2 : 0x80000000u;
          const v2i p = __builtin_amdgcn_raw_buffer_load_b64(rw, wo, 0, 0);
          wf[i][j] = v4i{p.x, p.y, 0, 0};
        } else {
          const uint32_t wo = in ? (uint32_t)l16 * ldw + (uint32_t)k : 0x80000000u;
          wf[i][j] = __builtin_amdgcn_raw_buffer_load_b128(rw, wo, 0, 0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int u = base + i * S;
      if (u >= KU) break;
#pragma unroll
      for (int j = 0; j < kMf; ++j) {
        v4i w = wf[i][j], x = xf[i][j];
        if constexpr (kI4) {
          w = unpack_int4(make_uint2((uint32_t)w.x, (uint32_t)w.y));
          x = even_odd_bytes(x);
        }
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, x, acc, 0, 0, 0);
      }
      if constexpr (GS != 0) {
        // one unit is one group: fold it into the fp32 sum and restart
        if constexpr (EPI == kEpiAccI32) {
          const int m = l16, n = n0 + 4 * l4;
          if (m < M) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < N) ACC[((int64_t)u * M + m) * N + n + r] = acc[r];
          }
        } else if constexpr (EPI == kEpiF16Tok || EPI == kEpiBF16Tok) {
          // per-token activations: s_a[m] is applied once, in the store stage
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sw = SW[(int64_t)min(n0 + 4 * l4 + r, N - 1) * G + u];
            facc[r] = __builtin_fmaf((float)acc[r], sw, facc[r]);
          }
        } else {
          const float sa = SA[(int64_t)min(l16, M - 1) * G + u];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sw = SW[(int64_t)min(n0 + 4 * l4 + r, N - 1) * G + u];
            facc[r] = __builtin_fmaf((float)acc[r] * sa, sw, facc[r]);
          }
        }
        acc = zero4();
      }
    }
  }

  // cross-wave sum in wave order, then the store stage
  using red_t = typename std::conditional<GS == 0, int, float>::type;
  __shared__ red_t red[S][4][64];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if constexpr (GS == 0) red[wave][r][lane] = acc[r];
    else red[wave][r][lane] = facc[r];
  }
  __syncthreads();
  if (wave != 0) return;
  const int m = l16;
  if (m >= M) return;
  const int n = n0 + 4 * l4;
  red_t t[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    t[r] = red[0][r][lane];
#pragma unroll
    for (int w = 1; w < S; ++w) t[r] += red[w][r][lane];
  }
  if constexpr (GS == 0) {
    if constexpr (EPI == kEpiAccI32) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) ACC[(int64_t)m * N + n + r] = t[r];
    } else if constexpr (EPI == kEpiBF16) {
      const float sam = SA[m];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n + r] = dequant1_bf(t[r], sam, SW[n + r]);
    } else {
      const float sam = SA[m];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) Y[(int64_t)m * N + n + r] = dequant1(t[r], sam, SW[n + r]);
    }
  } else if constexpr (EPI == kEpiBF16) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n + r] = to_bf16(t[r]);
  } else if constexpr (EPI == kEpiF16) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) Y[(int64_t)m * N + n + r] = (_Float16)t[r];
  } else if constexpr (EPI == kEpiF16Tok) {
    const float sam = SA[m];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) Y[(int64_t)m * N + n + r] = scale1(t[r], sam);
  } else if constexpr (EPI == kEpiBF16Tok) {
    const float sam = SA[m];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n + r] = scale1_bf(t[r], sam);
  }
}

// ---------------------------------------------------------------------------
// GEMV path, M <= 4, per-channel and W4A8: a pure weight stream. A block owns
// RI weight rows (RI = 8, 4 or 2: chosen so that the grid covers the 256 CUs
// evenly); each wave instruction loads RI rows x (1024 / RI) contiguous bytes
// (whole cache lines), lane L taking 16 bytes of row L / (64 / RI). The
// block's four waves take alternate steps along each row. The M activation
// rows are staged once in LDS (for W4A8 already in the even/odd code order
// the unpacked nibbles come in), and v_dot4_i32_i8 accumulates exact int32
// sums, reduced across the lanes of a row and then across the waves in order.
// ---------------------------------------------------------------------------
template <int MT, int WK, int EPI, int RI>
__global__ void __launch_bounds__(256)
gemm_gemv_kernel(const int8_t* __restrict__ X, const float* __restrict__ SA, const void* __restrict__ Wv,
                 const float* __restrict__ SW, int M, int N, int K, _Float16* __restrict__ Y,
                 int32_t* __restrict__ ACC) {
  constexpr bool kI4 = WK == kWeightI4;
  constexpr int kLanesPerRow = 64 / RI;
  constexpr int kStepBytes = 16 * kLanesPerRow;        // weight bytes per row per wave instruction
  constexpr int kCodes = kI4 ? 2 * kStepBytes : kStepBytes;   // codes per step
  constexpr int kBatch = RI == 8 ? 8 : 4;              // steps in flight per wave
  static_assert(RI == 8 || RI == 4 || RI == 2, "rows per instruction");
  extern __shared__ __attribute__((aligned(16))) int8_t xs[];   // [MT][Kpad]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Kpad = (K + kCodes - 1) / kCodes * kCodes;

  // block b owns row groups b, b + gridDim.x, ... of RI weight rows (one per
  // block except in the self-quantizing mode, whose grid is capped)
  int n0 = blockIdx.x * RI;
  const int row = lane / kLanesPerRow, sub = lane % kLanesPerRow;
  int rows_w = min(RI, N - n0);
  const uint32_t ldw = kI4 ? (uint32_t)K / 2 : (uint32_t)K;
  __amdgpu_buffer_rsrc_t rw =
      make_rsrc(static_cast<const int8_t*>(Wv) + (int64_t)n0 * ldw, (uint32_t)rows_w * ldw);
  const int steps = Kpad / kCodes;
  constexpr bool kLin = EPI == kEpiF16Linear || EPI == kEpiBF16Linear;
  constexpr bool kLinBF = EPI == kEpiBF16Linear;
  int acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = 0;

  // a batch = this wave's next kBatch steps (steps base, base+4, ...); steps
  // past the row load zeros, so every batch is kBatch loads (fixed wait counts)
  auto load_batch = [&](v4i (&wv)[kBatch], int base) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int st = base + 4 * i;
      const uint32_t kb = (uint32_t)st * kStepBytes + 16 * sub;   // byte offset within the row
      const bool in = st < steps && kb < ldw;
      wv[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, in ? (uint32_t)row * ldw + kb : 0x80000000u, 0, 0);
    }
  };
  auto process = [&](const v4i (&wv)[kBatch], int base) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int st = base + 4 * i;
      if (st >= steps) break;
      if constexpr (kI4) {
        // 16 packed bytes = codes st*kCodes + 32*sub .. +31, in 2 x 16 unpacked bytes
        const v4i lo = unpack_int4(make_uint2((uint32_t)wv[i].x, (uint32_t)wv[i].y));
        const v4i hi = unpack_int4(make_uint2((uint32_t)wv[i].z, (uint32_t)wv[i].w));
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int8_t* xp = xs + m * Kpad + st * kCodes + 32 * sub;
          v4i x0 = *reinterpret_cast<const v4i*>(xp);
          v4i x1 = *reinterpret_cast<const v4i*>(xp + 16);
          if constexpr (!kLin) {   // staged by DMA in natural order
            x0 = even_odd_bytes(x0);
            x1 = even_odd_bytes(x1);
          }
          int a = acc[m];
          a = __builtin_amdgcn_sdot4(lo.x, x0.x, a, false);
          a = __builtin_amdgcn_sdot4(lo.y, x0.y, a, false);
          a = __builtin_amdgcn_sdot4(lo.z, x0.z, a, false);
          a = __builtin_amdgcn_sdot4(lo.w, x0.w, a, false);
          a = __builtin_amdgcn_sdot4(hi.x, x1.x, a, false);
          a = __builtin_amdgcn_sdot4(hi.y, x1.y, a, false);
          a = __builtin_amdgcn_sdot4(hi.z, x1.z, a, false);
          a = __builtin_amdgcn_sdot4(hi.w, x1.w, a, false);
          acc[m] = a;
        }
      } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const v4i x = *reinterpret_cast<const v4i*>(xs + m * Kpad + st * kCodes + 16 * sub);
          int a = acc[m];
          a = __builtin_amdgcn_sdot4(wv[i].x, x.x, a, false);
          a = __builtin_amdgcn_sdot4(wv[i].y, x.y, a, false);
          a = __builtin_amdgcn_sdot4(wv[i].z, x.z, a, false);
          a = __builtin_amdgcn_sdot4(wv[i].w, x.w, a, false);
          acc[m] = a;
        }
      }
    }
  };

  // Activation codes (not self-quantizing): DMA'd straight into LDS before
  // any weight load, so waiting for them (vmcnt counts in issue order) does
  // not wait for the weight stream. Every wave issues the same number of
  // 1 KiB DMA instructions; chunks past the rows or past K load zeros, and
  // the LDS area is padded to whole 4 KiB rounds of the block.
  v4i wa[kBatch], wb[kBatch];
  if constexpr (!kLin) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (uint32_t)M * (uint32_t)K);
    const int chunks = MT * Kpad / 16, rounds = (chunks + 255) / 256;
    for (int j = 0; j < rounds; ++j) {
      const int i = j * 256 + wave * 64 + lane;
      const int m = i / (Kpad / 16), c = i % (Kpad / 16);
      const uint32_t off = (i < chunks && m < M && c * 16 < K) ? (uint32_t)m * (uint32_t)K + (uint32_t)c * 16
                                                                : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(xs + (j * 256 + wave * 64) * 16), 16, off, 0, 0, 0);
    }
    load_batch(wa, wave);
    wait_vmcnt<kBatch>();      // this wave's activation DMA landed (the weight batch may still fly)
    __syncthreads();           // everyone's
  } else {
    // the first weight batch goes out before x is quantized and staged, so
    // the weight stream and the x loads overlap
    load_batch(wa, wave);
  }

  // kEpiF16Linear / kEpiBF16Linear: X holds fp16 / bf16 rows; each row's
  // scale s = max|x| / 127 is formed here (block-wide max) and the codes
  // follow the quantizer's rule
  __shared__ float srow[MT];
  if constexpr (kLin) {
    const uint4* xh = reinterpret_cast<const uint4*>(X);
    const int C = K / 8;
    __shared__ uint32_t wmax[4][MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      uint32_t a = 0;
      if (m < M)
        for (int c = threadIdx.x; c < C; c += 256) a = max(a, abs_max_bits(xh[(int64_t)m * C + c]));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off));
      if (lane == 0) wmax[wave][m] = a;
    }
    __syncthreads();
    if (threadIdx.x < MT) {
      const int m = threadIdx.x;
      const uint32_t a = max(max(wmax[0][m], wmax[1][m]), max(wmax[2][m], wmax[3][m]));
      srow[m] = elem_to_float<kLinBF>(a) / 127.0f;
    }
    __syncthreads();
  }

  // self-quantizing modes: stage the codes of x (rows >= M and codes >= K as zero)
  if constexpr (kLin) {
  for (int i = threadIdx.x; i < MT * Kpad / 16; i += 256) {
    const int m = i / (Kpad / 16), c = i % (Kpad / 16);
    v4i v = zero4();
    {
      const float sc = m < MT ? srow[m] : 0.0f;
      if (m < M && c * 16 < K && sc != 0.0f) {
        const uint4* xp = reinterpret_cast<const uint4*>(X) + ((int64_t)m * K + c * 16) / 8;
        const float inv = 1.0f / sc;
        // min-max scale: no clamp needed (see code_bytes_of_chunk)
        const uint2 q0 = code_bytes_of_chunk<kLinBF, false>(xp[0], sc, inv, 127.0f);
        const uint2 q1 = code_bytes_of_chunk<kLinBF, false>(xp[1], sc, inv, 127.0f);
        v[0] = (int)q0.x;
        v[1] = (int)q0.y;
        v[2] = (int)q1.x;
        v[3] = (int)q1.y;
      }
    }
    if constexpr (kI4) v = even_odd_bytes(v);
    *reinterpret_cast<v4i*>(xs + m * Kpad + c * 16) = v;
  }
  __syncthreads();
  }

  constexpr int kStride = 4 * kBatch;          // steps between a wave's batches
  __shared__ int red[4][RI][MT];
  const int nrg = (N + RI - 1) / RI;
  for (int rg = blockIdx.x; rg < nrg; rg += gridDim.x) {
    if (rg != (int)blockIdx.x) {
      n0 = rg * RI;
      rows_w = min(RI, N - n0);
      rw = make_rsrc(static_cast<const int8_t*>(Wv) + (int64_t)n0 * ldw, (uint32_t)rows_w * ldw);
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = 0;
      load_batch(wa, wave);
    }
    for (int base = wave; base < steps; base += 2 * kStride) {
      if (base + kStride < steps) load_batch(wb, base + kStride);
      process(wa, base);
      if (base + kStride >= steps) break;
      if (base + 2 * kStride < steps) load_batch(wa, base + 2 * kStride);
      process(wb, base + kStride);
    }
    // sum the lanes of each row (integer: order does not matter)
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int off = 1; off < kLanesPerRow; off <<= 1) acc[m] += __shfl_xor(acc[m], off);
    if (sub == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) red[wave][row][m] = acc[m];
    }
    __syncthreads();
    if (threadIdx.x < RI * MT) {
      const int r = threadIdx.x / MT, m = threadIdx.x % MT;
      const int n = n0 + r;
      if (m < M && n < N) {
        const int t = red[0][r][m] + red[1][r][m] + red[2][r][m] + red[3][r][m];
        if constexpr (EPI == kEpiAccI32) ACC[(int64_t)m * N + n] = t;
        else if constexpr (EPI == kEpiF16Linear) Y[(int64_t)m * N + n] = dequant1(t, srow[m], SW[n]);
        else if constexpr (EPI == kEpiBF16Linear)
          reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n] = dequant1_bf(t, srow[m], SW[n]);
        else if constexpr (EPI == kEpiBF16)
          reinterpret_cast<__bf16*>(Y)[(int64_t)m * N + n] = dequant1_bf(t, SA[m], SW[n]);
        else Y[(int64_t)m * N + n] = dequant1(t, SA[m], SW[n]);
      }
    }
    __syncthreads();   // red is rewritten by the next row group
  }
}

constexpr int64_t kLinearBlocks = 512;   // two per CU

// Rows per block: 8 while that gives >= 1024 blocks (four per CU), else 4,
// else 2 (at least 4 for 4 activation rows, whose dot products make a block's
// work per byte higher), so that small N still spreads over the CUs. Same-box
// A/B against 8 rows everywhere (HIP events, rotating buffers): M=1 N=2560
// K=10240 9.06 -> 7.39 us (2 rows: 1280 blocks instead of 320, which ran as
// two rounds on a quarter of the CUs), W4A8 7.66 -> 5.62 us, M=4 N=2560
// K=10240 13.1 -> 9.3 us (4 rows). The self-quantizing mode keeps 8 (its
// grid is capped anyway).
inline int gemv_rows(int64_t N, int64_t M, bool self_quant) {
  if (self_quant || (N + 7) / 8 >= 1024) return 8;
  return ((N + 3) / 4 >= 1024 || M > 2) ? 4 : 2;
}

template <int MT, int WK, int EPI, int RI>
hipError_t launch_gemv_ri(const GemmArgs& g, hipStream_t st) {
  constexpr int kCodes = (WK == kWeightI4 ? 2 : 1) * 16 * (64 / RI);
  const int64_t kpad = (g.K + kCodes - 1) / kCodes * kCodes;
  const size_t lds = ((size_t)MT * kpad + 4095) / 4096 * 4096;   // whole DMA rounds of the block
  // the self-quantizing mode repeats the activation quantization in every
  // block, so its grid is capped (each block then loops over row groups)
  const int64_t nrg = (g.N + RI - 1) / RI;
  constexpr bool kLin = EPI == kEpiF16Linear || EPI == kEpiBF16Linear;
  const dim3 grid((unsigned)(kLin ? std::min<int64_t>(nrg, kLinearBlocks) : nrg)), block(256);
  gemm_gemv_kernel<MT, WK, EPI, RI><<<grid, block, lds, st>>>(g.a, g.sa, g.w, g.sw, (int)g.M, (int)g.N, (int)g.K,
                                                             static_cast<_Float16*>(g.y), g.acc);
  return hipGetLastError();
}

template <int MT, int WK, int EPI>
hipError_t launch_gemv_m(const GemmArgs& g, hipStream_t st) {
  constexpr bool kLin = EPI == kEpiF16Linear || EPI == kEpiBF16Linear;
  if constexpr (kLin) {
    return launch_gemv_ri<MT, WK, EPI, 8>(g, st);
  } else {
    switch (gemv_rows(g.N, g.M, false)) {
      case 8: return launch_gemv_ri<MT, WK, EPI, 8>(g, st);
      case 4: return launch_gemv_ri<MT, WK, EPI, 4>(g, st);
      default: return launch_gemv_ri<MT, WK, EPI, 2>(g, st);
    }
  }
}

// M <= 4 with the staged activations fitting in LDS (<= 64 KiB; the padding
// of the widest step, 1024 codes for int4 with 2 rows per block, bounds Kpad).
inline bool gemv_fits(const GemmArgs& g) {
  const int64_t mt = g.M <= 1 ? 1 : (g.M <= 2 ? 2 : 4);
  return g.M <= 4 && mt * ((g.K + 1023) / 1024 * 1024) <= 65536;
}

template <int WK, int EPI>
hipError_t launch_gemv(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 1) return launch_gemv_m<1, WK, EPI>(g, st);
  if (g.M <= 2) return launch_gemv_m<2, WK, EPI>(g, st);
  return launch_gemv_m<4, WK, EPI>(g, st);
}

template <int S, int WK, int GS, int EPI>
hipError_t launch_skinny_s(const GemmArgs& g, hipStream_t st) {
  const dim3 grid((unsigned)((g.N + 15) / 16)), block(S * 64);
  gemm_skinny_kernel<S, WK, GS, EPI><<<grid, block, 0, st>>>(g.a, g.sa, g.w, g.sw, (int)g.M, (int)g.N,
                                                             (int)g.K, static_cast<_Float16*>(g.y), g.acc);
  return hipGetLastError();
}

// K-split factor: enough waves in flight to stream the weights at HBM rate.
template <int WK, int GS, int EPI>
hipError_t launch_skinny(const GemmArgs& g, hipStream_t st) {
  const int64_t blocks = (g.N + 15) / 16;
  const int64_t units = (g.K + 63) / 64;
  if (blocks >= 1024 || units < 16) return launch_skinny_s<4, WK, GS, EPI>(g, st);
  if (blocks >= 384 || units < 64) return launch_skinny_s<8, WK, GS, EPI>(g, st);
  return launch_skinny_s<16, WK, GS, EPI>(g, st);
}

// ---------------------------------------------------------------------------
// Ragged K, per-channel: int8 rows whose length is not a multiple of 16
// codes, or packed int4 rows (K even) not a multiple of 32. A row then starts
// at an arbitrary byte offset, so a lane's fragment bytes are assembled from
// 4-byte-aligned dword loads and v_alignbyte (byte loads where the 4-byte
// window would leave the tile's rows). Activation codes at k >= K are
// zeroed, so whatever bytes the weight fragment holds there add nothing; rows
// past M or N load as zero (the buffer range ends at the tile's last row). A
// block of S waves owns one 16 x 16 output tile at a time (grid-stride over
// the tiles), the waves take alternate 64-code units of K, and their exact
// int32 sums are added through LDS in wave order before the store stage.
// This is the general path for unaligned rows; aligned K keeps the tiled
// kernels above.
// ---------------------------------------------------------------------------

// `nbytes` (8 or 16) bytes at byte offset `off` of a buffer whose range is
// `total` bytes (4-aligned base), as 2 or 4 dwords; bytes past the range are 0.
template <int NB>
__device__ __forceinline__ v4i load_unaligned(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t total) {
  constexpr int ND = NB / 4;
  const uint32_t base = off & ~3u, sh = off & 3u;
  uint32_t d[ND + 1];
  if (base + 4 * (ND + 1) <= total) {
#pragma unroll
    for (int i = 0; i <= ND; ++i) d[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, base + 4 * i, 0, 0);
  } else {
    // the window would cross the end of the range: one byte at a time
#pragma unroll
    for (int i = 0; i <= ND; ++i) {
      uint32_t v = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t o = base + 4 * i + b;
        const uint32_t byte = o < total ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, o, 0, 0) : 0u;
        v |= byte << (8 * b);
      }
      d[i] = v;
    }
  }
  v4i out = zero4();
#pragma unroll
  for (int i = 0; i < ND; ++i) out[i] = (int)__builtin_amdgcn_alignbyte(d[i + 1], d[i], sh);
  return out;
}

// Buffer over `rows` rows of `ld` bytes starting at row `r0` of `base`: the
// descriptor starts at the 4-byte boundary at or below the first byte (the
// base array is 16-byte aligned); `lead` is the first byte's offset in it.
struct RowRange {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t lead, total;
};

__device__ __forceinline__ RowRange row_range(const void* base, int64_t r0, int rows, uint32_t ld) {
  const int64_t first = r0 * (int64_t)ld;
  const int64_t start = first & ~(int64_t)3;
  RowRange rr;
  rr.lead = (uint32_t)(first - start);
  rr.total = rr.lead + (uint32_t)rows * ld;
  rr.rsrc = make_rsrc(static_cast<const int8_t*>(base) + start, rr.total);
  return rr;
}

template <int S, int WK, int EPI>
__global__ void __launch_bounds__(S * 64)
gemm_ragged_kernel(const int8_t* __restrict__ X, const float* __restrict__ SA, const void* __restrict__ Wv,
                   const float* __restrict__ SW, int M, int N, int K, _Float16* __restrict__ Y,
                   int32_t* __restrict__ ACC, int tiles_n, int64_t tiles) {
  constexpr bool kI4 = WK == kWeightI4;
  constexpr int kBatch = 4;                    // 64-code units in flight per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, l4 = lane >> 4;
  const uint32_t ldw = kI4 ? (uint32_t)K / 2 : (uint32_t)K;
  const int KU = (K + 63) / 64;
  __shared__ int red[S][4][64];
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int m0 = (int)(t / tiles_n) * 16, n0 = (int)(t % tiles_n) * 16;
    const RowRange ra = row_range(X, m0, min(16, M - m0), (uint32_t)K);
    const RowRange rw = row_range(Wv, n0, min(16, N - n0), ldw);
    v4i acc = zero4();
    for (int base = wave; base < KU; base += kBatch * S) {
      v4i xf[kBatch], wf[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int u = base + i * S;
        const int k = u * 64 + 16 * l4;           // first code of this lane's 16
        xf[i] = zero4();
        wf[i] = zero4();
        if (u < KU && k < K) {
          xf[i] = load_unaligned<16>(ra.rsrc, ra.lead + (uint32_t)l16 * (uint32_t)K + (uint32_t)k, ra.total);
          if constexpr (kI4)
            wf[i] = load_unaligned<8>(rw.rsrc, rw.lead + (uint32_t)l16 * ldw + (uint32_t)k / 2, rw.total);
          else
            wf[i] = load_unaligned<16>(rw.rsrc, rw.lead + (uint32_t)l16 * ldw + (uint32_t)k, rw.total);
          // activation codes at k + j >= K (the next row's bytes) become 0
          const int valid = K - k;
          if (valid < 16) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const int vb = min(max(valid - 4 * d, 0), 4);
              const uint32_t mask = vb >= 4 ? 0xFFFFFFFFu : ((1u << (8 * vb)) - 1u);
              xf[i][d] = (int)((uint32_t)xf[i][d] & mask);
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (base + i * S >= KU) break;
        v4i w = wf[i], x = xf[i];
        if constexpr (kI4) {
          w = unpack_int4(make_uint2((uint32_t)w.x, (uint32_t)w.y));
          x = even_odd_bytes(x);
        }
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w, x, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    if (wave == 0) {
      const int m = m0 + l16, n = n0 + 4 * l4;
      if (m < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (n + r >= N) break;
          int v = red[0][r][lane];
#pragma unroll
          for (int w2 = 1; w2 < S; ++w2) v += red[w2][r][lane];
          const int64_t o = (int64_t)m * N + n + r;
          if constexpr (EPI == kEpiAccI32) ACC[o] = v;
          else if constexpr (EPI == kEpiBF16) reinterpret_cast<__bf16*>(Y)[o] = dequant1_bf(v, SA[m], SW[n + r]);
          else Y[o] = dequant1(v, SA[m], SW[n + r]);
        }
      }
    }
    __syncthreads();   // red is rewritten by the next tile
  }
}

template <int WK, int EPI>
hipError_t launch_ragged_t(const GemmArgs& g, hipStream_t st) {
  const int64_t tn = (g.N + 15) / 16, tiles = ((g.M + 15) / 16) * tn;
  const unsigned blocks = (unsigned)std::min<int64_t>(tiles, 8192);
  gemm_ragged_kernel<4, WK, EPI><<<dim3(blocks), dim3(256), 0, st>>>(
      g.a, g.sa, g.w, g.sw, (int)g.M, (int)g.N, (int)g.K, static_cast<_Float16*>(g.y), g.acc, (int)tn, tiles);
  return hipGetLastError();
}

template <int WK>
hipError_t launch_ragged_wk(const GemmArgs& g, Epilogue epi, hipStream_t st) {
  switch (epi) {
    case kEpiF16: return launch_ragged_t<WK, kEpiF16>(g, st);
    case kEpiBF16: return launch_ragged_t<WK, kEpiBF16>(g, st);
    case kEpiAccI32: return launch_ragged_t<WK, kEpiAccI32>(g, st);
    default: return hipErrorInvalidValue;   // the other epilogues need aligned K
  }
}

// K whose rows the tiled kernels cannot load (16-byte operand chunks).
inline bool ragged_k(int64_t K, WeightKind wk) { return K % (wk == kWeightI4 ? 32 : 16) != 0; }

// ---------------------------------------------------------------------------
// Per-group variant of the direct-to-LDS pipeline (gs = 64 or 128 along K, for
// both operands). Each 128-code stage also gathers its group scales into LDS
// with 4-byte DMA loads (lane L fetches the scale of tile row 64p+L), so the
// scales arrive with the codes under the same vmcnt wait; they go to a ring of
// NS+1 scale slots, one deeper than the code stages, so a stage's scales stay
// valid while the next stage runs.
// Group g's first MFMA step visits each 16x16 tile once: it folds the tile's
// int32 sum of group g-1 into the fp32 sum, fp32(acc) * s_a[m,g-1] *
// s_w[n,g-1], and then starts the tile's group-g sum with a zero-accumulator
// MFMA. The fold's VALU work thus sits between independent MFMAs, which the
// SIMD overlaps with the matrix cores, instead of waiting for a group's MFMAs
// to drain. (Group -1 is a zero accumulator with zero scales.)
// With per-token activation scales (kEpiF16Tok) only the s_w segments are
// gathered, the fold is fp32(acc) * s_w[n,g-1] added with one fma, and s_a[m]
// multiplies the finished fp32 sum in the store stage.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WGM, int WGN, int NS, int GS, int EPI, bool SPLIT = false>
__global__ void __launch_bounds__(WGM * WGN * 64, WGM * WGN == 4 ? 2 : 1)
gemm_dma_pg_kernel(const int8_t* __restrict__ A, const float* __restrict__ SA, const int8_t* __restrict__ W,
                   const float* __restrict__ SW, int M, int N, int K, _Float16* __restrict__ Y,
                   int32_t* __restrict__ ACC, int splits = 1, float* __restrict__ PART = nullptr) {
  constexpr int BK = 128, RB = 128;
  constexpr int NW = WGM * WGN;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int GPS = BK / GS;                           // groups per stage
  constexpr int KPG = GS / 64;                           // 64-code MFMA steps per group
  constexpr int kCodeBytes = (BM + BN) * RB;
  constexpr bool kF16 = EPI != kEpiAccI32;
  constexpr bool kTok = EPI == kEpiF16Tok || EPI == kEpiBF16Tok;
  // 4-byte DMA instructions per stage and per wave (spares load nothing). The
  // int32-accumulator variant has no scales (its scale pointers are null), so
  // it issues none.
  // A group's scales sit in LDS as [BMp] s_a then [BNp] s_w (tile rows padded
  // to 64: one 4-byte DMA instruction per 64 rows; rows past the tile load 0);
  // per-token activation scales have no s_a segment.
  constexpr int BMp = kTok ? 0 : (BM + 63) / 64 * 64, BNp = (BN + 63) / 64 * 64, kSeg = BMp + BNp;
  constexpr int kScaleInstr = kF16 ? GPS * kSeg / 64 : 0;
  constexpr int kScalePer = (kScaleInstr + NW - 1) / NW;
  constexpr int kSlotFloats = GPS * kSeg;                // one stage's scales: [GPS][kSeg]
  constexpr int NSR = NS + 1;                            // scale ring slots
  constexpr int LPS = dma_per_wave<BM, RB, NW>() + dma_per_wave<BN, RB, NW>() + kScalePer;
  static_assert(TM * 16 == WTM && TN * 16 == WTN, "wave tile must be a multiple of 16");

  // NS code stages, the scale ring, a 1 KiB landing pad for spare DMAs
  constexpr int kRingOff = NS * kCodeBytes;
  constexpr int kPadOff = kRingOff + NSR * kSlotFloats * 4;
  __shared__ __attribute__((aligned(1024))) int8_t smem[kPadOff + 1024];
  float* const ring = reinterpret_cast<float*>(smem + kRingOff);
  int8_t* const pad = smem + kPadOff;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = (wave % WGM) * WTM, wn = (wave / WGM) * WTN;
  const int l16 = lane & 15, l4 = lane >> 4;

  const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const int total = nbm * nbn;
  // work unit = (tile, K range); split-K launches number them tile-major
  const int nsplit = SPLIT ? splits : 1;
  int tile, split;
  {
    const int units = total * nsplit;
    const int b = blockIdx.x, xcd = b & 7, idx = b >> 3;
    const int per = units >> 3, rem = units & 7;
    const int unit = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
    tile = unit / nsplit;
    split = unit - tile * nsplit;
  }
  constexpr int kGroupM = 8;
  const int group = tile / (kGroupM * nbn);
  const int first_m = group * kGroupM;
  const int gsz = min(nbm - first_m, kGroupM);
  const int tm = first_m + (tile % (kGroupM * nbn)) % gsz;
  const int tn = (tile % (kGroupM * nbn)) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int G = K / GS;
  const uint32_t ld = (uint32_t)K;
  const int rows_a = min(BM, M - m0), rows_w = min(BN, N - n0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)m0 * K, (uint32_t)rows_a * ld);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (int64_t)n0 * K, (uint32_t)rows_w * ld);
  // scale descriptors (never dereferenced by the int32-accumulator variant)
  const __amdgpu_buffer_rsrc_t rsa =
      make_rsrc(SA + (kF16 && !kTok ? (int64_t)m0 * G : 0), kF16 && !kTok ? (uint32_t)rows_a * G * 4 : 0u);
  const __amdgpu_buffer_rsrc_t rsw =
      make_rsrc(SW + (kF16 ? (int64_t)n0 * G : 0), kF16 ? (uint32_t)rows_w * G * 4 : 0u);

  v4i acc[TN][TM];
  float facc[TN][TM][4];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      acc[a][b] = zero4();
#pragma unroll
      for (int r = 0; r < 4; ++r) facc[a][b][r] = 0.0f;
    }

  // this unit's stages: [kt0, kt0 + KT) of the K loop (whole stages; a split
  // past the end of K has none and stores zeros)
  const int kc = ((K + nsplit - 1) / nsplit + BK - 1) / BK * BK;
  const int kt0 = split * (kc / BK);
  const int KT = max(0, min((K + BK - 1) / BK, kt0 + kc / BK) - kt0);
  // A lane's DMA byte offset at code 0 for its first 1 KiB block; block i of
  // the wave is NW * 8 rows further (a multiple of 16 rows keeps the row's
  // swizzle slot). A whole stage then costs one add per DMA instruction
  // instead of dma_stage's per-lane row, slot and range arithmetic, VALU work
  // that competes with the fold; a stage cut by the end of K still goes
  // through dma_stage. Same-box A/B (outputs bit-identical), N=2560,
  // K=10240: gs 64 M=4096 313 -> 304 us, gs 128 M=4096 161.6 -> 160.0 us,
  // M=2048 102.6 -> 101.1 us. (Interleaving the two operands' blocks ran
  // slower.)
  constexpr int kBA = BM * RB / 1024, kBW = BN * RB / 1024;
  constexpr bool kFastDma = kBA % NW == 0 && kBW % NW == 0 && (NW * (1024 / RB)) % 16 == 0;
  const int rl0 = wave * (1024 / RB) + lane / (RB / 16);
  const uint32_t off0 = (uint32_t)rl0 * ld + (uint32_t)(slot_of<RB>(rl0, lane % (RB / 16)) * 16);
  auto issue = [&](int kt) {
    int8_t* st = smem + (kt % NS) * kCodeBytes;
    const int kb = (kt0 + kt) * RB;
    if (kFastDma && kb + RB <= K) {
      const uint32_t off = off0 + (uint32_t)kb;
      const uint32_t step = (uint32_t)(NW * (1024 / RB)) * ld;
#pragma unroll
      for (int i = 0; i < kBA / NW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(st + (wave + i * NW) * 1024), 16,
                                                 off + (uint32_t)i * step, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < kBW / NW; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(st + BM * RB + (wave + i * NW) * 1024), 16,
                                                 off + (uint32_t)i * step, 0, 0, 0);
    } else {
      dma_stage<BM, RB, NW>(ra, st, pad, wave, lane, ld, kb, (int)ld);
      dma_stage<BN, RB, NW>(rw, st + BM * RB, pad, wave, lane, ld, kb, (int)ld);
    }
    float* slot = ring + (kt % NSR) * kSlotFloats;
    // the lane's scale-row offset, formed here (opaque to the optimizer): kept
    // live across the K loop, one register per instruction, it spilled
    uint32_t lrow = (uint32_t)lane_id() * (uint32_t)G * 4;
    asm volatile("" : "+v"(lrow));
#pragma unroll
    for (int i = 0; i < kScalePer; ++i) {
      const int j = wave + i * NW;
      if (j >= kScaleInstr) {   // keeps every wave's vmcnt count equal
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void*)pad, 4, 0x80000000u, 0, 0, 0);
        continue;
      }
      const int gi = j / (kSeg / 64), p = j % (kSeg / 64);
      const int g = (kt0 + kt) * GPS + gi;
      float* dst = slot + gi * kSeg + 64 * p;
      // rows past the tile's valid rows are past the descriptor's range: zero
      if (p < BMp / 64) {
        const uint32_t off = g < G ? lrow + ((uint32_t)(64 * p) * G + g) * 4 : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void*)dst, 4, off, 0, 0, 0);
      } else {
        const uint32_t off = g < G ? lrow + ((uint32_t)(64 * (p - BMp / 64)) * G + g) * 4 : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsw, (lds_void*)dst, 4, off, 0, 0, 0);
      }
    }
  };

  // fold tile (a, b)'s finished group-g sum (scales at gsc, its [kSeg] slice)
  auto fold_tile = [&](int a, int b, const float* gsc, int g) {
    if constexpr (kTok) {
      const float4 s4 = *reinterpret_cast<const float4*>(gsc + wn + 16 * a + 4 * l4);
      facc[a][b][0] = __builtin_fmaf((float)acc[a][b][0], s4.x, facc[a][b][0]);
      facc[a][b][1] = __builtin_fmaf((float)acc[a][b][1], s4.y, facc[a][b][1]);
      facc[a][b][2] = __builtin_fmaf((float)acc[a][b][2], s4.z, facc[a][b][2]);
      facc[a][b][3] = __builtin_fmaf((float)acc[a][b][3], s4.w, facc[a][b][3]);
    } else if constexpr (kF16) {
      // fp32(acc) * s_a rounded, then one fma with s_w into the sum
      const float sam = gsc[wm + 16 * b + l16];
      const float4 s4 = *reinterpret_cast<const float4*>(gsc + BMp + wn + 16 * a + 4 * l4);
      facc[a][b][0] = __builtin_fmaf((float)acc[a][b][0] * sam, s4.x, facc[a][b][0]);
      facc[a][b][1] = __builtin_fmaf((float)acc[a][b][1] * sam, s4.y, facc[a][b][1]);
      facc[a][b][2] = __builtin_fmaf((float)acc[a][b][2] * sam, s4.z, facc[a][b][2]);
      facc[a][b][3] = __builtin_fmaf((float)acc[a][b][3] * sam, s4.w, facc[a][b][3]);
    } else {
      if (g < 0 || g >= G) return;
      const int m = m0 + wm + 16 * b + l16, n = n0 + wn + 16 * a + 4 * l4;
      if (m < M) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) ACC[((int64_t)g * M + m) * N + n + r] = acc[a][b][r];
      }
    }
  };

  // group -1's scales: a zero slot (the ring slot that stage -1 would use)
  if constexpr (kF16) {
    float* z = ring + (NSR - 1) * kSlotFloats;
    for (int i = threadIdx.x; i < kSlotFloats; i += NW * 64) z[i] = 0.0f;
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): visible after the first stage barrier
  }

#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);

  for (int kt = 0; kt < KT; ++kt) {
    wait_vmcnt<(NS - 2) * LPS>();
    stage_barrier();
    issue(kt + NS - 1);   // past the end: out-of-range offsets, zero fill, never read
    const int8_t* sa_ = smem + (kt % NS) * kCodeBytes;
    const int8_t* sw_ = sa_ + BM * RB;
    const float* cur = ring + (kt % NSR) * kSlotFloats;
    const float* prev = ring + ((kt + NSR - 1) % NSR) * kSlotFloats;
#pragma unroll
    for (int gi = 0; gi < GPS; ++gi) {
      // keep each group's fragment loads with its own MFMAs (bounds register use)
      if (gi > 0) __builtin_amdgcn_sched_barrier(0);
      const int g = (kt0 + kt) * GPS + gi;
      const float* psc = gi == 0 ? prev + (GPS - 1) * kSeg : cur + (gi - 1) * kSeg;
#pragma unroll
      for (int s = 0; s < KPG; ++s) {
        const int ks = gi * KPG + s;
        v4i wf[TN], af[TM];
#pragma unroll
        for (int a = 0; a < TN; ++a)
          wf[a] = *reinterpret_cast<const v4i*>(sw_ + tile_off<RB>(wn + 16 * a + l16, 4 * ks + l4));
#pragma unroll
        for (int b = 0; b < TM; ++b)
          af[b] = *reinterpret_cast<const v4i*>(sa_ + tile_off<RB>(wm + 16 * b + l16, 4 * ks + l4));
#pragma unroll
        for (int t = 0; t < TN * TM; ++t) {
          const int a = t / TM, b = t % TM;
          if (s == 0) {
            fold_tile(a, b, psc, g - 1);
            acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[a], af[b], zero4(), 0, 0, 0);
          } else {
            acc[a][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wf[a], af[b], acc[a][b], 0, 0, 0);
          }
        }
      }
    }
  }
  // the last group (its slot was not overwritten: later zero-fill stages used other slots)
  if (KT > 0) {
    const int g = (kt0 + KT) * GPS - 1;
    const float* lsc = ring + ((KT - 1) % NSR) * kSlotFloats + (GPS - 1) * kSeg;
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
      for (int b = 0; b < TM; ++b) fold_tile(a, b, lsc, g);
  }
  wait_vmcnt<0>();
  if constexpr (SPLIT) {
    // the unit's fp32 partial sums (without s_a[m] for per-token scales) to
    // slab `split` of PART [splits][M][N]; a second kernel adds the slabs
    static_assert(kF16, "split-K per-group units store fp32 partial sums");
    const bool vec_ok = (N & 3) == 0;
    float* const slab = PART + (int64_t)split * M * N;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      const int m = m0 + wm + 16 * b + l16;
      if (m >= M) continue;
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int n = n0 + wn + 16 * a + 4 * l4;
        if (n >= N) continue;
        float* dst = slab + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
          *reinterpret_cast<float4*>(dst) = make_float4(facc[a][b][0], facc[a][b][1], facc[a][b][2], facc[a][b][3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = facc[a][b][r];
        }
      }
    }
    return;
  }
  if constexpr (kF16) {
    // N % 8 == 0: through LDS as whole 16-byte row chunks with nontemporal
    // stores, as in gemm_dma_kernel (the code stages are free after the loop)
    if ((N & 7) == 0) {
      constexpr int kRowB = BN * 2 + 16;
      constexpr int kAvail = NS * kCodeBytes;
      constexpr int R = BM * kRowB <= kAvail ? BM : (BM / 2) * kRowB <= kAvail ? BM / 2 : BM / 4;
      static_assert(R % 16 == 0 && R * kRowB <= kAvail, "store slab fits the code stages");
      constexpr int CPR = BN / 8;
      constexpr int kIt = (R * CPR + NW * 64 - 1) / (NW * 64);
      stage_barrier();
      const int s16 = lane_id() & 15, s4 = lane_id() >> 4;
#pragma unroll
      for (int p = 0; p < BM / R; ++p) {
#pragma unroll
        for (int b = 0; b < TM; ++b) {
          const int r0 = wm + 16 * b - p * R;
          if (r0 >= 0 && r0 < R) {
            const int m = m0 + wm + 16 * b + s16;
            const float sam = kTok && m < M ? SA[m] : 1.0f;
#pragma unroll
            for (int a = 0; a < TN; ++a) {
              int8_t* d = smem + (r0 + s16) * kRowB + (wn + 16 * a + 4 * s4) * 2;
              if constexpr (EPI == kEpiBF16 || EPI == kEpiBF16Tok) {
                bf4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = kTok ? scale1_bf(facc[a][b][r], sam) : to_bf16(facc[a][b][r]);
                *reinterpret_cast<bf4*>(d) = o;
              } else {
                h4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = kTok ? scale1(facc[a][b][r], sam) : (_Float16)facc[a][b][r];
                *reinterpret_cast<h4*>(d) = o;
              }
            }
          }
        }
        lds_write_barrier();
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
          const int f = (i * NW + wave) * 64 + lane_id();
          const int row = f / CPR, ch = f - row * CPR;
          const int m = m0 + p * R + row, n = n0 + ch * 8;
          if (f < R * CPR && m < M && n < N) {
            const v4i v = *reinterpret_cast<const v4i*>(smem + row * kRowB + ch * 16);
            __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(Y + (int64_t)m * N + n));
          }
        }
        if (p + 1 < BM / R) stage_barrier();
      }
      return;
    }
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      const int m = m0 + wm + 16 * b + l16;
      if (m >= M) continue;
      const float sam = kTok ? SA[m] : 1.0f;
#pragma unroll
      for (int a = 0; a < TN; ++a) {
        const int n = n0 + wn + 16 * a + 4 * l4;
        if (n >= N) continue;
        if constexpr (EPI == kEpiBF16 || EPI == kEpiBF16Tok) {
          bf4 o;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = kTok ? scale1_bf(facc[a][b][r], sam) : to_bf16(facc[a][b][r]);
          __bf16* dst = reinterpret_cast<__bf16*>(Y) + (int64_t)m * N + n;
          if (vec_ok && n + 3 < N) {
            *reinterpret_cast<bf4*>(dst) = o;
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < N) dst[r] = o[r];
          }
          continue;
        }
        h4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = kTok ? scale1(facc[a][b][r], sam) : (_Float16)facc[a][b][r];
        _Float16* dst = Y + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
          *reinterpret_cast<h4*>(dst) = o;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) dst[r] = o[r];
        }
      }
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int NS, int GS, int EPI>
hipError_t launch_dma_pg(const GemmArgs& g, hipStream_t st) {
  const int64_t nbm = (g.M + BM - 1) / BM, nbn = (g.N + BN - 1) / BN;
  const dim3 grid((unsigned)(nbm * nbn)), block(WGM * WGN * 64);
  gemm_dma_pg_kernel<BM, BN, WGM, WGN, NS, GS, EPI><<<grid, block, 0, st>>>(
      g.a, g.sa, static_cast<const int8_t*>(g.w), g.sw, (int)g.M, (int)g.N, (int)g.K,
      static_cast<_Float16*>(g.y), g.acc);
  return hipGetLastError();
}

// Most K ranges of any split-K plan: a reduction thread issues the loads of
// every range before it adds any (one memory latency instead of one per
// range; a loop over a run-time count had kept one load batch in flight).
constexpr int kMaxSplits = 8;

// Split-K reduction of fp32 per-group partial sums P [splits][M][N], added in
// split order; per-token activation scales multiply the sum (fp32 product,
// then fp16), as in the unsplit store stage.
template <int EPI, bool VEC>
__global__ void __launch_bounds__(256)
splitk_reduce_f32_kernel(const float* __restrict__ P, int splits, int M, int N, const float* __restrict__ SA,
                         void* __restrict__ Y) {
  constexpr int E = VEC ? 4 : 1;
  const int64_t total = (int64_t)M * N / E;
  const int64_t slab = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t e0 = i * E;
    const int m = (int)(e0 / N);
    float p[kMaxSplits][E];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      if (s >= splits) break;
      if constexpr (VEC) {
        const float4 v = *reinterpret_cast<const float4*>(P + s * slab + e0);
        p[s][0] = v.x, p[s][1] = v.y, p[s][2] = v.z, p[s][3] = v.w;
      } else {
        p[s][0] = P[s * slab + e0];
      }
    }
    float t[E];
#pragma unroll
    for (int r = 0; r < E; ++r) t[r] = p[0][r];
#pragma unroll
    for (int s = 1; s < kMaxSplits; ++s) {
      if (s >= splits) break;
#pragma unroll
      for (int r = 0; r < E; ++r) t[r] += p[s][r];
    }
#pragma unroll
    for (int r = 0; r < E; ++r) {
      if constexpr (EPI == kEpiBF16) static_cast<__bf16*>(Y)[e0 + r] = to_bf16(t[r]);
      else if constexpr (EPI == kEpiF16Tok) static_cast<_Float16*>(Y)[e0 + r] = scale1(t[r], SA[m]);
      else if constexpr (EPI == kEpiBF16Tok) static_cast<__bf16*>(Y)[e0 + r] = scale1_bf(t[r], SA[m]);
      else static_cast<_Float16*>(Y)[e0 + r] = (_Float16)t[r];
    }
  }
}

template <int BM, int BN, int WGM, int WGN, int NS, int GS, int EPI>
hipError_t launch_dma_pg_split(const GemmArgs& g, int splits, hipStream_t st) {
  const int64_t nbm = (g.M + BM - 1) / BM, nbn = (g.N + BN - 1) / BN;
  if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  float* parts = static_cast<float*>(g.ws);
  gemm_dma_pg_kernel<BM, BN, WGM, WGN, NS, GS, EPI, true>
      <<<dim3((unsigned)(nbm * nbn * splits)), dim3(WGM * WGN * 64), 0, st>>>(
          g.a, g.sa, static_cast<const int8_t*>(g.w), g.sw, (int)g.M, (int)g.N, (int)g.K, nullptr, nullptr, splits,
          parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool vec = (g.N & 3) == 0;
  const int64_t items = g.M * g.N / (vec ? 4 : 1);
  const unsigned blocks = (unsigned)std::min<int64_t>((items + 255) / 256, 4096);
  if (vec)
    splitk_reduce_f32_kernel<EPI, true><<<blocks, 256, 0, st>>>(parts, splits, (int)g.M, (int)g.N, g.sa, g.y);
  else
    splitk_reduce_f32_kernel<EPI, false><<<blocks, 256, 0, st>>>(parts, splits, (int)g.M, (int)g.N, g.sa, g.y);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int BK, int NS, int WK, int EPI>
hipError_t launch_dma(const GemmArgs& g, hipStream_t st) {
  const int64_t nbm = (g.M + BM - 1) / BM, nbn = (g.N + BN - 1) / BN;
  const dim3 grid((unsigned)(nbm * nbn)), block(WGM * WGN * 64);
  gemm_dma_kernel<BM, BN, WGM, WGN, BK, NS, WK, EPI><<<grid, block, 0, st>>>(
      g.a, g.sa, g.w, g.sw, (int)g.M, (int)g.N, (int)g.K, static_cast<_Float16*>(g.y), g.acc, 1, g.split);
  return hipGetLastError();
}

// Split-K reduction: y[m, n] = dequant(sum over the `splits` int32 slabs of
// P [splits][M][N]), adding the slabs in order (integers: exact), with the
// same store-stage arithmetic as the unsplit kernels (bit-identical y). Four
// consecutive outputs per thread when N % 4 == 0, else one.
template <int EPI, bool VEC>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const int32_t* __restrict__ P, int splits, int M, int N, const float* __restrict__ SA,
                     const float* __restrict__ SW, void* __restrict__ Y) {
  constexpr int E = VEC ? 4 : 1;
  const int64_t total = (int64_t)M * N / E;
  const int64_t slab = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t e0 = i * E;
    const int m = (int)(e0 / N), n = (int)(e0 % N);
    if constexpr (VEC) {
      v4i p[kMaxSplits];
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s) {
        if (s >= splits) break;
        p[s] = *reinterpret_cast<const v4i*>(P + s * slab + e0);
      }
      v4i t = p[0];
#pragma unroll
      for (int s = 1; s < kMaxSplits; ++s) {
        if (s >= splits) break;
        t += p[s];
      }
      const float4 sw = *reinterpret_cast<const float4*>(SW + n);
      if constexpr (EPI == kEpiBF16) *reinterpret_cast<bf4*>(static_cast<__bf16*>(Y) + e0) = dequant4_bf(t, SA[m], sw);
      else *reinterpret_cast<h4*>(static_cast<_Float16*>(Y) + e0) = dequant4(t, SA[m], sw);
    } else {
      int p[kMaxSplits];
#pragma unroll
      for (int s = 0; s < kMaxSplits; ++s) {
        if (s >= splits) break;
        p[s] = P[s * slab + e0];
      }
      int t = p[0];
#pragma unroll
      for (int s = 1; s < kMaxSplits; ++s) {
        if (s >= splits) break;
        t += p[s];
      }
      if constexpr (EPI == kEpiBF16) static_cast<__bf16*>(Y)[e0] = dequant1_bf(t, SA[m], SW[n]);
      else static_cast<_Float16*>(Y)[e0] = dequant1(t, SA[m], SW[n]);
    }
  }
}

// Workspace bytes of a split-K launch: the int32 slabs.
inline int64_t split_ws_bytes(int64_t M, int64_t N, int splits) { return (int64_t)splits * M * N * 4; }

// Split-K launch of BM x BN tiles over `splits` K ranges (whole stages; the
// last range takes the rest), then the reduction. g.ws holds at least
// split_ws_bytes(M, N, splits) bytes.
template <int BM, int BN, int WGM, int WGN, int BK, int NS, int WK, int EPI>
hipError_t launch_dma_split(const GemmArgs& g, int splits, hipStream_t st) {
  const int64_t nbm = (g.M + BM - 1) / BM, nbn = (g.N + BN - 1) / BN;
  if (splits < 1 || splits > kMaxSplits) return hipErrorInvalidValue;
  int32_t* parts = static_cast<int32_t*>(g.ws);
  gemm_dma_kernel<BM, BN, WGM, WGN, BK, NS, WK, kEpiAccI32, true>
      <<<dim3((unsigned)(nbm * nbn * splits)), dim3(WGM * WGN * 64), 0, st>>>(
          g.a, nullptr, g.w, nullptr, (int)g.M, (int)g.N, (int)g.K, nullptr, parts, splits, g.split);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool vec = (g.N & 3) == 0;
  const int64_t items = g.M * g.N / (vec ? 4 : 1);
  const unsigned blocks = (unsigned)std::min<int64_t>((items + 255) / 256, 4096);
  if (vec)
    splitk_reduce_kernel<EPI, true><<<blocks, 256, 0, st>>>(parts, splits, (int)g.M, (int)g.N, g.sa, g.sw, g.y);
  else
    splitk_reduce_kernel<EPI, false><<<blocks, 256, 0, st>>>(parts, splits, (int)g.M, (int)g.N, g.sa, g.sw, g.y);
  return hipGetLastError();
}

inline int64_t tiles_of(const GemmArgs& g, int bm, int bn) {
  return ((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn);
}

// The persistent kernel pays off where the one-tile-per-block launch would run
// more than one round (one block per CU); it takes whole 128-code stages, and
// its stores need N % 8 == 0 and byte offsets within one tile's rows below 2^31. Same-box A/B (outputs
// bit-identical): see gemm_persist_kernel's dispatch in launch_pc.
inline bool persist_fits(const GemmArgs& g, int bm, int bn) {
  return tiles_of(g, bm, bn) > 256 && (g.N & 7) == 0 && g.K % 128 == 0 &&
         (int64_t)bm * g.N * 2 < (int64_t(1) << 31);
}

template <int BM, int BN, int WGM, int WGN, int EPI, int WK = kWeightI8>
hipError_t launch_persist(const GemmArgs& g, hipStream_t st) {
  gemm_persist_kernel<BM, BN, WGM, WGN, EPI, WK><<<dim3(256), dim3(WGM * WGN * 64), 0, st>>>(
      g.a, g.sa, static_cast<const int8_t*>(g.w), g.sw, (int)g.M, (int)g.N, (int)g.K, g.y);
  return hipGetLastError();
}

// Tile choice. A launch of T tiles whose blocks fit `bpc` to a CU (LDS and
// registers) runs in about ceil(T / (256 * bpc)) rounds, and a round of
// BM x BN tiles costs about BM * BN * cost, where `cost` (time per output
// element per round, relative) was measured on MI355X with quantized
// Gaussian codes: large tiles reuse each staged byte over more MFMAs, small
// tiles fill the 256 CUs when M or N is small. The candidate with the lowest
// rounds * BM * BN * cost is launched (ties: the earlier one). With the
// per-channel costs (K = 2560, one block per CU) e.g. M=4096 N=10240 takes
// 256 x 320 (512 tiles: two full rounds) and M=1024 N=10240 or M=4096
// N=2560 take 128 x 320 (256 tiles).
struct TileCost {
  int bm, bn, cost, bpc = 1;
};

template <int NC>
int cheapest_tile(const GemmArgs& g, const TileCost (&c)[NC], int64_t* est_out = nullptr) {
  int best = 0;
  int64_t best_est = 0;
  for (int i = 0; i < NC; ++i) {
    const int64_t slots = 256 * (int64_t)c[i].bpc;
    const int64_t est = (tiles_of(g, c[i].bm, c[i].bn) + slots - 1) / slots * c[i].bm * c[i].bn * c[i].cost;
    if (i == 0 || est < best_est) {
      best = i;
      best_est = est;
    }
  }
  if (est_out) *est_out = best_est;
  return best;
}

// Per-channel / W4A8 tile tables (costs as described above). 128 x 128 keeps
// three 128-code stages (96 KB of LDS): same-box A/B against three 64-code
// stages, M=1024 N=4096 K=2048 (the stack's fused q/k/v) 16.5 -> 14.5 us,
// M=768 16.3 -> 14.1 us, M=1024 N=3072 K=3072 23.2 -> 19.5 us, M=512 N=8192
// K=4096 29.7 -> 24.3 us; two 128-code stages lost (17.7 us) and four tied.
// 64 x 128 (four waves of 32 x 64, four 128-code stages, 96 KB): one round
// where 64 x 64 needs two, with a quarter less DMA per CU than two 64 x 64
// blocks; it takes over from 64 x 64 wherever the estimate picks it.
// Same-box A/B on all 11 shapes where the pick changes: M=1024 N=2048
// K=6144 (the stack's down projection) 26.5 -> 24.6 us, K=2048 10.8 -> 10.4
// us, M=512 N=4096 K=4096 19.0 -> 17.3 us, M=192 N=8192 K=4096 20.1 -> 18.1
// us, M=128 N=12288 K=2560 16.3 -> 15.1 us, none slower. 256 x 192 (wave
// tiles of 128 x 48) for one round of up to 256 tiles where 128 x 320 or
// 256 x 320 would leave CUs idle or need a second round; same-box A/B: M=1024
// N=12288 K=2048 (exactly 256 tiles) 33.4 us against 43.8 us for the 156 tiles
// of 256 x 320, M=4096 N=2560 K=10240 (224 tiles) 112 us against 122 us for
// 128 x 320, M=1024 N=10240 K=2560 a tie (41.5 / 40.5 us).
// 64 x 64 and 64 x 80 keep four 128-code stages in flight (64 / 72 KB of
// LDS): at small M the weight stream is HBM-bound and two stages leave too few
// bytes in flight per CU. Same-box A/B against two-stage 64 x 64 tiles
// (three 64-code stages at <= 256 tiles): M=128 N=10240 K=2560 18.0 -> 12.8
// us (64 x 80: 256 tiles, one round), M=64 N=10240 K=2560 17.0 -> 11.6 us,
// M=1024 N=1024 K=2048 13.3 -> 8.6 us, M=1024 N=2048 K=2048 14.8 -> 12.8 us;
// and, with the lower 64 x 64 cost, unsplit 64 x 64 beats split-K 128 x 128
// at M=256 N=4096 K=4096 (19.8 -> 13.2 us) and M=512 (27.8 -> 21.6 us).
// 64 x 160 (also as the split-K tile) has four stages too (112 KB): M=128
// N=2560 K=10240 19.4 -> 17.6 us, M=64 18.6 -> 16.5 us.
constexpr TileCost kTilesI8[] = {{256, 320, 62}, {128, 320, 92}, {128, 256, 102}, {128, 128, 105},
                                 {64, 160, 167}, {64, 64, 150}, {256, 192, 76}, {64, 80, 185}, {64, 128, 139}};
constexpr TileCost kTilesI4[] = {{256, 320, 62}, {128, 320, 92}, {128, 256, 102}, {128, 128, 105}, {64, 64, 194}};

// Split-K plan for medium M with long K: too few output tiles to fill the
// 256 CUs are cut along K into `splits` ranges (int32 partial slabs, then a
// reduction). Candidates: 64x160 (int8 only), 128x128, 128x320, each with the
// largest power-of-two split count <= min(8, 256 / tiles) (one round),
// at least 4 and leaving >= 1024 codes per range; a block of a split launch
// costs about BM * BN * cost * (K / splits) / 2560 by the same measured
// costs. The cheapest candidate is used when it is below 0.6 x the unsplit
// estimate (the margin pays for the reduction and the second launch).
// Measured on MI355X (N=2560, K=10240): M=128 50.8 -> 18.2 us, M=256 50.9 ->
// 24.1 us, M=1024 65.9 -> 46.6 us; outputs are bit-identical.
// Per-group (gs 64 / 128, both operands or per-token activations) units
// store fp32 partial sums. Plan by tile count (K >= 4096, >= 1024 codes per
// range): 64x64 tiles with 4 K ranges up to 160 tiles and 2 up to 320; else
// 128x128 tiles with 3 ranges when 3 x tiles fill at most one round of two
// blocks per CU (512); else, for gs 128, 128x160 tiles with 2 ranges on the
// same condition; none beyond. Measured on MI355X, N=2560, K=10240, gs 128 /
// 64: M=128 60.7 / 69.3 -> 24.3 / 28.0 us, M=256 61.7 / 70.5 -> 31.7 / 35.3
// us, M=512 65.7 / 75.3 -> 52.8 / 64.6 us (64x64); M=1024 81.2 / 92.6 ->
// 67.3 / 86.1 us (128x128, 3 ranges); gs 128 M=2048 129.0 -> 106.8 us
// (128x160, 2 ranges). The tile-cost model above mispredicts these
// launches, hence a table by tile count.
struct SplitPlan {
  int tile = -1;     // per-channel 0: 64x160, 1: 128x128, 2: 128x320; per-group 0: 64x64, 1: 128x128, 2: 128x160, 3: 64x160
  int splits = 0;
};

SplitPlan plan_split_pg(const GemmArgs& g) {
  SplitPlan plan;
  if (g.M <= 16 || g.K < 4096) return plan;
  const int64_t t64 = tiles_of(g, 64, 64), t128 = tiles_of(g, 128, 128), t160 = tiles_of(g, 128, 160);
  // At most 32 tiles of 64 x 160 (M <= 128 at N = 2560) and K >= 8192: eight
  // K ranges of 64 x 160 (two 128-code stages), 256 units, one per CU.
  // Same-box A/B at N=2560, K=10240: M=128 31.0 -> 25.3 us (gs 128) and
  // 32.7 -> 29.1 us (gs 64), M=64 27.4 -> 24.5 us. With four ranges it lost
  // (M=256 gs 64 41.1 -> 44.9 us; M=128, N=4096, K=4096 19.4 -> 22.0 us),
  // and three or four stages ran slower than two (27.7 / 26.3 us at M=128).
  if (tiles_of(g, 64, 160) * 8 <= 256 && g.K / 8 >= 1024) {
    plan.tile = 3;
    plan.splits = 8;
    return plan;
  }
  // 161..320 tiles of 64 x 64 with K >= 8192: four K ranges of 128 x 128
  // rather than two of 64 x 64. Same-box A/B: M=512, N=2560, K=10240 60.4 ->
  // 51.0 us (gs 128) and 66.2 -> 60.6 us (gs 64), M=500, N=2000, K=8192
  // 42.2 -> 37.7 us, M=384, N=3072, K=8192 45.5 -> 43.0 us (gs 64: 49.7 ->
  // 50.3); at K=4096 (M=512, N=2048) it lost, 26.2 -> 26.8 us.
  if (t64 > 160 && t64 <= 320 && 4 * t128 <= 512 && g.K >= 8192) {
    plan.tile = 1;
    plan.splits = 4;
  } else if (t64 <= 320) {
    plan.tile = 0;
    plan.splits = t64 <= 160 ? 4 : 2;
  } else if (3 * t128 <= 512) {
    plan.tile = 1;
    plan.splits = 3;
  } else if (g.group_size == 128 && 2 * t160 <= 512) {
    plan.tile = 2;
    plan.splits = 2;
  }
  if (plan.splits && g.K / plan.splits < 1024) plan = SplitPlan{};
  return plan;
}

SplitPlan plan_split(const GemmArgs& g, WeightKind wk) {
  SplitPlan plan;
  if (ragged_k(g.K, wk)) return plan;
  if (g.group_size != 0) return wk == kWeightI8 ? plan_split_pg(g) : plan;
  if (g.M <= 16 || g.K < 4096) return plan;
  int64_t est_plain = 0;
  const int pick = wk == kWeightI4 ? cheapest_tile(g, kTilesI4, &est_plain) : cheapest_tile(g, kTilesI8, &est_plain);
  // a plain launch of fewer than 256 tiles leaves CUs idle that split-K
  // units would use: its estimate is scaled by 256 / tiles. Same-box A/B,
  // M=256 N=2560 K=10240 (160 tiles of 64 x 64): split-K 22.2 us against
  // 27.3 us plain; at 256 tiles (M=256 N=4096 K=4096) plain wins, 13.3 / 19.7 us.
  {
    const TileCost& c = wk == kWeightI4 ? kTilesI4[pick] : kTilesI8[pick];
    const int64_t t = tiles_of(g, c.bm, c.bn);
    if (t < 256) est_plain = est_plain * 256 / t;
  }
  static constexpr TileCost kCand[] = {{64, 160, 167}, {128, 128, 105}, {128, 320, 92}};
  int64_t best = 0;
  for (int i = wk == kWeightI4 ? 1 : 0; i < 3; ++i) {
    const int64_t t = tiles_of(g, kCand[i].bm, kCand[i].bn);
    int s = 8;
    while (s > 1 && t * s > 256) s >>= 1;
    // two ranges only when each is long: M=1024 N=2048 K=6144 (128 x 128,
    // 2 x 3072 codes) ran 30.5 us against 34.5 us for 128 x 320 in 4 ranges
    if (s < 2 || (s == 2 && g.K < 6144) || g.K / s < 1024) continue;
    const int64_t est = (int64_t)kCand[i].bm * kCand[i].bn * kCand[i].cost * (g.K / s) / 2560;
    if (plan.tile < 0 || est < best) {
      plan.tile = i;
      plan.splits = s;
      best = est;
    }
  }
  const int64_t plain = est_plain * g.K / 2560;
  if (plan.tile < 0 || best * 10 >= plain * 6) return SplitPlan{};
  return plan;
}


// Wave tiles stay <= 128 x 80 (160 accumulator registers) with two waves per
// SIMD: larger wave tiles (128 x 128) made the register allocator shuffle
// accumulators between MFMAs.
template <int WK, int EPI>
hipError_t launch_pc(const GemmArgs& g, hipStream_t st) {
  if constexpr (EPI == kEpiF16 || EPI == kEpiBF16) {
    if (g.ws) {
      const SplitPlan p = plan_split(g, (WeightKind)WK);
      if (p.splits && g.ws_bytes >= split_ws_bytes(g.M, g.N, p.splits)) {
        if constexpr (WK == kWeightI4) {
          if (p.tile == 1) return launch_dma_split<128, 128, 2, 2, 128, 2, WK, EPI>(g, p.splits, st);
          return launch_dma_split<128, 320, 2, 4, 128, 2, WK, EPI>(g, p.splits, st);
        } else {
          if (p.tile == 0) return launch_dma_split<64, 160, 2, 2, 128, 4, WK, EPI>(g, p.splits, st);
          if (p.tile == 1) return launch_dma_split<128, 128, 2, 2, 128, 3, WK, EPI>(g, p.splits, st);
          return launch_dma_split<128, 320, 2, 4, 128, 2, WK, EPI>(g, p.splits, st);
        }
      }
    }
  }
  if constexpr (WK == kWeightI4) {
    switch (cheapest_tile(g, kTilesI4)) {
      case 0:
        if constexpr (EPI == kEpiF16 || EPI == kEpiBF16)
          if (persist_fits(g, 256, 320)) return launch_persist<256, 320, 2, 4, EPI, WK>(g, st);
        return launch_dma<256, 320, 2, 4, 128, 2, WK, EPI>(g, st);
      case 1: return launch_dma<128, 320, 2, 4, 128, 2, WK, EPI>(g, st);
      case 2: return launch_dma<128, 256, 2, 4, 128, 2, WK, EPI>(g, st);
      case 3: return launch_dma<128, 128, 2, 2, 128, 2, WK, EPI>(g, st);
      default: return launch_dma<64, 64, 1, 4, 128, 2, WK, EPI>(g, st);
    }
  } else {
    switch (cheapest_tile(g, kTilesI8)) {
      case 0:
        if constexpr (EPI == kEpiF16 || EPI == kEpiBF16)
          if (persist_fits(g, 256, 320)) return launch_persist<256, 320, 2, 4, EPI>(g, st);
        return launch_dma<256, 320, 2, 4, 128, 2, WK, EPI>(g, st);
      case 1: return launch_dma<128, 320, 2, 4, 128, 2, WK, EPI>(g, st);
      case 2: return launch_dma<128, 256, 2, 4, 128, 2, WK, EPI>(g, st);
      case 3: return launch_dma<128, 128, 2, 2, 128, 3, WK, EPI>(g, st);
      case 4: return launch_dma<64, 160, 2, 2, 128, 4, WK, EPI>(g, st);
      case 5: return launch_dma<64, 64, 1, 4, 128, 4, WK, EPI>(g, st);
      case 6: return launch_dma<256, 192, 2, 4, 128, 2, WK, EPI>(g, st);
      case 7: return launch_dma<64, 80, 4, 1, 128, 4, WK, EPI>(g, st);
      default: return launch_dma<64, 128, 2, 2, 128, 4, WK, EPI>(g, st);
    }
  }
}

// Per-group tiles, chosen by the same round-count estimate with costs measured
// on MI355X at N = 2560, K = 10240 (the fp32 fold after every group makes
// per-group VALU-heavy, so its costs differ from the per-channel ones). Wave
// tiles stay at 64 x 64 / 64 x 80: the fp32 sums double the accumulator
// registers. All per-group blocks have 4 waves and are built for two blocks
// per CU (<= 256 registers, <= 80 KB of LDS; 64 x 64 fits four): the fold is
// VALU work that all waves of a block reach at the same point of each stage,
// and blocks at different points let a SIMD overlap one wave's fold with
// another wave's MFMAs. Same-box A/B against the former 8-wave 256 x 160 /
// 256 x 128 tiles: gs 128, M=4096 203 -> 167 us, M=2048 159 -> 118 us, M=8192
// 375 -> 324 us; per-token activations M=4096 175 -> 142 us (gs 128) and
// 270 -> 197 us (gs 64). 128 x 160 is left out for gs 64 with both operands
// per-group: its s_a segments push it past 256 registers.
template <int GS, int EPI>
hipError_t launch_pg(const GemmArgs& g, hipStream_t st) {
  if constexpr (EPI != kEpiAccI32) {
    if (g.ws) {
      const SplitPlan p = plan_split_pg(g);
      if (p.splits && g.ws_bytes >= split_ws_bytes(g.M, g.N, p.splits)) {
        if (p.tile == 3) return launch_dma_pg_split<64, 160, 2, 2, 2, GS, EPI>(g, p.splits, st);
        if (p.tile == 0) return launch_dma_pg_split<64, 64, 1, 4, 2, GS, EPI>(g, p.splits, st);
        if constexpr (GS == 128) {
          if (p.tile == 2) return launch_dma_pg_split<128, 160, 2, 2, 2, GS, EPI>(g, p.splits, st);
        }
        return launch_dma_pg_split<128, 128, 2, 2, 2, GS, EPI>(g, p.splits, st);
      }
    }
  }
  constexpr bool kTok = EPI == kEpiF16Tok || EPI == kEpiBF16Tok;
  if constexpr (GS == 64 && !kTok) {
    static constexpr TileCost kTiles[] = {{128, 128, 985, 2}, {64, 64, 2500, 4}};
    if (cheapest_tile(g, kTiles) == 0) return launch_dma_pg<128, 128, 2, 2, 2, GS, EPI>(g, st);
    return launch_dma_pg<64, 64, 1, 4, 2, GS, EPI>(g, st);
  } else {
    static constexpr TileCost kPg128[] = {{128, 160, 851, 2}, {128, 128, 737, 2}, {64, 64, 2033, 4}};
    static constexpr TileCost kTok128[] = {{128, 160, 722, 2}, {128, 128, 648, 2}, {64, 64, 1660, 4}};
    static constexpr TileCost kTok64[] = {{128, 160, 1001, 2}, {128, 128, 762, 2}, {64, 64, 2110, 4}};
    switch (cheapest_tile(g, !kTok ? kPg128 : (GS == 128 ? kTok128 : kTok64))) {
      case 0: return launch_dma_pg<128, 160, 2, 2, 2, GS, EPI>(g, st);
      case 1: return launch_dma_pg<128, 128, 2, 2, 2, GS, EPI>(g, st);
      default: return launch_dma_pg<64, 64, 1, 4, 2, GS, EPI>(g, st);
    }
  }
}

template <int EPI>
hipError_t launch_epi(const GemmArgs& g, WeightKind wk, hipStream_t st) {
  if (g.group_size == 0 && gemv_fits(g))
    return wk == kWeightI4 ? launch_gemv<kWeightI4, EPI>(g, st) : launch_gemv<kWeightI8, EPI>(g, st);
  if (g.M <= 16) {
    if (wk == kWeightI4) return launch_skinny<kWeightI4, 0, EPI>(g, st);
    switch (g.group_size) {
      case 0: return launch_skinny<kWeightI8, 0, EPI>(g, st);
      case 64: return launch_skinny<kWeightI8, 64, EPI>(g, st);
      default: return launch_skinny<kWeightI8, 128, EPI>(g, st);
    }
  }
  if (wk == kWeightI4) return launch_pc<kWeightI4, EPI>(g, st);
  switch (g.group_size) {
    case 0: return launch_pc<kWeightI8, EPI>(g, st);
    case 64: return launch_pg<64, EPI>(g, st);
    default: return launch_pg<128, EPI>(g, st);
  }
}

// Per-token activations x per-group int8 weights: the skinny kernel for
// M <= 16, else the per-group pipeline (tile costs as for per-group scales).
template <int EPI>
hipError_t launch_tok(const GemmArgs& g, hipStream_t st) {
  if (g.M <= 16)
    return g.group_size == 64 ? launch_skinny<kWeightI8, 64, EPI>(g, st) : launch_skinny<kWeightI8, 128, EPI>(g, st);
  return g.group_size == 64 ? launch_pg<64, EPI>(g, st) : launch_pg<128, EPI>(g, st);
}

}  // namespace

int64_t gemm_split_workspace_bytes(int64_t M, int64_t N, int64_t K, WeightKind wk, int group_size) {
  GemmArgs g{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.group_size = group_size;
  const SplitPlan p = plan_split(g, wk);
  return p.splits ? split_ws_bytes(M, N, p.splits) : 0;
}

bool linear_is_one_launch(int64_t M, int64_t K, int group_size, WeightKind wk) {
  GemmArgs g{};
  g.M = M;
  g.K = K;
  return group_size == 0 && M >= 1 && M <= 2 && !ragged_k(K, wk) && gemv_fits(g);
}

hipError_t launch_gemm(const GemmArgs& g, WeightKind wk, Epilogue epi, hipStream_t st) {
  // Unaligned rows (per-channel only; the entry points keep every other
  // kind at aligned K) take the general kernel.
  if (ragged_k(g.K, wk))
    return wk == kWeightI4 ? launch_ragged_wk<kWeightI4>(g, epi, st) : launch_ragged_wk<kWeightI8>(g, epi, st);
  // Tile table by M (the README's tile section also switches configs by M).
  if (epi == kEpiF16Tok) return launch_tok<kEpiF16Tok>(g, st);
  if (epi == kEpiBF16Tok) return launch_tok<kEpiBF16Tok>(g, st);
  if (epi == kEpiBF16) return launch_epi<kEpiBF16>(g, wk, st);
  if (epi == kEpiF16Linear)   // g.a holds fp16 activations; linear_is_one_launch() holds
    return wk == kWeightI4 ? launch_gemv<kWeightI4, kEpiF16Linear>(g, st) : launch_gemv<kWeightI8, kEpiF16Linear>(g, st);
  if (epi == kEpiBF16Linear)  // the same with bf16 activations and output
    return wk == kWeightI4 ? launch_gemv<kWeightI4, kEpiBF16Linear>(g, st) : launch_gemv<kWeightI8, kEpiBF16Linear>(g, st);
  if (epi == kEpiF16Split || epi == kEpiBF16Split) {
    const bool bf = epi == kEpiBF16Split;
    if (g.M > 16) return bf ? launch_pc<kWeightI8, kEpiBF16Split>(g, st) : launch_pc<kWeightI8, kEpiF16Split>(g, st);
    // small M: one launch per part over its rows of the weights (the same
    // per-channel arithmetic, so the same bits as the fused launch)
    int start = 0;
    for (int i = 0; i < kMaxSplitParts && start < g.N; ++i) {
      GemmArgs p = g;
      p.w = static_cast<const int8_t*>(g.w) + (int64_t)start * g.K;
      p.sw = g.sw + start;
      p.N = g.split.end[i] - start;
      p.y = g.split.y[i];
      const hipError_t e = bf ? launch_epi<kEpiBF16>(p, kWeightI8, st) : launch_epi<kEpiF16>(p, kWeightI8, st);
      if (e != hipSuccess) return e;
      start = g.split.end[i];
    }
    return hipSuccess;
  }
  return epi == kEpiF16 ? launch_epi<kEpiF16>(g, wk, st) : launch_epi<kEpiAccI32>(g, wk, st);
}

}  // namespace cider
