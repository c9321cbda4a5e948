// Internal declarations shared by the HIP translation units of libcider.
// Nothing here is part of the public ABI (include/cider.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cider {

// Launches the activation / weight quantization kernel.
//   x: fp16 [R, K]; qmax 127 (int8 codes into q8 [R, K]) or 7 (packed int4
//   codes into q4 [R, K/2]); s: fp32 [R, G].
//   bf16: the rows are bfloat16 instead of fp16.
hipError_t launch_quant_rows(const void* x, int64_t R, int64_t K, int group_size, int qmax,
                             void* q, float* s, hipStream_t stream, bool bf16 = false);

// The same with percentile-clipped scales: s = t / qmax, t = the percentile
// (0..100) of the group's magnitudes (linear interpolation between order
// statistics, fp64, rounded to fp32). R * K / group size groups, one
// workgroup each.
hipError_t launch_quant_rows_clip(const void* x, int64_t R, int64_t K, int group_size, int qmax,
                                  double percentile, void* q, float* s, hipStream_t stream, bool bf16 = false);

// Epilogue kinds of the GEMM kernels. kEpiF16Tok: per-group weight scales
// [N, G] with per-token activation scales [M] (int8 weights, gs 64 / 128).
// kEpiF16Split: per-channel fp16 output whose columns go to up to 4 separate
// matrices (GemmArgs::split).
// kEpiF16Linear: the GEMV kernel takes fp16 activations and quantizes them
// itself (per token), then dequantizes as kEpiF16.
// kEpiBF16: as kEpiF16 with a bfloat16 output; kEpiBF16Tok: as kEpiF16Tok
// with a bfloat16 output; kEpiBF16Linear: as kEpiF16Linear with bfloat16
// activations and output; kEpiBF16Split: as kEpiF16Split with bfloat16
// output matrices.
enum Epilogue {
  kEpiF16 = 0, kEpiAccI32 = 1, kEpiF16Tok = 2, kEpiF16Split = 3, kEpiF16Linear = 4, kEpiBF16 = 5, kEpiBF16Tok = 6,
  kEpiBF16Linear = 7, kEpiBF16Split = 8
};

// Column split of a GEMM's output: columns [end[i-1], end[i]) (end[-1] = 0)
// go to y[i], a row-major fp16 (bf16 for kEpiBF16Split) matrix of
// end[i] - end[i-1] columns. Unused
// trailing parts repeat the last end and are never selected.
constexpr int kMaxSplitParts = 4;
struct OutSplit {
  _Float16* y[kMaxSplitParts];
  int end[kMaxSplitParts];
};

// Weight encodings of the GEMM kernels.
enum WeightKind { kWeightI8 = 0, kWeightI4 = 1 };

struct GemmArgs {
  const int8_t* a;   // activation codes [M, K]
  const float* sa;   // activation scales [M] or [M, G] ([M] for kEpiF16Tok)
  const void* w;     // weight codes [N, K] int8 or packed [N, K/2]
  const float* sw;   // weight scales [N] or [N, G]
  int64_t M, N, K;
  int group_size;    // 0, 64, 128
  void* y;           // fp16 [M, N]
  int32_t* acc;      // int32 [M, N] or [G, M, N] (accumulator test hook)
  void* ws = nullptr;     // split-K workspace (counters zero on entry), or null
  int64_t ws_bytes = 0;
  OutSplit split{};       // kEpiF16Split only
};

hipError_t launch_gemm(const GemmArgs& args, WeightKind wk, Epilogue epi, hipStream_t stream);

// True when the one-launch linear applies: per-channel, M <= 2, K a multiple
// of 16 (32 for int4 weights) and the activation codes fit the GEMV kernel's
// LDS staging. (From M = 3 on, the activation quantization that every block
// repeats costs more than the separate quantization launch it saves.)
bool linear_is_one_launch(int64_t M, int64_t K, int group_size, WeightKind wk);

// Workspace bytes the GEMM dispatch uses for split-K at this shape (0: none).
int64_t gemm_split_workspace_bytes(int64_t M, int64_t N, int64_t K, WeightKind wk, int group_size);

struct MvArgs {
  const void* x;     // fp16 activations [M, K], 1 <= M <= 4
  const int8_t* w;   // int8 weight codes [N, K]
  const float* sw;   // weight scales [N] or [N, K / group_size]
  int64_t M, N, K;
  int group_size;    // 0, 64, 128
  void* y;           // fp16 [M, N]
};

// Decode matrix-vector product (no activation quantization).
hipError_t launch_mv(const MvArgs& args, hipStream_t stream);

// One pass over bytes (a multiple of 16) of buf; sink receives nothing
// (written only for an impossible data pattern).
hipError_t launch_read_probe(const void* buf, int64_t bytes, int32_t* sink, hipStream_t stream);

}  // namespace cider
