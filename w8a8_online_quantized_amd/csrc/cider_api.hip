// C ABI of libcider (declared in include/cider.h): argument validation,
// device gate and kernel dispatch. Every argument check runs before the first
// HIP call, so a bad call returns CIDER_ERROR_INVALID_VALUE with nothing
// enqueued, also on a machine without a GPU.
#include "../../include/cider.h"

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>

#include "cider_internal.h"

namespace {

constexpr int kVersion = 100;   // 0.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_gs(int32_t gs) { return gs == 0 || gs == 64 || gs == 128; }

// K must be a positive multiple of `mult` (1 for int8 codes, 2 for packed
// int4, 16 where a kernel family needs aligned rows), at most CIDER_MAX_K,
// and a multiple of the group size.
bool valid_k(int64_t K, int64_t mult, int32_t gs) {
  if (K <= 0 || K > CIDER_MAX_K || K % mult) return false;
  return gs == 0 || K % gs == 0;
}

// Per-device architecture flag: 1 = gfx950, 0 = other, -1 = not yet queried.
constexpr int kMaxDevices = 64;
struct ArchCache {
  std::atomic<int> ok[kMaxDevices];
  ArchCache() {
    for (auto& a : ok) a.store(-1);
  }
};

ArchCache& arch_cache() {
  static ArchCache cache;   // thread-safe one-time construction
  return cache;
}

bool device_is_gfx950() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return false;
  if (dev < kMaxDevices) {
    const int cached = arch_cache().ok[dev].load();
    if (cached >= 0) return cached == 1;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) arch_cache().ok[dev].store(ok ? 1 : 0);
  return ok;
}

cider_status_t from_hip(hipError_t e) { return e == hipSuccess ? CIDER_SUCCESS : CIDER_ERROR_LAUNCH; }

// Split-K scratch of cider_w8a8_gemm_noalloc (for callers that cannot
// allocate). Every GPU that loads the library holds its own copy of this
// array until the process ends; in host code its name is only a stand-in, so
// the kernels get the device address looked up below, never the name.
static __device__ __align__(256) int8_t scratch[CIDER_NOALLOC_SCRATCH_BYTES];

// This device's address of `scratch`, looked up on the device's first
// no-allocation call (with the device current) and kept; null if the lookup
// fails.
std::atomic<void*> g_scratch[kMaxDevices];
std::atomic<int> g_scratch_state[kMaxDevices];   // 0 = not looked up, 1 = ok, 2 = failed
std::mutex g_scratch_mu;

void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (g_scratch_state[dev].load(std::memory_order_acquire) == 0) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_state[dev].load(std::memory_order_relaxed) == 0) {
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      g_scratch[dev].store(e == hipSuccess ? ptr : nullptr, std::memory_order_relaxed);
      g_scratch_state[dev].store(e == hipSuccess && ptr ? 1 : 2, std::memory_order_release);
    }
  }
  return g_scratch_state[dev].load(std::memory_order_acquire) == 1 ? g_scratch[dev].load() : nullptr;
}

}  // namespace

extern "C" {

int cider_version(void) { return kVersion; }

const char* cider_status_string(cider_status_t s) {
  switch (s) {
    case CIDER_SUCCESS: return "success";
    case CIDER_ERROR_INVALID_VALUE: return "invalid argument (null/misaligned pointer, bad size or group size)";
    case CIDER_ERROR_NOT_SUPPORTED: return "not supported (no gfx950 device is current)";
    case CIDER_ERROR_LAUNCH: return "kernel launch failed";
    case CIDER_ERROR_SCRATCH_LIMIT:
      return "the shape's split-K plan needs more scratch than cider_w8a8_gemm_noalloc holds "
             "(CIDER_NOALLOC_SCRATCH_BYTES = 48 MiB)";
  }
  return "unknown status";
}

int cider_is_available(void) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return 0;
  return device_is_gfx950() ? 1 : 0;
}

static bool valid_dtype(int32_t d) { return d == CIDER_DTYPE_F16 || d == CIDER_DTYPE_BF16; }

cider_status_t cider_quant_act_dt(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t group_size,
                                  int8_t* x_q, float* x_scale, void* stream) {
  if (!valid_dtype(x_dtype)) return CIDER_ERROR_INVALID_VALUE;
  if (M < 0 || !valid_gs(group_size) || !valid_k(K, 1, group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (M == 0) return CIDER_SUCCESS;
  if (!x || !x_q || !x_scale || !aligned16(x) || !aligned16(x_q) || !aligned16(x_scale))
    return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  return from_hip(cider::launch_quant_rows(x, M, K, group_size, 127, x_q, x_scale, static_cast<hipStream_t>(stream),
                                           x_dtype == CIDER_DTYPE_BF16));
}

cider_status_t cider_quant_act(const void* x_f16, int64_t M, int64_t K, int32_t group_size, int8_t* x_q,
                               float* x_scale, void* stream) {
  return cider_quant_act_dt(x_f16, CIDER_DTYPE_F16, M, K, group_size, x_q, x_scale, stream);
}

cider_status_t cider_quant_weight(const void* w_f16, int64_t N, int64_t K, int32_t bits, int32_t group_size,
                                  void* w_q, float* w_scale, void* stream) {
  return cider_quant_weight_dt(w_f16, CIDER_DTYPE_F16, N, K, bits, group_size, w_q, w_scale, stream);
}

cider_status_t cider_quant_weight_dt(const void* w, int32_t w_dtype, int64_t N, int64_t K, int32_t bits,
                                     int32_t group_size, void* w_q, float* w_scale, void* stream) {
  if (!valid_dtype(w_dtype)) return CIDER_ERROR_INVALID_VALUE;
  const void* w_f16 = w;
  if (N < 0 || !valid_gs(group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (bits == 8) {
    if (!valid_k(K, 1, group_size)) return CIDER_ERROR_INVALID_VALUE;
  } else if (bits == 4) {
    if (group_size != 0 || !valid_k(K, 2, 0)) return CIDER_ERROR_INVALID_VALUE;
  } else {
    return CIDER_ERROR_INVALID_VALUE;
  }
  if (N == 0) return CIDER_SUCCESS;
  if (!w_f16 || !w_q || !w_scale || !aligned16(w_f16) || !aligned16(w_q) || !aligned16(w_scale))
    return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  return from_hip(cider::launch_quant_rows(w_f16, N, K, group_size, bits == 8 ? 127 : 7, w_q, w_scale,
                                           static_cast<hipStream_t>(stream), w_dtype == CIDER_DTYPE_BF16));
}

cider_status_t cider_quant_weight_clip(const void* w_f16, int32_t w_dtype, int64_t N, int64_t K, int32_t bits,
                                       int32_t group_size, double percentile, void* w_q, float* w_scale,
                                       void* stream) {
  if (!valid_dtype(w_dtype) || N < 0 || !valid_gs(group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (!(percentile >= 0.0 && percentile <= 100.0)) return CIDER_ERROR_INVALID_VALUE;   // NaN fails too
  if (bits == 8) {
    if (!valid_k(K, 16, group_size)) return CIDER_ERROR_INVALID_VALUE;
  } else if (bits == 4) {
    if (group_size != 0 || !valid_k(K, 32, 0)) return CIDER_ERROR_INVALID_VALUE;
  } else {
    return CIDER_ERROR_INVALID_VALUE;
  }
  const int64_t G = group_size ? K / group_size : 1;
  if (N * G >= (int64_t(1) << 31)) return CIDER_ERROR_INVALID_VALUE;
  if (N == 0) return CIDER_SUCCESS;
  if (!w_f16 || !w_q || !w_scale || !aligned16(w_f16) || !aligned16(w_q) || !aligned16(w_scale))
    return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  return from_hip(cider::launch_quant_rows_clip(w_f16, N, K, group_size, bits == 8 ? 127 : 7, percentile, w_q,
                                                w_scale, static_cast<hipStream_t>(stream),
                                                w_dtype == CIDER_DTYPE_BF16));
}

static cider_status_t gemm_common(cider::GemmArgs& g, cider::WeightKind wk, cider::Epilogue epi,
                                  void* stream) {
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  return from_hip(cider::launch_gemm(g, wk, epi, static_cast<hipStream_t>(stream)));
}

static bool gemm_sizes_ok(int64_t M, int64_t N) {
  return M >= 0 && N >= 0 && M < (int64_t(1) << 31) && N < (int64_t(1) << 31);
}

cider_status_t cider_w8a8_gemm(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                               const float* w_scale, int64_t M, int64_t N, int64_t K, int32_t group_size,
                               void* y_f16, void* stream) {
  return cider_w8a8_gemm_dt(x_q, x_scale, w_q, w_scale, M, N, K, group_size, y_f16, CIDER_DTYPE_F16, stream);
}

int64_t cider_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t bits, int32_t group_size) {
  if (!gemm_sizes_ok(M, N) || !valid_gs(group_size) || (bits != 8 && bits != 4)) return -1;
  if (bits == 4 && (group_size != 0 || !valid_k(K, 2, 0))) return -1;
  if (bits == 8 && !valid_k(K, 1, group_size)) return -1;
  if (M == 0 || N == 0) return 0;
  return cider::gemm_split_workspace_bytes(M, N, K, bits == 4 ? cider::kWeightI4 : cider::kWeightI8, group_size);
}

// A caller workspace, when given, must hold the size query's bytes.
static bool workspace_ok(const void* ws, int64_t ws_bytes, int64_t need) {
  if (!ws) return true;
  return aligned16(ws) && ws_bytes >= need;
}

cider_status_t cider_w8a8_gemm_dt(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, int32_t group_size,
                                  void* y_f16, int32_t y_dtype, void* stream) {
  return cider_w8a8_gemm_ex(x_q, x_scale, w_q, w_scale, M, N, K, group_size, y_f16, y_dtype, nullptr, 0, stream);
}

cider_status_t cider_w8a8_gemm_ex(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, int32_t group_size,
                                  void* y_f16, int32_t y_dtype, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
  if (!valid_dtype(y_dtype)) return CIDER_ERROR_INVALID_VALUE;
  if (!gemm_sizes_ok(M, N) || !valid_gs(group_size) || !valid_k(K, 1, group_size))
    return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_q || !x_scale || !w_q || !w_scale || !y_f16) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_q) || !aligned16(x_scale) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y_f16))
    return CIDER_ERROR_INVALID_VALUE;
  if (!workspace_ok(workspace, workspace_bytes, cider_gemm_workspace_size(M, N, K, 8, group_size)))
    return CIDER_ERROR_INVALID_VALUE;
  cider::GemmArgs g{x_q, x_scale, w_q, w_scale, M, N, K, group_size, y_f16, nullptr};
  g.ws = workspace;
  g.ws_bytes = workspace ? workspace_bytes : 0;
  return gemm_common(g, cider::kWeightI8, y_dtype == CIDER_DTYPE_BF16 ? cider::kEpiBF16 : cider::kEpiF16, stream);
}

cider_status_t cider_w8a8_gemm_noalloc(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                       const float* w_scale, int64_t M, int64_t N, int64_t K, int32_t group_size,
                                       void* y, int32_t y_dtype, void* stream) {
  if (!valid_dtype(y_dtype)) return CIDER_ERROR_INVALID_VALUE;
  if (!gemm_sizes_ok(M, N) || !valid_gs(group_size) || !valid_k(K, 1, group_size))
    return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_q || !x_scale || !w_q || !w_scale || !y) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_q) || !aligned16(x_scale) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y))
    return CIDER_ERROR_INVALID_VALUE;
  const int64_t need = cider_gemm_workspace_size(M, N, K, 8, group_size);
  if (need > CIDER_NOALLOC_SCRATCH_BYTES) return CIDER_ERROR_SCRATCH_LIMIT;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  cider::GemmArgs g{x_q, x_scale, w_q, w_scale, M, N, K, group_size, y, nullptr};
  if (need > 0) {
    // every slab element the reduction reads is written first by the same
    // call's split kernel, so nothing in the scratch needs clearing
    g.ws = scratch_address();
    if (!g.ws) return CIDER_ERROR_LAUNCH;
    g.ws_bytes = CIDER_NOALLOC_SCRATCH_BYTES;
  }
  return from_hip(cider::launch_gemm(g, cider::kWeightI8,
                                     y_dtype == CIDER_DTYPE_BF16 ? cider::kEpiBF16 : cider::kEpiF16,
                                     static_cast<hipStream_t>(stream)));
}

cider_status_t cider_w4a8_gemm(const int8_t* x_q, const float* x_scale, const uint8_t* w_packed,
                               const float* w_scale, int64_t M, int64_t N, int64_t K, void* y_f16,
                               void* stream) {
  return cider_w4a8_gemm_dt(x_q, x_scale, w_packed, w_scale, M, N, K, y_f16, CIDER_DTYPE_F16, stream);
}

cider_status_t cider_w4a8_gemm_dt(const int8_t* x_q, const float* x_scale, const uint8_t* w_packed,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* y_f16,
                                  int32_t y_dtype, void* stream) {
  return cider_w4a8_gemm_ex(x_q, x_scale, w_packed, w_scale, M, N, K, y_f16, y_dtype, nullptr, 0, stream);
}

cider_status_t cider_w4a8_gemm_ex(const int8_t* x_q, const float* x_scale, const uint8_t* w_packed,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* y_f16,
                                  int32_t y_dtype, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!valid_dtype(y_dtype)) return CIDER_ERROR_INVALID_VALUE;
  if (!gemm_sizes_ok(M, N) || !valid_k(K, 2, 0)) return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_q || !x_scale || !w_packed || !w_scale || !y_f16) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_q) || !aligned16(x_scale) || !aligned16(w_packed) || !aligned16(w_scale) ||
      !aligned16(y_f16))
    return CIDER_ERROR_INVALID_VALUE;
  if (!workspace_ok(workspace, workspace_bytes, cider_gemm_workspace_size(M, N, K, 4, 0)))
    return CIDER_ERROR_INVALID_VALUE;
  cider::GemmArgs g{x_q, x_scale, w_packed, w_scale, M, N, K, 0, y_f16, nullptr};
  g.ws = workspace;
  g.ws_bytes = workspace ? workspace_bytes : 0;
  return gemm_common(g, cider::kWeightI4, y_dtype == CIDER_DTYPE_BF16 ? cider::kEpiBF16 : cider::kEpiF16, stream);
}

cider_status_t cider_w8a8_gemm_token_group_dt(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                              const float* w_scale, int64_t M, int64_t N, int64_t K,
                                              int32_t group_size, void* y, int32_t y_dtype, void* workspace,
                                              int64_t workspace_bytes, void* stream) {
  if (!valid_dtype(y_dtype)) return CIDER_ERROR_INVALID_VALUE;
  if (!gemm_sizes_ok(M, N) || (group_size != 64 && group_size != 128) || !valid_k(K, 16, group_size))
    return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_q || !x_scale || !w_q || !w_scale || !y) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_q) || !aligned16(x_scale) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y))
    return CIDER_ERROR_INVALID_VALUE;
  if (!workspace_ok(workspace, workspace_bytes, cider_gemm_workspace_size(M, N, K, 8, group_size)))
    return CIDER_ERROR_INVALID_VALUE;
  cider::GemmArgs g{x_q, x_scale, w_q, w_scale, M, N, K, group_size, y, nullptr};
  g.ws = workspace;
  g.ws_bytes = workspace ? workspace_bytes : 0;
  return gemm_common(g, cider::kWeightI8, y_dtype == CIDER_DTYPE_BF16 ? cider::kEpiBF16Tok : cider::kEpiF16Tok,
                     stream);
}

cider_status_t cider_w8a8_gemm_token_group(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                           const float* w_scale, int64_t M, int64_t N, int64_t K,
                                           int32_t group_size, void* y_f16, void* workspace,
                                           int64_t workspace_bytes, void* stream) {
  return cider_w8a8_gemm_token_group_dt(x_q, x_scale, w_q, w_scale, M, N, K, group_size, y_f16, CIDER_DTYPE_F16,
                                        workspace, workspace_bytes, stream);
}

cider_status_t cider_w8a8_gemm_split_dt(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                        const float* w_scale, int64_t M, int64_t K, int32_t n_parts,
                                        const int64_t* part_n, void* const* y_parts, int32_t y_dtype,
                                        void* stream) {
  if (!valid_dtype(y_dtype)) return CIDER_ERROR_INVALID_VALUE;
  if (M < 0 || M >= (int64_t(1) << 31) || !valid_k(K, 16, 0)) return CIDER_ERROR_INVALID_VALUE;
  if (n_parts < 1 || n_parts > CIDER_SPLIT_MAX_PARTS || !part_n || !y_parts) return CIDER_ERROR_INVALID_VALUE;
  cider::OutSplit sp{};
  int64_t N = 0;
  for (int32_t i = 0; i < n_parts; ++i) {
    if (part_n[i] <= 0 || part_n[i] % 16 != 0) return CIDER_ERROR_INVALID_VALUE;
    N += part_n[i];
    if (N >= (int64_t(1) << 31)) return CIDER_ERROR_INVALID_VALUE;
    sp.y[i] = static_cast<_Float16*>(y_parts[i]);
    sp.end[i] = (int)N;
  }
  for (int32_t i = n_parts; i < CIDER_SPLIT_MAX_PARTS; ++i) {
    sp.y[i] = sp.y[n_parts - 1];
    sp.end[i] = (int)N;
  }
  if (M == 0) return CIDER_SUCCESS;
  if (!x_q || !x_scale || !w_q || !w_scale) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_q) || !aligned16(x_scale) || !aligned16(w_q) || !aligned16(w_scale)) return CIDER_ERROR_INVALID_VALUE;
  for (int32_t i = 0; i < n_parts; ++i)
    if (!y_parts[i] || !aligned16(y_parts[i])) return CIDER_ERROR_INVALID_VALUE;
  cider::GemmArgs g{x_q, x_scale, w_q, w_scale, M, N, K, 0, sp.y[0], nullptr};
  g.split = sp;
  return gemm_common(g, cider::kWeightI8, y_dtype == CIDER_DTYPE_BF16 ? cider::kEpiBF16Split : cider::kEpiF16Split,
                     stream);
}

cider_status_t cider_w8a8_gemm_split(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                     const float* w_scale, int64_t M, int64_t K, int32_t n_parts,
                                     const int64_t* part_n, void* const* y_parts, void* stream) {
  return cider_w8a8_gemm_split_dt(x_q, x_scale, w_q, w_scale, M, K, n_parts, part_n, y_parts, CIDER_DTYPE_F16,
                                  stream);
}

// The one-call linear's workspace: the activation codes and scales (each
// 256-byte aligned), then room for the GEMM's split-K slabs.
static int64_t linear_quant_bytes(int64_t M, int64_t K, int32_t group_size) {
  const int64_t G = group_size ? K / group_size : 1;
  return (M * K + 255) / 256 * 256 + (4 * M * G + 255) / 256 * 256;
}

int64_t cider_linear_workspace_size(int64_t M, int64_t N, int64_t K, int32_t bits, int32_t group_size) {
  if (!gemm_sizes_ok(M, N) || !valid_gs(group_size) || (bits != 8 && bits != 4)) return -1;
  if (bits == 4 && group_size != 0) return -1;
  if (!valid_k(K, bits == 4 ? 2 : 1, group_size)) return -1;
  if (M == 0 || N == 0 || cider::linear_is_one_launch(M, K, group_size, bits == 4 ? cider::kWeightI4 : cider::kWeightI8)) return 0;
  return linear_quant_bytes(M, K, group_size) + cider_gemm_workspace_size(M, N, K, bits, group_size);
}

cider_status_t cider_linear_dt(const void* x_f16, int32_t dtype, const void* w, const float* w_scale, int64_t M,
                               int64_t N, int64_t K, int32_t bits, int32_t group_size, void* workspace,
                               int64_t workspace_bytes, void* y_f16, void* stream) {
  if (!valid_dtype(dtype)) return CIDER_ERROR_INVALID_VALUE;
  const bool bf = dtype == CIDER_DTYPE_BF16;
  const int64_t need = cider_linear_workspace_size(M, N, K, bits, group_size);
  if (need < 0) return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_f16 || !w || !w_scale || !y_f16) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_f16) || !aligned16(w) || !aligned16(w_scale) || !aligned16(y_f16)) return CIDER_ERROR_INVALID_VALUE;
  if (need > 0 && (!workspace || !aligned16(workspace) || workspace_bytes < need)) return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  const cider::WeightKind wk = bits == 4 ? cider::kWeightI4 : cider::kWeightI8;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (need == 0) {   // one launch: the GEMV kernel quantizes its activations itself
    cider::GemmArgs g{static_cast<const int8_t*>(x_f16), nullptr, w, w_scale, M, N, K, 0, y_f16, nullptr};
    return from_hip(cider::launch_gemm(g, wk, bf ? cider::kEpiBF16Linear : cider::kEpiF16Linear, st));
  }
  int8_t* xq = static_cast<int8_t*>(workspace);
  float* sa = reinterpret_cast<float*>(static_cast<char*>(workspace) + (M * K + 255) / 256 * 256);
  hipError_t e = cider::launch_quant_rows(x_f16, M, K, group_size, 127, xq, sa, st, bf);
  if (e != hipSuccess) return from_hip(e);
  cider::GemmArgs g{xq, sa, w, w_scale, M, N, K, group_size, y_f16, nullptr};
  const int64_t qb = linear_quant_bytes(M, K, group_size);
  if (need > qb) {   // the split-K slabs follow the codes and scales
    g.ws = static_cast<char*>(workspace) + qb;
    g.ws_bytes = workspace_bytes - qb;
  }
  return from_hip(cider::launch_gemm(g, wk, bf ? cider::kEpiBF16 : cider::kEpiF16, st));
}

cider_status_t cider_linear(const void* x_f16, const void* w, const float* w_scale, int64_t M, int64_t N,
                            int64_t K, int32_t bits, int32_t group_size, void* workspace,
                            int64_t workspace_bytes, void* y_f16, void* stream) {
  return cider_linear_dt(x_f16, CIDER_DTYPE_F16, w, w_scale, M, N, K, bits, group_size, workspace, workspace_bytes,
                         y_f16, stream);
}

cider_status_t cider_int8_mv(const void* x_f16, const int8_t* w_q, const float* w_scale, int64_t M, int64_t N,
                             int64_t K, int32_t group_size, void* y_f16, void* stream) {
  if (M < 0 || M > CIDER_MV_MAX_M || !gemm_sizes_ok(M, N) || !valid_gs(group_size) || !valid_k(K, 16, group_size))
    return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_f16 || !w_q || !w_scale || !y_f16) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_f16) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y_f16))
    return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  cider::MvArgs a{x_f16, w_q, w_scale, M, N, K, group_size, y_f16};
  return from_hip(cider::launch_mv(a, static_cast<hipStream_t>(stream)));
}

cider_status_t cider_read_probe(const void* buf, int64_t bytes, int32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16) return CIDER_ERROR_INVALID_VALUE;
  if (bytes == 0) return CIDER_SUCCESS;
  if (!buf || !sink || !aligned16(buf) || !aligned16(sink)) return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  return from_hip(cider::launch_read_probe(buf, bytes, sink, static_cast<hipStream_t>(stream)));
}

cider_status_t cider_gemm_acc_i32(int32_t mode, const int8_t* x_q, const void* w, int64_t M, int64_t N,
                                  int64_t K, int32_t group_size, int32_t* acc, void* stream) {
  if (mode != 0 && mode != 1) return CIDER_ERROR_INVALID_VALUE;
  if (!gemm_sizes_ok(M, N) || !valid_gs(group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (mode == 1 && (group_size != 0 || !valid_k(K, 2, 0))) return CIDER_ERROR_INVALID_VALUE;
  if (mode == 0 && !valid_k(K, 1, group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_q || !w || !acc || !aligned16(x_q) || !aligned16(w) || !aligned16(acc)) return CIDER_ERROR_INVALID_VALUE;
  cider::GemmArgs g{x_q, nullptr, w, nullptr, M, N, K, group_size, nullptr, acc};
  return gemm_common(g, mode == 1 ? cider::kWeightI4 : cider::kWeightI8, cider::kEpiAccI32, stream);
}

}  // extern "C"

// Stack workspace regions 0..8 (see include/cider.h) plus region 9: the int32
// partial sums of a split-K GEMM (the largest the stack's per-projection GEMMs
// need; 0 bytes when none splits). Returns the total, 0 for invalid dims.
static int64_t stack_layout(int64_t M, int64_t hidden, int64_t q_dim, int64_t kv_dim, int64_t mlp_dim,
                            int64_t off[10]) {
  if (M < 0 || hidden <= 0 || q_dim <= 0 || kv_dim <= 0 || mlp_dim <= 0) return 0;
  if (hidden % 16 || q_dim % 16 || kv_dim % 16 || mlp_dim % 16) return 0;
  const int64_t kmax = std::max(hidden, std::max(q_dim, mlp_dim));
  int64_t split = 0;
  if (M > 0) {
    const int64_t nk[4][2] = {{q_dim, hidden}, {kv_dim, hidden}, {hidden, q_dim}, {mlp_dim, hidden}};
    for (const auto& p : nk)
      split = std::max(split, cider::gemm_split_workspace_bytes(M, p[0], p[1], cider::kWeightI8, 0));
    split = std::max(split, cider::gemm_split_workspace_bytes(M, hidden, mlp_dim, cider::kWeightI8, 0));
  }
  const int64_t sizes[10] = {M * kmax, 4 * M, 2 * M * q_dim, 2 * M * kv_dim, 2 * M * kv_dim,
                             2 * M * hidden, 2 * M * mlp_dim, 2 * M * mlp_dim, 2 * M * hidden, split};
  int64_t o = 0;
  for (int i = 0; i < 10; ++i) {
    off[i] = o;
    o += (sizes[i] + 255) / 256 * 256;
  }
  return o;
}

extern "C" {

int64_t cider_stack_workspace_layout(int64_t M, int64_t hidden, int64_t q_dim, int64_t kv_dim, int64_t mlp_dim,
                                     int64_t* offsets) {
  int64_t off[10];
  const int64_t total = stack_layout(M, hidden, q_dim, kv_dim, mlp_dim, off);
  if (total && offsets)
    for (int i = 0; i < 9; ++i) offsets[i] = off[i];
  return total;
}

cider_status_t cider_stack_forward_dt(const void* x_f16, int32_t dtype, int64_t M, int64_t hidden, int64_t q_dim,
                                      int64_t kv_dim, int64_t mlp_dim, int32_t n_layers,
                                      const cider_stack_layer_t* layers, void* workspace, int64_t workspace_bytes,
                                      void* y_f16, void* stream) {
  if (!valid_dtype(dtype)) return CIDER_ERROR_INVALID_VALUE;
  const bool bf = dtype == CIDER_DTYPE_BF16;
  int64_t off[10];
  const int64_t need = stack_layout(M, hidden, q_dim, kv_dim, mlp_dim, off);
  if (need == 0 || n_layers < 0 || M >= (int64_t(1) << 31)) return CIDER_ERROR_INVALID_VALUE;
  if (std::max(hidden, std::max(q_dim, mlp_dim)) > CIDER_MAX_K) return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || n_layers == 0) return CIDER_SUCCESS;
  if (!x_f16 || !layers || !workspace || !y_f16 || workspace_bytes < need) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_f16) || !aligned16(workspace) || !aligned16(y_f16)) return CIDER_ERROR_INVALID_VALUE;
  for (int32_t l = 0; l < n_layers; ++l)
    for (int j = 0; j < 7; ++j)
      if (!layers[l].w[j] || !layers[l].s[j] || !aligned16(layers[l].w[j]) || !aligned16(layers[l].s[j]))
        return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;

  char* ws = static_cast<char*>(workspace);
  int8_t* xq = reinterpret_cast<int8_t*>(ws + off[0]);
  float* sa = reinterpret_cast<float*>(ws + off[1]);
  void* q = ws + off[2];
  void* k = ws + off[3];
  void* v = ws + off[4];
  void* o = ws + off[5];
  void* g = ws + off[6];
  void* u = ws + off[7];
  void* h = ws + off[8];
  hipStream_t st = static_cast<hipStream_t>(stream);

  auto quant = [&](const void* in, int64_t K) { return cider::launch_quant_rows(in, M, K, 0, 127, xq, sa, st, bf); };
  auto gemm = [&](const cider_stack_layer_t& L, int j, int64_t N, int64_t K, void* out) {
    cider::GemmArgs a{xq, sa, L.w[j], L.s[j], M, N, K, 0, out, nullptr};
    // split-K partials (e.g. the long-K down projection); stream order keeps
    // one GEMM's partials from overlapping the next one's
    if (need > off[9]) {
      a.ws = ws + off[9];
      a.ws_bytes = need - off[9];
    }
    return cider::launch_gemm(a, cider::kWeightI8, bf ? cider::kEpiBF16 : cider::kEpiF16, st);
  };
  // Projections j, j+1[, j+2] of one input as one GEMM when their codes and
  // scales are adjacent in memory, in that order (columns split to `outs`).
  auto adjacent = [&](const cider_stack_layer_t& L, int j, int parts, const int64_t* n) {
    for (int i = 1; i < parts; ++i) {
      if (L.w[j + i] != L.w[j + i - 1] + n[i - 1] * hidden) return false;
      if (L.s[j + i] != L.s[j + i - 1] + n[i - 1]) return false;
    }
    return true;
  };
  auto gemm_fused = [&](const cider_stack_layer_t& L, int j, int parts, const int64_t* n, void* const* outs) {
    cider::GemmArgs a{xq, sa, L.w[j], L.s[j], M, 0, hidden, 0, outs[0], nullptr};
    int64_t end = 0;
    for (int i = 0; i < cider::kMaxSplitParts; ++i) {
      if (i < parts) end += n[i];
      a.split.y[i] = static_cast<_Float16*>(outs[i < parts ? i : parts - 1]);
      a.split.end[i] = (int)end;
    }
    a.N = end;
    return cider::launch_gemm(a, cider::kWeightI8, bf ? cider::kEpiBF16Split : cider::kEpiF16Split, st);
  };
  const int64_t n_qkv[3] = {q_dim, kv_dim, kv_dim}, n_gu[2] = {mlp_dim, mlp_dim};
  const void* in = x_f16;
  for (int32_t l = 0; l < n_layers; ++l) {
    const cider_stack_layer_t& L = layers[l];
    void* out = l + 1 == n_layers ? y_f16 : h;
    void* const qkv_out[3] = {q, k, v};
    void* const gu_out[2] = {g, u};
    hipError_t e = quant(in, hidden);
    if (adjacent(L, 0, 3, n_qkv)) {
      if (e == hipSuccess) e = gemm_fused(L, 0, 3, n_qkv, qkv_out);
    } else {
      if (e == hipSuccess) e = gemm(L, 0, q_dim, hidden, q);
      if (e == hipSuccess) e = gemm(L, 1, kv_dim, hidden, k);
      if (e == hipSuccess) e = gemm(L, 2, kv_dim, hidden, v);
    }
    if (e == hipSuccess) e = quant(q, q_dim);
    if (e == hipSuccess) e = gemm(L, 3, hidden, q_dim, o);
    if (e == hipSuccess) e = quant(o, hidden);
    if (adjacent(L, 4, 2, n_gu)) {
      if (e == hipSuccess) e = gemm_fused(L, 4, 2, n_gu, gu_out);
    } else {
      if (e == hipSuccess) e = gemm(L, 4, mlp_dim, hidden, g);
      if (e == hipSuccess) e = gemm(L, 5, mlp_dim, hidden, u);
    }
    if (e == hipSuccess) e = quant(u, mlp_dim);
    if (e == hipSuccess) e = gemm(L, 6, hidden, mlp_dim, out);
    if (e != hipSuccess) return CIDER_ERROR_LAUNCH;
    in = out;   // stream order: the next layer's first quant reads h before h is rewritten
  }
  return CIDER_SUCCESS;
}

cider_status_t cider_stack_forward(const void* x_f16, int64_t M, int64_t hidden, int64_t q_dim, int64_t kv_dim,
                                   int64_t mlp_dim, int32_t n_layers, const cider_stack_layer_t* layers,
                                   void* workspace, int64_t workspace_bytes, void* y_f16, void* stream) {
  return cider_stack_forward_dt(x_f16, CIDER_DTYPE_F16, M, hidden, q_dim, kv_dim, mlp_dim, n_layers, layers,
                                workspace, workspace_bytes, y_f16, stream);
}

}  // extern "C"
