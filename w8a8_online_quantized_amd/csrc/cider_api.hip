// C ABI of libcider (declared in include/cider.h): argument validation,
// device gate and kernel dispatch. Every argument check runs before the first
// HIP call, so a bad call returns CIDER_ERROR_INVALID_VALUE with nothing
// enqueued, also on a machine without a GPU.
#include "../../include/cider.h"

#include <atomic>
#include <cstring>

#include "cider_internal.h"

namespace {

constexpr int kVersion = 100;   // 0.1.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_gs(int32_t gs) { return gs == 0 || gs == 64 || gs == 128; }

// K must be a positive multiple of `mult`, at most CIDER_MAX_K, and a multiple
// of the group size.
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

}  // namespace

extern "C" {

int cider_version(void) { return kVersion; }

const char* cider_status_string(cider_status_t s) {
  switch (s) {
    case CIDER_SUCCESS: return "success";
    case CIDER_ERROR_INVALID_VALUE: return "invalid argument (null/misaligned pointer, bad size or group size)";
    case CIDER_ERROR_NOT_SUPPORTED: return "not supported (no gfx950 device is current)";
    case CIDER_ERROR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int cider_is_available(void) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return 0;
  return device_is_gfx950() ? 1 : 0;
}

cider_status_t cider_quant_act(const void* x_f16, int64_t M, int64_t K, int32_t group_size, int8_t* x_q,
                               float* x_scale, void* stream) {
  if (M < 0 || !valid_gs(group_size) || !valid_k(K, 16, group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (M == 0) return CIDER_SUCCESS;
  if (!x_f16 || !x_q || !x_scale || !aligned16(x_f16) || !aligned16(x_q) || !aligned16(x_scale))
    return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  return from_hip(cider::launch_quant_rows(x_f16, M, K, group_size, 127, x_q, x_scale,
                                           static_cast<hipStream_t>(stream)));
}

cider_status_t cider_quant_weight(const void* w_f16, int64_t N, int64_t K, int32_t bits, int32_t group_size,
                                  void* w_q, float* w_scale, void* stream) {
  if (N < 0 || !valid_gs(group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (bits == 8) {
    if (!valid_k(K, 16, group_size)) return CIDER_ERROR_INVALID_VALUE;
  } else if (bits == 4) {
    if (group_size != 0 || !valid_k(K, 32, 0)) return CIDER_ERROR_INVALID_VALUE;
  } else {
    return CIDER_ERROR_INVALID_VALUE;
  }
  if (N == 0) return CIDER_SUCCESS;
  if (!w_f16 || !w_q || !w_scale || !aligned16(w_f16) || !aligned16(w_q) || !aligned16(w_scale))
    return CIDER_ERROR_INVALID_VALUE;
  if (!device_is_gfx950()) return CIDER_ERROR_NOT_SUPPORTED;
  return from_hip(cider::launch_quant_rows(w_f16, N, K, group_size, bits == 8 ? 127 : 7, w_q, w_scale,
                                           static_cast<hipStream_t>(stream)));
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
  if (!gemm_sizes_ok(M, N) || !valid_gs(group_size) || !valid_k(K, 16, group_size))
    return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_q || !x_scale || !w_q || !w_scale || !y_f16) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_q) || !aligned16(x_scale) || !aligned16(w_q) || !aligned16(w_scale) || !aligned16(y_f16))
    return CIDER_ERROR_INVALID_VALUE;
  cider::GemmArgs g{x_q, x_scale, w_q, w_scale, M, N, K, group_size, y_f16, nullptr};
  return gemm_common(g, cider::kWeightI8, cider::kEpiF16, stream);
}

cider_status_t cider_w4a8_gemm(const int8_t* x_q, const float* x_scale, const uint8_t* w_packed,
                               const float* w_scale, int64_t M, int64_t N, int64_t K, void* y_f16,
                               void* stream) {
  if (!gemm_sizes_ok(M, N) || !valid_k(K, 32, 0)) return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_q || !x_scale || !w_packed || !w_scale || !y_f16) return CIDER_ERROR_INVALID_VALUE;
  if (!aligned16(x_q) || !aligned16(x_scale) || !aligned16(w_packed) || !aligned16(w_scale) ||
      !aligned16(y_f16))
    return CIDER_ERROR_INVALID_VALUE;
  cider::GemmArgs g{x_q, x_scale, w_packed, w_scale, M, N, K, 0, y_f16, nullptr};
  return gemm_common(g, cider::kWeightI4, cider::kEpiF16, stream);
}

cider_status_t cider_gemm_acc_i32(int32_t mode, const int8_t* x_q, const void* w, int64_t M, int64_t N,
                                  int64_t K, int32_t group_size, int32_t* acc, void* stream) {
  if (mode != 0 && mode != 1) return CIDER_ERROR_INVALID_VALUE;
  if (!gemm_sizes_ok(M, N) || !valid_gs(group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (mode == 1 && (group_size != 0 || !valid_k(K, 32, 0))) return CIDER_ERROR_INVALID_VALUE;
  if (mode == 0 && !valid_k(K, 16, group_size)) return CIDER_ERROR_INVALID_VALUE;
  if (M == 0 || N == 0) return CIDER_SUCCESS;
  if (!x_q || !w || !acc || !aligned16(x_q) || !aligned16(w) || !aligned16(acc)) return CIDER_ERROR_INVALID_VALUE;
  cider::GemmArgs g{x_q, nullptr, w, nullptr, M, N, K, group_size, nullptr, acc};
  return gemm_common(g, mode == 1 ? cider::kWeightI4 : cider::kWeightI8, cider::kEpiAccI32, stream);
}

}  // extern "C"
