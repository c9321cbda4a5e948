// Measurement helper: one cold pass over a device buffer, the single-launch
// HBM read ceiling that the bandwidth-bound small-M kernels (GEMV, decode MV)
// are compared against. Not part of the method.
#include <algorithm>

#include "cider_internal.h"

namespace cider {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

// Block b reads bytes [b * chunk, (b + 1) * chunk) of the buffer in 16-byte
// lanes, kUnroll loads in flight per lane, and folds them into a value that is
// stored only if it equals an impossible pattern (keeps the loads live).
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(256) read_probe_kernel(const v4i* __restrict__ p, int64_t n16, int64_t chunk,
                                                         int32_t* __restrict__ sink) {
  const int64_t b0 = (int64_t)blockIdx.x * chunk;
  const int64_t b1 = std::min(n16, b0 + chunk);
  v4i acc = {0, 0, 0, 0};
  for (int64_t base = b0 + threadIdx.x; base < b1; base += 256 * kUnroll) {
    v4i v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < b1 ? p[i] : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  const int s = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (s == 0x7F3C1A5D && threadIdx.x == 0) sink[0] = s;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t bytes, int32_t* sink, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  const int64_t blocks = std::min<int64_t>(4096, std::max<int64_t>(1, (n16 + 255) / 256));
  const int64_t chunk = (n16 + blocks - 1) / blocks;
  read_probe_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(static_cast<const v4i*>(buf), n16, chunk, sink);
  return hipGetLastError();
}

}  // namespace cider
