// Streaming-read reference for the rooflines: one plain read of a buffer.
//
// Not a step of the method.  The Full scan is bound by HBM reads, so its
// achieved bandwidth is reported against the nominal 8 TB/s and also against
// what this machine's HBM delivers to the simplest possible reader: every
// workgroup reads one contiguous chunk with 16-byte nontemporal loads into
// VGPRs, eight in flight per thread, and folds them into one word that is
// stored only if it equals a constant that a sum of loaded values is never
// compared to before (so the loads cannot be dropped, and nothing is
// written).
#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void k_stream_read(const v4u* __restrict__ p, int64_t n16,
                                                               int64_t chunk16, uint32_t* sink) {
  const int64_t b = (int64_t)blockIdx.x * chunk16;
  const int64_t e = b + chunk16 < n16 ? b + chunk16 : n16;
  v4u acc = {0u, 0u, 0u, 0u};
  for (int64_t i = b + threadIdx.x; i < e; i += (int64_t)kReadThreads * kReadUnroll) {
    v4u x[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t j = i + (int64_t)u * kReadThreads;
      x[u] = j < e ? __builtin_nontemporal_load(p + j) : v4u{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= x[u];
  }
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x9E3779B9u) sink[0] = r;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int cus, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 <= 0) return hipSuccess;
  const int64_t wgs = 2 * (int64_t)cus;                 // one round of two workgroups per CU
  const int64_t chunk = (n16 + wgs - 1) / wgs;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)wgs), dim3(kReadThreads), 0, s, (const v4u*)buf, n16, chunk,
                     sink);
  return hipGetLastError();
}

}  // namespace csa2
