// Reference kernels for the benchmark's context figures, beside the 8 TB/s denominator: the
// cost of one empty launch back to back, and the rate of a plain read stream.  Not part of the
// verification library (libspecbench.so, loaded by bench.py only).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadLoads = 16;  // 16-byte loads per thread in flight: 64 KB per workgroup

__global__ void k_empty() {}

// Each workgroup reads one contiguous 64 KB block with 16-byte nontemporal loads, all in
// flight together, and folds them so the loads are kept.
__global__ __launch_bounds__(kReadThreads) void k_read(const u32x4 *__restrict__ p, int64_t n16,
                                                       uint32_t *sink) {
  const int64_t base = (int64_t)blockIdx.x * (kReadThreads * kReadLoads);
  uint32_t acc = 0;
#pragma unroll
  for (int j = 0; j < kReadLoads; ++j) {
    const int64_t i = base + j * kReadThreads + threadIdx.x;
    if (i < n16) {
      const u32x4 v = __builtin_nontemporal_load(p + i);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;  // almost never taken; keeps the loads
}

}  // namespace

extern "C" {

// n back-to-back launches of an empty one-wavefront kernel on `stream`.
int spec_bench_empty(int n, void *stream) {
  for (int i = 0; i < n; ++i) k_empty<<<1, 64, 0, static_cast<hipStream_t>(stream)>>>();
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// One read of `bytes` (a multiple of 16) at device pointer `p`; `sink` is one device uint32.
int spec_bench_read(const void *p, int64_t bytes, uint32_t *sink, void *stream) {
  if (!p || !sink || bytes < 16) return -1;
  const int64_t n16 = bytes / 16;
  const int64_t grid = (n16 + kReadThreads * kReadLoads - 1) / (kReadThreads * kReadLoads);
  if (grid > INT32_MAX) return -2;
  k_read<<<(unsigned)grid, kReadThreads, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4 *>(p), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
