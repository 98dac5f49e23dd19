// readprobe.hip -- the benchmark's read-bandwidth reference: one pass of
// 16-byte non-temporal loads over a device buffer, the access the scans make
// to their databases, with no arithmetic beyond an xor that keeps the loads
// live.  Not part of any scan; bench.py times it beside them so that their
// HBM fractions can be read against what a plain read stream reaches.
#include <hip/hip_runtime.h>

#include "internal.hpp"

namespace pirscan {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 8;                  // 4 KiB blocks in flight per workgroup
constexpr uint64_t kChunk = 64ull << 10;    // bytes per workgroup

// One workgroup per 64 KiB chunk, dispatched in address order, so the chunks
// in flight form one window that moves through the buffer as the scans'
// tiles do (measured on bench-sized buffers: 7.17 TB/s, against 6.70 TB/s
// for one long contiguous share per resident workgroup).  Per round the 256
// threads load kUnroll consecutive 4 KiB blocks (thread t the 16-byte word t
// of each).  A thread stores its xor only when it equals a run-time tag
// (rare, and harmless: the caller's sink word), which keeps the loads live.
__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4* __restrict__ src, uint64_t n,
                                                               uint32_t* __restrict__ sink, uint32_t tag) {
  constexpr uint64_t per = kChunk / 16;  // words per workgroup
  const uint64_t lo = blockIdx.x * per, hi = lo + per < n ? lo + per : n;
  u32x4 acc = {0u, 0u, 0u, 0u};
  uint64_t i = lo + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < hi; i += kUnroll * kThreads) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < hi; i += kThreads) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == tag) sink[0] = x;
}

}  // namespace

hipError_t launch_read_stream(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream) {
  const uint64_t grid = (bytes + kChunk - 1) / kChunk;
  if (grid == 0 || grid > 0x7FFFFFFFull) return hipErrorInvalidValue;
  timer_mark_start(stream);
  hipLaunchKernelGGL(read_stream_kernel, dim3((uint32_t)grid), dim3(kThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink, 0x9E3779B9u);
  const hipError_t e = hipGetLastError();
  timer_mark_stop(stream);
  return e;
}

}  // namespace pirscan
