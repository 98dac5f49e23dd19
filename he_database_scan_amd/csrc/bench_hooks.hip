// bench_hooks.hip -- the benchmark instrumentation of libpirscan_bench.so
// (include/pirscan_bench.h): the per-thread kernel timer that the launchers
// drive through timer_mark_start / timer_mark_stop, and the read-stream
// reference.  Built only with PIRSCAN_BENCH_HOOKS=1; the product library
// libpirscan.so contains none of it.
#include <hip/hip_runtime.h>

#include <new>

#include "../../include/pirscan.h"
#include "../../include/pirscan_bench.h"
#include "internal.hpp"

#if !PIRSCAN_BENCH_HOOKS
#error "bench_hooks.hip belongs to the build with PIRSCAN_BENCH_HOOKS=1"
#endif

namespace {

// Timer state of one thread: `cap` event pairs, `count` recorded, `open`
// while a start has no stop yet.
struct KernelTimer {
  bool on = false, open = false;
  uint32_t cap = 0, count = 0;
  hipEvent_t* start = nullptr;
  hipEvent_t* stop = nullptr;
};
thread_local KernelTimer g_timer;

void timer_release() {
  for (uint32_t i = 0; i < g_timer.cap; ++i) {
    (void)hipEventDestroy(g_timer.start[i]);
    (void)hipEventDestroy(g_timer.stop[i]);
  }
  delete[] g_timer.start;
  delete[] g_timer.stop;
  g_timer = KernelTimer{};
}

}  // namespace

namespace pirscan {

void timer_mark_start(hipStream_t stream) {
  if (!g_timer.on || g_timer.open || g_timer.count >= g_timer.cap) return;
  if (hipEventRecord(g_timer.start[g_timer.count], stream) == hipSuccess) g_timer.open = true;
}

void timer_mark_stop(hipStream_t stream) {
  if (!g_timer.on || !g_timer.open) return;
  g_timer.open = false;
  if (hipEventRecord(g_timer.stop[g_timer.count], stream) == hipSuccess) ++g_timer.count;
}

}  // namespace pirscan

extern "C" {

int pirscan_kernel_timer_begin(uint32_t capacity) {
  if (capacity == 0 || capacity > (1u << 20)) return PIRSCAN_EINVAL;
  timer_release();
  g_timer.start = new (std::nothrow) hipEvent_t[capacity];
  g_timer.stop = new (std::nothrow) hipEvent_t[capacity];
  if (!g_timer.start || !g_timer.stop) {
    timer_release();
    return PIRSCAN_EINVAL;
  }
  for (uint32_t i = 0; i < capacity; ++i) {
    hipError_t e = hipEventCreate(&g_timer.start[i]);
    if (e == hipSuccess) {
      e = hipEventCreate(&g_timer.stop[i]);
      if (e != hipSuccess) (void)hipEventDestroy(g_timer.start[i]);
    }
    if (e != hipSuccess) {
      g_timer.cap = i;
      timer_release();
      return pirscan::api_device_status(e);
    }
    g_timer.cap = i + 1;
  }
  g_timer.on = true;
  return PIRSCAN_OK;
}

int pirscan_kernel_timer_end(float* ms, uint32_t max_count, uint32_t* count) {
  if (!g_timer.on) return PIRSCAN_EINVAL;
  const uint32_t n = g_timer.count < max_count ? g_timer.count : max_count;
  int st = PIRSCAN_OK;
  for (uint32_t i = 0; i < n && st == PIRSCAN_OK; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.stop[i]);
    if (e == hipSuccess && ms) e = hipEventElapsedTime(&ms[i], g_timer.start[i], g_timer.stop[i]);
    st = pirscan::api_device_status(e);
  }
  if (count) *count = st == PIRSCAN_OK ? n : 0;
  timer_release();
  return st;
}

int pirscan_bench_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0) return PIRSCAN_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0) return PIRSCAN_EINVAL;
  const int dc = pirscan::api_device_check();
  if (dc != PIRSCAN_OK) return dc;
  return pirscan::api_device_status(pirscan::launch_read_stream(buf, bytes, sink, (hipStream_t)stream));
}

}  // extern "C"
