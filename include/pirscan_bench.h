/*
 * pirscan_bench.h -- benchmark instrumentation of libpirscan, exported only by
 * libpirscan_bench.so: the library's sources compiled with the timing hooks
 * on (PIRSCAN_BENCH_HOOKS=1).  It also exports every entry point of
 * pirscan.h, with the same kernels and results; the product library
 * libpirscan.so exports none of the functions below.  Not part of the scan:
 * they let a benchmark price each scan's main kernel with HIP events on the
 * stream it runs on, and compare the scans with a plain read stream.
 */
#ifndef PIRSCAN_BENCH_H
#define PIRSCAN_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Kernel timer of the calling thread.
 * pirscan_kernel_timer_begin(capacity) makes the thread's next `capacity`
 * scan calls record a pair of HIP events on their stream around their main
 * kernel -- the scan kernel itself, without the per-query pre- and
 * post-passes (digit split, ct / output relayout, split-K reduction); the
 * passes of a batch wider than one kernel launch are timed as one interval.
 * pirscan_kernel_timer_end waits for the recorded events, writes the elapsed
 * milliseconds of each call, in call order, to the HOST array ms[0..*count)
 * (at most max_count entries) and turns the hook off.  The events belong to
 * the library.  Not for use under stream capture.  Returns PIRSCAN_EINVAL for
 * capacity 0 or > 2^20, or for _end without _begin.
 */
int pirscan_kernel_timer_begin(uint32_t capacity);
int pirscan_kernel_timer_end(float* ms, uint32_t max_count, uint32_t* count);

/*
 * Read-stream reference: one pass of 16-byte
 * non-temporal loads over `bytes` of the device buffer buf -- the access the
 * scans make to their databases, without their arithmetic -- so that a
 * scan's HBM rate can be compared with a plain read stream's on the same
 * device.  Timed by the kernel-timer hook like a scan call.  buf: device
 * memory, 16-byte aligned, bytes a non-zero multiple of 16, only read.
 * sink: device memory of at least 4 bytes that a thread may overwrite with
 * its running xor (which keeps the loads from being optimised away); its
 * contents are unspecified afterwards.  PIRSCAN_EINVAL otherwise.
 */
int pirscan_bench_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PIRSCAN_BENCH_H */
