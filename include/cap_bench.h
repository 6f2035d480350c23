/*
 * cap_bench.h -- measurement helpers exported by libcap (not part of the
 * attention path).  They exist so that timings of the attention kernels can
 * be taken with inputs resident in HBM rather than in on-chip caches, and so
 * that HBM-traffic counters can be calibrated against kernels of known size.
 * The CREDIT summary (section III.D, "Baseline Timing") warns that cache
 * residency makes peak-bandwidth assumptions unreliable; these helpers make
 * that effect controllable.
 *
 * All pointers are device pointers owned by the caller; sizes are bytes and
 * must be multiples of 16 with 16-byte aligned buffers.  Each call launches
 * one kernel on `stream` (a hipStream_t) and returns CAP_ERR_INVALID_ARG for
 * bad sizes/pointers or CAP_ERR_HIP if the launch fails.
 */
#ifndef CAP_BENCH_H
#define CAP_BENCH_H

#include "cap.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Write `value` to every 32-bit word of buf (evicts caches when buf is larger
 * than L2 + the 256 MB Infinity Cache). */
cap_status cap_bench_fill(void *buf, size_t bytes, uint32_t value, cap_stream_t stream);

/* Read every byte of buf once (128-bit loads, grid-stride, cached) and write
 * one 32-bit word per workgroup into sink (>= 4 x 8192 bytes) so the reads
 * are not dead.  Used to evict L2 and the Infinity Cache before a timed step
 * (reads allocate there; a fill would leave dirty lines behind). */
cap_status cap_bench_read(const void *buf, size_t bytes, void *sink, cap_stream_t stream);

/* The achievable-read probe: every byte of buf once, each workgroup streaming
 * contiguous 256 KB runs with non-temporal 128-bit loads (the fastest read
 * shape measured); sink as above.  bytes a multiple of 16. */
cap_status cap_bench_read_stream(const void *buf, size_t bytes, void *sink, cap_stream_t stream);

/* Plain copy of `bytes` from src to dst: reads and writes a known byte count,
 * for scaling FETCH_SIZE / WRITE_SIZE counters. */
cap_status cap_bench_copy(void *dst, const void *src, size_t bytes, cap_stream_t stream);

/* The achievable read-plus-write probe: copy `bytes` from src to dst, each
 * workgroup copying contiguous runs of `run_bytes` (0 = 256 KB; else a
 * multiple of 16: e.g. one row, for the shape of a one-row-per-workgroup
 * kernel) with non-temporal 128-bit loads and stores, eight loads in flight
 * per lane; up to 8192 workgroups, each looping over its runs.  src and dst
 * must not overlap. */
cap_status cap_bench_copy_stream(void *dst, const void *src, size_t bytes, size_t run_bytes,
                                 cap_stream_t stream);

/* cap_decode_attention (same arguments, same checks and errors), launched
 * with two HIP events bound to the kernel's own dispatch (hipExtLaunchKernel)
 * that the call creates and destroys; it waits for the kernel and writes its
 * execution time in microseconds to *us (from the start of the dispatch to
 * the end of its last workgroup, without the queueing and the end-of-kernel
 * cache flush that events recorded on the stream around a launch include:
 * what a profiler's kernel trace reports).  Blocks the calling thread;
 * CAP_ERR_HIP if an event call fails. */
cap_status cap_bench_decode_timed(const cap_plan *plan, const void *q, const void *k_pool,
                                  const void *v_pool, void *workspace, size_t ws_bytes,
                                  cap_stream_t stream, float *us);

#ifdef __cplusplus
}
#endif
#endif /* CAP_BENCH_H */
