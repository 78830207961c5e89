/* kvattn_probe.h -- measurement helper shipped beside libkvattn
 * (libkvattn_probe.so): the HBM read ceiling of one GPU for a given read
 * size, measured with a plain streaming-read kernel.  It is not part of the
 * attention path; the benchmark uses it to put the attention kernels'
 * quantised-KV bandwidth next to what a plain read of the same bytes per
 * launch reaches on the same device (the published 8 TB/s peak stays the
 * roofline).
 */
#ifndef KVATTN_PROBE_H
#define KVATTN_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of grid sizes and load policies kvattn_probe_read_ceiling times. */
#define KVATTN_PROBE_GRIDS 4    /* 256, 512, 1024, 2048 workgroups of 512 threads */
#define KVATTN_PROBE_POLICIES 2 /* 0: default loads, 1: non-temporal loads */

/* Plain-read ceiling on the current device.
 *   bytes      read size of one launch (a multiple of 16, at least 16)
 *   n_buffers  distinct device buffers of `bytes` each (1..4096), read one
 *              launch per buffer in turn, so that a pass over them does not
 *              fit the device caches when n_buffers * bytes is large
 *   reps       timed passes (1..100); the median pass is reported
 *   out_us     receives KVATTN_PROBE_POLICIES * KVATTN_PROBE_GRIDS values:
 *              microseconds per launch of policy p and grid g at
 *              out_us[p * KVATTN_PROBE_GRIDS + g] (host memory, caller-owned)
 *   best_gbps  receives the highest bytes / time over all of them, GB/s
 * Each launch reads its buffer completely: workgroup b of the grid reads one
 * contiguous slice of bytes / grid, 16-byte loads, eight in flight per
 * thread, folded into a value that is stored only when it equals a constant
 * (so the loads cannot be dropped).  One untimed pass per configuration
 * precedes the timed ones; timing uses HIP events on a stream of its own.
 * Everything allocated is freed before return.
 * Returns 0; -1 for invalid arguments; -2 when the device memory cannot be
 * allocated; -3 for any other HIP error (nothing is left allocated). */
int kvattn_probe_read_ceiling(uint64_t bytes, uint32_t n_buffers, uint32_t reps, double *out_us, double *best_gbps);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_PROBE_H */
