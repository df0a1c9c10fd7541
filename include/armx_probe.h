/*
 * armx_probe.h -- measurement only: a plain HBM read stream, the ceiling the
 * reductions of armx.h are compared with.  Built as libarmx_probe.so, apart
 * from libarmx.so; no reduction calls it.
 *
 * All pointers are device pointers; the call is asynchronous on `stream` (a
 * hipStream_t, NULL = the null stream).  Returns 0, or -1 for a NULL
 * pointer, -2 for a misaligned one, -3 for an invalid launch shape, -5 when
 * n is not a multiple of 512 * loads or out is too small, -6 for a HIP error.
 */
#ifndef ARMX_PROBE_H
#define ARMX_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * armx_probe_read -- reads x[0..n) (binary16 values, 16-byte aligned) once
 * with 16-byte loads and writes one 32-bit XOR of the loaded words per lane
 * to out (blocks * block_threads words, so the loads cannot be dropped).
 *
 * A grid of `blocks` blocks of `block_threads` threads (a multiple of 64, at
 * most 1024); wavefront g of T takes steps g, g + T, ..., each step `loads`
 * consecutive 1 KiB wavefront loads (1, 2, 4, 8 or 16) issued back to back
 * and then consumed.  nontemporal != 0 uses non-temporal loads.  pause (0,
 * 2, 4 or 8) makes each wavefront sleep about 64 * pause clocks after every
 * step.
 * start_event / stop_event (hipEvent_t, may be NULL) are stamped by the
 * kernel's dispatch when it starts and completes.
 */
int armx_probe_read(const void* x, size_t n, uint32_t* out, size_t out_words, int blocks,
                    int block_threads, int loads, int nontemporal, int pause,
                    void* start_event, void* stop_event, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ARMX_PROBE_H */
