/*
 * attn_clock.h -- shader-clock probe used by the benchmark to record the GPU
 * clock before and after a timed region (a clock that drops under load
 * changes what a timing means).  Not part of the attention path.
 *
 * attn_clock_probe -- enqueue n_wg workgroups of one wave each on `stream`
 * (a hipStream_t, NULL = null stream).  Each wave reads the shader cycle
 * counter (s_memtime) and the constant 100 MHz reference counter
 * (s_memrealtime), runs `iters` rounds of a dependent chain of vector
 * multiply-adds, reads both counters again, and writes the two deltas to
 * out[2*w] (cycles) and out[2*w + 1] (reference ticks).  The shader clock in
 * MHz is then 100 * cycles / ticks.
 *   out   : DEVICE pointer to 2*n_wg uint64 values, 8-byte aligned, owned by
 *           the caller.
 *   n_wg  : 1 .. 4096;  iters : 1 .. 1<<24.
 * Returns 0 once enqueued; 1 for a NULL or misaligned `out`, 2 for n_wg or
 * iters out of range, 10 if the launch reported an error.  Nothing is
 * allocated; the caller synchronises before reading `out`.
 */
#ifndef ATTN_CLOCK_H
#define ATTN_CLOCK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int attn_clock_probe(uint64_t *out, int n_wg, int iters, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CLOCK_H */
