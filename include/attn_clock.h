/*
 * attn_clock.h -- probes used by the benchmark, not part of the attention
 * path: the shader clock before and after a timed region (a clock that drops
 * under load changes what a timing means), and the MFMA throughput a pure
 * matrix loop sustains (the measured ceiling next to the datasheet peak).
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

/*
 * attn_mfma_probe -- the matrix throughput the chip sustains: enqueue n_wg
 * workgroups of four waves on `stream`; each wave runs `iters` rounds of 16
 * MFMAs in four independent accumulator chains and nothing else
 * (v_mfma_f32_32x32x2_f32 for dtype 0, 4096 FLOP each; 32x32x16 f16 for
 * dtype 1 and bf16 for dtype 2, 32768 FLOP each), so one launch executes
 * n_wg * 4 * iters * 16 MFMAs.  Time it with events on the same stream.
 *   out   : DEVICE pointer to 4*n_wg floats (one sum per wave, which keeps
 *           the chains live; the values mean nothing), 4-byte aligned, owned
 *           by the caller.
 *   n_wg  : 1 .. 65536;  iters : 1 .. 1<<24;  dtype : 0, 1 or 2 (the
 *           ATTN_F32 / ATTN_F16 / ATTN_BF16 codes of attn.h).
 * Returns 0 once enqueued; 1 for a NULL or misaligned `out`, 2 for an
 * argument out of range, 10 if the launch reported an error.  Nothing is
 * allocated.
 */
int attn_mfma_probe(float *out, int n_wg, int iters, int dtype, void *stream);

/*
 * attn_copy_probe -- the HBM rate a plain stream reaches: enqueue a copy of
 * `bytes` bytes from src to dst on `stream` (n_wg workgroups of 256 lanes,
 * each lane moving 16 bytes per access with four accesses in flight).  Time
 * it with events on the same stream; it reads and writes `bytes` each.
 *   src, dst : DEVICE pointers, 16-byte aligned, not overlapping, owned by
 *              the caller;  bytes : a multiple of 16, at least 16;
 *   n_wg     : 1 .. 65536.
 * Returns 0 once enqueued; 1 for a NULL or misaligned pointer, 2 for a size
 * out of range or overlapping ranges, 10 if the launch reported an error.
 * Nothing is allocated.
 */
int attn_copy_probe(const void *src, void *dst, int64_t bytes, int n_wg, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CLOCK_H */
