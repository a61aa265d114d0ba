/*
 * moe_tail_probes.h -- C ABI of the measurement probes that sit beside the
 * latent-MoE tail library (libmoe_tail_probes.so).
 *
 * These are not steps of the tail.  They are small kernels the tests and the
 * benchmark use to pin what the tail's kernels rely on:
 *   - the FP8 block product of the routed GEMMs (the same gfx950 scaled MFMA,
 *     v_mfma_scale_f32_16x16x128_f8f6f4 with unit e8m0 scales), so that tests
 *     can measure how it rounds sums of products;
 *   - a plain copy of known size, which calibrates the HBM byte counters
 *     (FETCH_SIZE, WRITE_SIZE) that the traffic figures are scaled by;
 *   - a streaming read, the practical HBM read ceiling that the bandwidth-bound
 *     kernels are compared with.
 *
 * Conventions: device pointers, 16-byte aligned; work is enqueued on `stream`
 * (a hipStream_t; NULL = null stream); nothing is allocated or synchronized.
 * Every argument check runs on the host before anything is enqueued; the
 * return value is 0 (ok), 1 (invalid argument) or 4 (the runtime rejected the
 * launch).
 */
#ifndef MOE_TAIL_PROBES_H
#define MOE_TAIL_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* n independent 16 x 16 x 128 FP8 block products, one wave each:
 *   c[i][m][j] = sum over k < 128 of e4m3(a[i][m][k]) * e4m3(b[i][j][k])
 * as one matrix-core instruction computes it (unit scales, FP32 result, no
 * accumulator input).  a, b: [n, 16, 128] e4m3 codes; c: [n, 16, 16] f32.
 * 1 <= n <= 65536. */
int moe_tail_probe_mfma_fp8(const uint8_t *a, const uint8_t *b, float *c, int32_t n, void *stream);

/* dst[0 .. bytes) = src[0 .. bytes) by 16-byte loads and stores, every byte
 * read once and written once.  bytes % 16 == 0; the ranges must not overlap. */
int moe_tail_probe_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Reads src[0 .. bytes) once with 16-byte loads spread over the whole chip
 * and writes to sink[0] only if the xor of everything read equals `magic`
 * (a data dependence that keeps the loads; sink is otherwise untouched).
 * bytes % 4096 == 0. */
int moe_tail_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, uint32_t magic, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TAIL_PROBES_H */
