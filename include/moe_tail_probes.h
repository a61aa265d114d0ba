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
 *     kernels are compared with;
 *   - the per-workgroup rates of the load paths (direct-to-LDS rings, loads
 *     into registers) from HBM and from L2, which bound what a tile's staging
 *     can move.
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

/* Streaming rate of one load path, nothing computed: `grid` workgroups of 512
 * threads each read per_wg bytes, workgroup b the run src + b * per_wg (or,
 * with `shared`, all of them the run at src).  sink[0] = magic is written
 * only if, for some thread t, what it read equals `magic`: in modes 0 and 1
 * the 4-byte word t of the last stage in LDS, in modes 2 and 3 the xor of
 * every 4-byte word it loaded (a data dependence that keeps the loads and lets
 * a test check what arrived); sink is otherwise untouched.  mode:
 *   0  direct global -> LDS loads into a ring of 4 stages of 32 KB (3 in
 *      flight), each wave-wide load 1 KB of consecutive bytes;
 *   1  the same ring, each stage 128 bytes of each of 256 consecutive rows of
 *      row_bytes bytes (the routed GEMMs' weight-tile pattern: per load 8 rows
 *      x 128 bytes), the rows of one 256-row matrix after another;
 *   2  loads into registers, 16 in flight per lane, each wave-wide load 1 KB
 *      of consecutive bytes;
 *   3  the same, each wave-wide load 16 rows x 64 bytes (half cache lines).
 * per_wg: a multiple of 32 KB below 2 GiB (mode 1: also of 256 * row_bytes,
 * row_bytes a positive multiple of 128); 1 <= grid <= 65535; src holds
 * (shared ? 1 : grid) * per_wg bytes. */
int moe_tail_probe_stream_paths(const void *src, size_t per_wg, int32_t grid, int32_t shared, int32_t mode,
                                int32_t row_bytes, uint32_t *sink, uint32_t magic, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TAIL_PROBES_H */
