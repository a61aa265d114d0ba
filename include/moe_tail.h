/*
 * moe_tail.h -- C ABI of the MI355X (gfx950) latent-MoE layer tail.
 *
 * The tail (pages: "[Kimi K3][Kernel] Fuse BF16 shared experts into latent
 * MegaMoE tail", Summary and "Sequence-parallel implementation"; DeepGEMM PR
 * 416 mirror, Summary and Implementation; tokenspeed PR 1062, Summary):
 *
 *   route:    logits = x_lat . W_g^T (+ bias); top-k; softmax over the k
 *             selected logits; tokens permuted into per-expert row segments
 *   forward:  x_lat -> e4m3 codes with one fp32 scale per 1x128 block;
 *             routed L1 gate/up (FP8 128x128 block-scaled or MXFP4 weights),
 *             SwiGLU, h -> e4m3 per 1x128, routed L2 down to the latent;
 *             top-k weighted combine in FP32 fused with RMSNorm -> bf16;
 *             shared BF16 SwiGLU MLP on x_hid (its own token count Ms >= Mr);
 *             out = bf16(up(RMSNorm(routed)) + f32(shared)) for t < Mr, with
 *             the up-projection accumulated in FP32 and one final rounding;
 *             shared rows t >= Mr go to shared_out.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major with the reduction
 *     (K) dimension contiguous, 16-byte aligned.  bf16 travels as uint16_t
 *     bit patterns.
 *   - The caller allocates and owns every buffer.  The library allocates no
 *     device memory, keeps no pointer after returning, never synchronizes,
 *     and enqueues all work on `stream` (a hipStream_t; NULL = null stream),
 *     or, in moe_tail_forward, partly on a second stream of its own that it
 *     forks from `stream` and joins back into it (see there): every result
 *     is ordered on `stream` either way.
 *   - Every argument check runs on the host before anything is enqueued.  On
 *     any error nothing has been enqueued ("fail closed").  A launch failure
 *     reported by the runtime returns MOE_TAIL_ERR_DEVICE.
 *   - The library keeps no state between calls beyond per-device caches
 *     (the CU count; per host thread, moe_tail_forward's second stream and
 *     its two events) and is re-entrant; concurrent calls need disjoint
 *     workspaces and outputs.
 *   - Behaviour is undefined for non-finite inputs and for a routing that
 *     moe_tail_route did not produce for the same x_lat / Mr.
 */
#ifndef MOE_TAIL_H
#define MOE_TAIL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_TAIL_OK = 0,
  MOE_TAIL_ERR_INVALID = 1,      /* null/misaligned pointer, bad count, bad dims */
  MOE_TAIL_ERR_UNSUPPORTED = 2,  /* dims or format outside what the kernels implement */
  MOE_TAIL_ERR_WORKSPACE = 3,    /* ws_bytes smaller than moe_tail_workspace_bytes() */
  MOE_TAIL_ERR_DEVICE = 4        /* the HIP runtime rejected a launch */
} moe_tail_status;

typedef enum {
  MOE_TAIL_W_FP8_BLOCK128 = 0,   /* e4m3 codes + fp32 scale per 128 (N) x 128 (K) block */
  MOE_TAIL_W_MXFP4 = 1,          /* e2m1 pairs (even K in the low nibble) + e8m0 scale per 32 along K */
  MOE_TAIL_W_MXFP4_PACKED = 2,   /* MXFP4 with the e8m0 scales in the tile order of moe_tail_pack_mxfp4_scales */
  MOE_TAIL_W_NVFP4 = 3,          /* e2m1 pairs + e4m3 scale per 16 along K + fp32 scale per expert matrix */
  MOE_TAIL_W_NVFP4_PACKED = 4    /* NVFP4 with the e4m3 scales in the tile order of moe_tail_pack_nvfp4_scales */
} moe_tail_wfmt;

/* Sizes of one tail.  hidden (H) and latent (L) are the shared and routed
 * widths (7168 and 3584 in the served model), inter (I) and shared_inter
 * (I_s) the routed and shared intermediate sizes.
 * Valid: all sizes > 0, 1 <= top_k <= num_experts, finite rms_eps > 0.
 * Supported by the kernels: H and L multiples of 256 with L <= 8192; I and
 * I_s multiples of 128 with I <= 8192; num_experts <= 1024; top_k <= 16. */
typedef struct {
  int32_t hidden;
  int32_t latent;
  int32_t num_experts;
  int32_t top_k;
  int32_t inter;
  int32_t shared_inter;
  int32_t wfmt;          /* moe_tail_wfmt */
  float rms_eps;
} moe_tail_dims;

/* Weights (device, read-only).  Row r of w1 for r < I is the gate projection,
 * r >= I the up projection; the same split holds for ws1 with I_s.
 * NVFP4 (MOE_TAIL_W_NVFP4): the routed weights as served with NVFP4
 * quantization (tokenspeed recipe "Kimi-K3 DEP16 with sharded shared
 * experts", Allocation and launch): W = e2m1 * e4m3 block scale (one per 16
 * weights along K) * the expert matrix's fp32 scale.  The gfx950 scaled
 * matrix cores take e8m0 scales per 32 only, so these weights run on the
 * FP16 matrix cores, dequantized exactly in registers. */
typedef struct {
  const float *gate;          /* [E, L] fp32 router weights */
  const float *gate_bias;     /* [E] fp32 router bias, or NULL for none */
  const uint8_t *w1;          /* FP8: [E, 2I, L] e4m3      | MXFP4, NVFP4: [E, 2I, L/2] packed e2m1 */
  const void *w1_scale;       /* FP8: [E, 2I/128, L/128] f32 | MXFP4: [E, 2I, L/32] e8m0 | NVFP4: [E, 2I, L/16] e4m3 */
  const uint8_t *w2;          /* FP8: [E, L, I] e4m3       | MXFP4, NVFP4: [E, L, I/2] packed e2m1 */
  const void *w2_scale;       /* FP8: [E, L/128, I/128] f32  | MXFP4: [E, L, I/32] e8m0 | NVFP4: [E, L, I/16] e4m3 */
  const uint16_t *rms_gamma;  /* [L] bf16 */
  const uint16_t *w_up;       /* [H, L] bf16 up-projection */
  const uint16_t *ws1;        /* [2 I_s, H] bf16 shared gate/up */
  const uint16_t *ws2;        /* [H, I_s] bf16 shared down */
  const float *w1_tensor_scale;  /* NVFP4: [E] fp32 scale of each expert's w1; ignored by the other formats */
  const float *w2_tensor_scale;  /* NVFP4: [E] fp32 scale of each expert's w2; ignored by the other formats */
} moe_tail_weights;

/* Routing produced by moe_tail_route (device buffers owned by the caller). */
typedef struct {
  int32_t *topk_ids;        /* [Mr, k]: experts by (logit desc, index asc) */
  float *topk_weights;      /* [Mr, k]: softmax over the k selected logits */
  int32_t *expert_offsets;  /* [E + 1]: exclusive prefix of per-expert row counts */
  int32_t *sorted_pair;     /* [Mr * k]: row -> pair t*k + j, tokens ascending within an expert */
  int32_t *pair_to_row;     /* [Mr * k]: pair t*k + j -> row (inverse of sorted_pair) */
} moe_tail_routing;

/* Bytes of device workspace that moe_tail_route and moe_tail_forward need
 * for these sizes (one workspace serves both calls).  Returns 0 when the
 * dims or counts are invalid or unsupported. */
size_t moe_tail_workspace_bytes(const moe_tail_dims *dims, int32_t Mr, int32_t Ms);

/* Indices into moe_tail_workspace_layout's offsets[]: the intermediates the
 * forward pass materializes, exposed so tests can read them. */
enum {
  MOE_TAIL_WS_XQ = 0,   /* [Mr, L] u8 e4m3 codes of x_lat */
  MOE_TAIL_WS_SX = 1,   /* [Mr, L/128] f32 scales of x_lat */
  MOE_TAIL_WS_HQ = 2,   /* [Mr*k, I] u8 e4m3 codes of h, rows in sorted order */
  MOE_TAIL_WS_SH = 3,   /* [I/128, Mr*k] f32 scales of h, K-block-major: block b of sorted row r at b*Mr*k + r */
  MOE_TAIL_WS_Y = 4,    /* [Mr*k, L] f32 routed L2 output, rows in sorted order */
  MOE_TAIL_WS_RN = 5,   /* [Mr, L] bf16 normalized combined latent */
  MOE_TAIL_WS_HS = 6,   /* [Ms, I_s] bf16 shared intermediate */
  MOE_TAIL_WS_S = 7,    /* [Mr, H] bf16 shared output rows 0..Mr-1 */
  MOE_TAIL_WS_STATUS = 8, /* int32 status of the last moe_tail_forward_fused call on this workspace:
                             0 = complete, 1 = a stage wait gave up and out / shared_out hold NaN;
                             SIZE_MAX where these sizes have no single-launch path */
  MOE_TAIL_WS_NUM = 9
};

/* Byte offsets of the intermediates above inside the workspace (SIZE_MAX
 * for one these sizes do not have).
 * Returns MOE_TAIL_OK or MOE_TAIL_ERR_INVALID / _UNSUPPORTED. */
int moe_tail_workspace_layout(const moe_tail_dims *dims, int32_t Mr, int32_t Ms, size_t offsets[MOE_TAIL_WS_NUM]);

/* Routing of Mr tokens (0 <= Mr <= 2^20).  Reads x_lat [Mr, L] bf16 and
 * weights->gate / gate_bias; writes every array of *out.
 * Logits use a fixed FP32 summation order (64 strided partial sums, each a
 * sequential fused multiply-add chain, combined by an xor butterfly over
 * 32,16,8,4,2,1), so expert ids are reproducible bit for bit.  Ties between
 * equal logits go to the lower expert index. */
int moe_tail_route(const moe_tail_dims *dims, const moe_tail_weights *weights, const uint16_t *x_lat, int32_t Mr,
                   const moe_tail_routing *out, void *workspace, size_t ws_bytes, void *stream);

/* The tail for Mr routed tokens and Ms >= Mr shared tokens (0 <= Mr <= Ms <= 2^20).
 * Routed token t is shared token t (t < Mr).
 *   x_lat  [Mr, L] bf16 routed latent input
 *   x_hid  [Ms, H] bf16 shared-expert input
 *   routing  from moe_tail_route for this x_lat (read only)
 *   out        [Mr, H] bf16: bf16(up(RMSNorm(routed)) + f32(shared)) for t < Mr
 *   shared_out [Ms-Mr, H] bf16: shared rows t >= Mr at row t-Mr; NULL iff Ms == Mr
 * With FP8 routed weights, the experts averaging at most 64 routed rows
 * (Mr * top_k <= 64 * E, Mr * top_k > 32 * E) and Ms >= 2 * Mr (Ms > 128), the
 * shared expert's L1 and L2 run on a second stream of the library's own (one
 * per host thread and device, created on first use at the default priority)
 * beside the routed GEMMs, each on a share of the CUs: an event recorded on
 * `stream` at the start forks it, an event recorded on it joins it back into
 * `stream` before the up-projection.  The outputs are ordered on `stream` as
 * usual, are the same bits as on one stream, and capturing `stream` into a
 * graph captures both. */
int moe_tail_forward(const moe_tail_dims *dims, const moe_tail_weights *weights, const uint16_t *x_lat, int32_t Mr,
                     const uint16_t *x_hid, int32_t Ms, const moe_tail_routing *routing, uint16_t *out,
                     uint16_t *shared_out, void *workspace, size_t ws_bytes, void *stream);

/* moe_tail_forward with the residual stream joined in the same epilogue
 * ("add3"): out[t, n] = bf16((up(RMSNorm(routed))[t, n] + f32(shared[t, n]))
 * + f32(residual[t, n])) for t < Mr, the three terms added in FP32 in that
 * order and rounded to bf16 once.  The pages' finalize tail joins
 * projection, shared partial and residual in one step and finds that
 * storing bf16 before the residual add rounds twice and biases the output
 * (tokenspeed PR "MNNVL CuTe-DSL finalize tail + K3 comm layer extraction",
 * commit log).
 *   residual [Mr, H] bf16, read only; may be NULL only when Mr == 0.
 * Every other argument, the workspace and the errors are those of
 * moe_tail_forward; shared_out rows get no residual. */
int moe_tail_forward_add3(const moe_tail_dims *dims, const moe_tail_weights *weights, const uint16_t *x_lat,
                          int32_t Mr, const uint16_t *x_hid, int32_t Ms, const moe_tail_routing *routing,
                          const uint16_t *residual, uint16_t *out, uint16_t *shared_out, void *workspace,
                          size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture that must not call the allocator, tight serving loops, harnesses
 * that forbid it): moe_tail_forward without a workspace argument.  The
 * library keeps one workspace of MOE_TAIL_NOALLOC_MAX_BYTES in device memory
 * for the whole process (a static device array, one per GPU it runs on) and
 * the call uses that; it allocates nothing and frees nothing.
 *   Sizes whose moe_tail_workspace_bytes exceeds MOE_TAIL_NOALLOC_MAX_BYTES
 *   return MOE_TAIL_ERR_WORKSPACE with nothing enqueued (48 MiB covers the
 *   decode sizes: 128 routed and 128 shared tokens with 64..1024 experts,
 *   top-8, I = I_s = 2048 at the served widths take about 35 MiB).
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents: calls that overlap on one GPU (other streams, other
 *   threads) race and must be serialized by the caller.  Whatever must start
 *   at zero is cleared by the call's own kernels.
 *   It enqueues everything on `stream` (never moe_tail_forward's second
 *   stream, which it would have to create).
 *   Results are bit for bit those of moe_tail_forward; every other argument
 *   and error is moe_tail_forward's.  MOE_TAIL_ERR_DEVICE also reports that
 *   the runtime could not give this device's copy of the array. */
#define MOE_TAIL_NOALLOC_MAX_BYTES ((size_t)48 << 20)
int moe_tail_forward_noalloc(const moe_tail_dims *dims, const moe_tail_weights *weights, const uint16_t *x_lat,
                             int32_t Mr, const uint16_t *x_hid, int32_t Ms, const moe_tail_routing *routing,
                             uint16_t *out, uint16_t *shared_out, void *stream);

/* moe_tail_forward (residual NULL) or moe_tail_forward_add3 (residual
 * non-NULL) as two launches: the x quantizer, then ONE persistent launch
 * that runs the routed experts, the shared expert, combine + RMSNorm and the
 * up-projection as a fixed sequence of stages, one workgroup per CU, the
 * stages joined by completion counters in the workspace instead of kernel
 * boundaries.  The pages' producer schedules routed and shared work together
 * in one kernel (DeepGEMM PR 416 mirror, Summary); here the tail's
 * up-projection and final join run in the same launch as well.
 *   Sizes: decode-sized token counts, Ms <= 128 (hence Mr <= 128), with
 *   num_experts <= 512, L >= 384 and I >= 384; Mr = 0 runs the shared expert
 *   alone exactly as moe_tail_forward does.  Other sizes return
 *   MOE_TAIL_ERR_UNSUPPORTED with nothing enqueued (use moe_tail_forward).
 *   Results: bit for bit those of moe_tail_forward / _add3 (the same tiles
 *   and summation orders).  Workspace: moe_tail_workspace_bytes.
 *   The persistent launch needs all of its workgroups resident together (its
 *   stages wait on each other): do not run it concurrently with other work
 *   that occupies CUs for long, including another call of this entry point
 *   on another stream.
 *   Fail closed: a stage that waits for more than about a second gives up
 *   (the launch always finishes); the launch then writes NaN over every
 *   element of out and shared_out and sets the workspace's status word
 *   (moe_tail_workspace_layout, MOE_TAIL_WS_STATUS) to 1.  The word is 0
 *   after a complete launch; read it after the stream has passed the call. */
int moe_tail_forward_fused(const moe_tail_dims *dims, const moe_tail_weights *weights, const uint16_t *x_lat,
                           int32_t Mr, const uint16_t *x_hid, int32_t Ms, const moe_tail_routing *routing,
                           const uint16_t *residual, uint16_t *out, uint16_t *shared_out, void *workspace,
                           size_t ws_bytes, void *stream);

/* moe_tail_forward_fused with each stage wait polling its counter at most
 * max_polls times (about 0.1 us apart) before it gives up, for callers that
 * want a shorter bound and for tests of the failure path: max_polls = 0
 * gives up every wait at once, which always ends in the NaN outputs and
 * status 1 described above.  max_polls < 0 is MOE_TAIL_ERR_INVALID. */
int moe_tail_forward_fused_bounded(const moe_tail_dims *dims, const moe_tail_weights *weights, const uint16_t *x_lat,
                                   int32_t Mr, const uint16_t *x_hid, int32_t Ms, const moe_tail_routing *routing,
                                   const uint16_t *residual, uint16_t *out, uint16_t *shared_out, void *workspace,
                                   size_t ws_bytes, void *stream, int32_t max_polls);

/* Number of stages moe_tail_forward_profiled brackets with events. */
#define MOE_TAIL_NUM_STAGES 7
/* Stage order: 0 quantize x_lat, 1 routed L1 (+SwiGLU + h quantization),
 * 2 routed L2, 3 combine + RMSNorm, 4 shared L1 (+SwiGLU), 5 shared L2,
 * 6 up-projection + shared add.  A stage with no work records its events
 * back to back. */

/* moe_tail_forward that also records stage_events[i] (hipEvent_t) on `stream`
 * right before stage i and stage_events[MOE_TAIL_NUM_STAGES] after the last
 * one.  stage_events must hold MOE_TAIL_NUM_STAGES + 1 created events. */
int moe_tail_forward_profiled(const moe_tail_dims *dims, const moe_tail_weights *weights, const uint16_t *x_lat,
                              int32_t Mr, const uint16_t *x_hid, int32_t Ms, const moe_tail_routing *routing,
                              uint16_t *out, uint16_t *shared_out, void *workspace, size_t ws_bytes, void *stream,
                              void *const *stage_events);

/* moe_tail_forward (residual NULL) or moe_tail_forward_add3 (residual
 * non-NULL), the same launches in the same order, with events[i]
 * (hipEvent_t) recorded on `stream` right before launch group i of that
 * schedule and the events after the last group recorded back to back after
 * it.  events must hold MOE_TAIL_NUM_STAGES + 1 created events.  The groups
 * are named by moe_tail_stage_name; for measuring each group of the schedule
 * the plain call runs (every other argument as moe_tail_forward). */
int moe_tail_forward_timed(const moe_tail_dims *dims, const moe_tail_weights *weights, const uint16_t *x_lat,
                           int32_t Mr, const uint16_t *x_hid, int32_t Ms, const moe_tail_routing *routing,
                           const uint16_t *residual, uint16_t *out, uint16_t *shared_out, void *workspace,
                           size_t ws_bytes, void *stream, void *const *events);

/* Static name of launch group i of the schedule moe_tail_forward runs for
 * these sizes (decode sizes: "quant_x", "routed_l1", "routed_l2+shared_l1",
 * "combine_rmsnorm+shared_l1_reduce", "shared_l2+up_proj", "final_join";
 * otherwise the MOE_TAIL_NUM_STAGES stages of moe_tail_forward_profiled), or
 * NULL past the last group or for invalid arguments. */
const char *moe_tail_stage_name(const moe_tail_dims *dims, int32_t Mr, int32_t Ms, int32_t i);

/* The device 1x128 FP8 quantizer the forward pass uses, exported for tests:
 * per row and 128-wide block, s = amax / 448 (1.0 for an all-zero block),
 * code = e4m3(x / s) rounded to nearest even, saturating at +-448, sign of
 * zero kept.  x is [rows, cols] bf16 (x_is_bf16 = 1) or fp32; cols % 128 == 0.
 * codes [rows, cols] u8, scales [rows, cols/128] f32. */
int moe_tail_quant_fp8_1x128(const void *x, int32_t x_is_bf16, int32_t rows, int32_t cols, uint8_t *codes,
                             float *scales, void *stream);

/* MXFP4 weight scales rearranged for the tiled kernels (same values, same
 * byte count per matrix), to be done once when the weights are loaded.  The
 * pages' routed FP8/FP4 experts (DeepGEMM PR 416 mirror, Summary) fix the
 * format (an e8m0 scale per 32 weights along K), not the order of the scales
 * in memory; this order is the library's: the scales of one tile's 256
 * weight rows for one 256-wide K step are one contiguous 2 KB run, which the
 * tiled kernels load with whole lines instead of two 4-byte loads per row
 * and step.
 *   For each expert e and each weight matrix W [N, K] with natural scales
 *   S[n][K/32] (w1: N = 2I, K = L; w2: N = L, K = I), the packed scales are
 *   P[e][t][s][h][j][g] = S[e][n(t, j)][8 s + 4 h + g] with t < N/256 (tile),
 *   s < K/256 (K step), h < 2 (128-wide K block), j < 256 (tile row), g < 4
 *   (32-wide group); tile row j of w1 is gate row 128 t + j for j < 128 and up
 *   row I + 128 t + (j - 128) otherwise, of w2 row 256 t + j.
 * dims->wfmt is MOE_TAIL_W_MXFP4 or _PACKED; L and I must be multiples of
 * 256 (else MOE_TAIL_ERR_UNSUPPORTED).  w1_scale / w2_scale are the natural
 * [E, 2I, L/32] / [E, L, I/32] e8m0 arrays, the packed outputs the same
 * sizes (device, caller-owned, not overlapping the inputs).  Either pair may
 * be NULL to skip that matrix.  A forward with dims->wfmt =
 * MOE_TAIL_W_MXFP4_PACKED takes the packed arrays in weights->w1_scale /
 * w2_scale and gives bit for bit the results of MOE_TAIL_W_MXFP4 with the
 * natural ones; it needs the shapes the tiled kernels cover (L and I
 * multiples of 256, at least 512, num_experts <= 512), else it returns
 * MOE_TAIL_ERR_UNSUPPORTED. */
int moe_tail_pack_mxfp4_scales(const moe_tail_dims *dims, const uint8_t *w1_scale, const uint8_t *w2_scale,
                               uint8_t *w1_scale_packed, uint8_t *w2_scale_packed, void *stream);

/* NVFP4 weight scales rearranged for the tiled kernels (same values, same
 * byte count per matrix), to be done once when the weights are loaded.  The
 * NVFP4 recipe the pages serve (tokenspeed recipe "Kimi-K3 DEP16 with
 * sharded shared experts", Allocation and launch) fixes the format (an e4m3
 * scale per 16 weights along K), not the order of the scales in memory; in
 * this order the scales of one tile's 256 weight rows for one 256-wide K
 * step are one contiguous 4 KB run (whole-line loads instead of 16 bytes
 * from each of 256 rows).
 *   For each expert e and each weight matrix W [N, K] with natural scales
 *   S[n][K/16] (w1: N = 2I, K = L; w2: N = L, K = I), the packed scales are
 *   P[e][t][s][j][q] = S[e][n(t, j)][16 s + q] with t < N/256 (tile),
 *   s < K/256 (K step), j < 256 (tile row), q < 16; tile row j of w1 is gate
 *   row 128 t + j for j < 128 and up row I + 128 t + (j - 128) otherwise, of
 *   w2 row 256 t + j.
 * dims->wfmt is MOE_TAIL_W_NVFP4 or _PACKED; L and I must be multiples of
 * 256 (else MOE_TAIL_ERR_UNSUPPORTED).  w1_scale / w2_scale are the natural
 * [E, 2I, L/16] / [E, L, I/16] e4m3 arrays, the packed outputs the same sizes
 * (device, caller-owned, not overlapping the inputs).  Either pair may be
 * NULL to skip that matrix.  A forward with dims->wfmt =
 * MOE_TAIL_W_NVFP4_PACKED takes the packed arrays in weights->w1_scale /
 * w2_scale (and the matrix scales as for MOE_TAIL_W_NVFP4) and gives bit for
 * bit the results of MOE_TAIL_W_NVFP4 with the natural ones; it needs the
 * shapes the tiled kernels cover (L and I multiples of 256, at least 512,
 * num_experts <= 512), else it returns MOE_TAIL_ERR_UNSUPPORTED. */
int moe_tail_pack_nvfp4_scales(const moe_tail_dims *dims, const uint8_t *w1_scale, const uint8_t *w2_scale,
                               uint8_t *w1_scale_packed, uint8_t *w2_scale_packed, void *stream);

/* Static description of a status code. */
const char *moe_tail_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_TAIL_H */
