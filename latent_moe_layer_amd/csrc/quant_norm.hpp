// 1x128 FP8 activation quantizer and the fused top-k combine + RMSNorm.
#pragma once

#include "common.hpp"

namespace moe_tail {

// Per 1x128 block: s = amax / 448 (IEEE division), 1.0 for an all-zero
// block; code = e4m3(x / s).  Activations are quantized per 1x128 block with
// fp32 scales, matching the 128-wide K blocks of the weights.  A row-major
// [rows, cols] matrix is a sequence of blocks (cols % 128 == 0), block i
// covering elements [128 i, 128 i + 128) and owning scale i.  Wave w takes
// blocks 4 w .. 4 w + 3: lanes 16 j .. 16 j + 15 block 4 w + j, eight
// neighbouring elements each (16-byte loads).
constexpr int kQuantBlocksPerWave = 4;

// Optional second copy of the scales for the routed GEMMs: block kb of
// token t also goes to out[kb * R + pair_to_row[t * k + j]] for every slot j,
// i.e. K-block-major over the sorted routed rows, so that the tiled kernels
// read a tile's row scales for one K block as one contiguous run (instead of
// one 4-byte load from each row's own line, once per weight tile).
struct RowScales {
  const int32_t* pair_to_row;  // [tokens * k], or null: no copy
  float* out;                  // [cols / 128, R]
  int k, nkb;                  // slots per token (<= 16), scale blocks per row
  long R;                      // routed rows (tokens * k)
};

template <bool kBf16In>
__device__ __forceinline__ void quant_wave(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                           float* __restrict__ scales, long nblocks, long w, int lane,
                                           const RowScales& rs) {
  const long blk = w * kQuantBlocksPerWave + (lane >> 4);
  if (w * kQuantBlocksPerWave >= nblocks) return;  // wave-uniform
  const bool live = blk < nblocks;                 // uniform within a block's 16 lanes
  const size_t e0 = static_cast<size_t>(live ? blk : 0) * 128 + 8 * (lane & 15);
  float v[8];
  if (kBf16In) {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e0);
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(u[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
    }
  } else {
    const float4 p0 = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + e0);
    const float4 p1 = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + e0 + 4);
    v[0] = p0.x; v[1] = p0.y; v[2] = p0.z; v[3] = p0.w;
    v[4] = p1.x; v[5] = p1.y; v[6] = p1.z; v[7] = p1.w;
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  const float amax = group16_max(m);
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3(v[i] / s) << (8 * i);
    hi |= f32_to_e4m3(v[4 + i] / s) << (8 * i);
  }
  if (live) {
    *reinterpret_cast<uint2*>(codes + e0) = make_uint2(lo, hi);
    if ((lane & 15) == 0) scales[blk] = s;
    if (rs.out != nullptr && (lane & 15) < rs.k) {  // lane j of the block: slot j's row
      const long t = blk / rs.nkb, kb = blk - t * rs.nkb;
      rs.out[kb * rs.R + rs.pair_to_row[t * rs.k + (lane & 15)]] = s;
    }
  }
}

template <bool kBf16In>
__global__ __launch_bounds__(256) void k_quant_1x128(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                     float* __restrict__ scales, long nblocks, RowScales rs) {
  quant_wave<kBf16In>(x, codes, scales, nblocks, static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6),
                      threadIdx.x & 63, rs);
}

// Workgroups of 256 threads for nblocks 1x128 blocks.
inline unsigned quant_grid(long nblocks) {
  const long per = 4L * kQuantBlocksPerWave;
  return static_cast<unsigned>((nblocks + per - 1) / per);
}

// The same quantizer of x, whose first workgroup also clears n words at
// `zero` (the completion counters of the single-launch tail that follows).
__global__ __launch_bounds__(256) void k_quant_clear(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                     float* __restrict__ scales, long nblocks,
                                                     int* __restrict__ zero, int n, RowScales rs) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n; i += 256) zero[i] = 0;
  quant_wave<true>(x, codes, scales, nblocks, static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6),
                   threadIdx.x & 63, rs);
}

// One workgroup (256 threads) per routed token: z = sum_j w_j * y[row(t, j)]
// in FP32 (slot order), then RMSNorm with FP32 statistics:
// rn = bf16((z / sqrt(mean(z^2) + eps)) * gamma).  The routed latent is
// normalised before the up-projection ("[Kimi K3][Kernel] Fuse BF16 shared
// experts into latent MegaMoE tail", Summary); FP32-internal statistics follow
// the bias study in tokenspeed PR 1062.
constexpr int kNormMaxCols = 32;  // L <= 256 * 32

// One workgroup per token; thread tid owns the 4-column groups tid + 256 c
// (NC4 = an upper bound of L / 1024: groups past L are clamped, loaded and
// unused).  The rows' 16-byte loads are issued in batches before any is
// used; each column still sums its k slots in slot order.
//
// combine_token: token t by the 256 threads tid = 0..255 of one half of a
// workgroup (s_part: 4 words of that half); t < 0 only takes part in the
// workgroup barrier.
template <int NC4>
__device__ __forceinline__ void combine_token(const float* __restrict__ y, const float* __restrict__ topk_w,
                                              const int32_t* __restrict__ pair_to_row,
                                              const uint16_t* __restrict__ gamma, uint16_t* __restrict__ rn, int L,
                                              int k, float eps, int t, int tid, float* s_part) {
  const bool live = t >= 0;
  if (!live) t = 0;
  const int ng = L / 4;  // 4-column groups
  int grp[NC4];
#pragma unroll
  for (int c = 0; c < NC4; ++c) grp[c] = min(tid + 256 * c, ng - 1);
  float4 z[NC4];
#pragma unroll
  for (int c = 0; c < NC4; ++c) z[c] = float4{0.f, 0.f, 0.f, 0.f};
  // rows in batches of kB (k <= 16): each batch's loads are issued before
  // any is used; rows past k are clamped to the last slot, loaded and unused
  constexpr int kB = (NC4 <= 4) ? 8 : 4;
  for (int j0 = 0; j0 < (live ? k : 0); j0 += kB) {
    float4 v[kB][NC4];
    float w[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int jj = min(j0 + j, k - 1);
      w[j] = topk_w[static_cast<size_t>(t) * k + jj];
      const float4* yr =
          reinterpret_cast<const float4*>(y + static_cast<size_t>(pair_to_row[static_cast<size_t>(t) * k + jj]) * L);
#pragma unroll
      for (int c = 0; c < NC4; ++c) v[j][c] = yr[grp[c]];
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      if (j0 + j < k) {
#pragma unroll
        for (int c = 0; c < NC4; ++c) {
          z[c].x = z[c].x + w[j] * v[j][c].x;
          z[c].y = z[c].y + w[j] * v[j][c].y;
          z[c].z = z[c].z + w[j] * v[j][c].z;
          z[c].w = z[c].w + w[j] * v[j][c].w;
        }
      }
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < NC4; ++c)
    if (tid + 256 * c < ng) ss += ((z[c].x * z[c].x + z[c].y * z[c].y) + z[c].z * z[c].z) + z[c].w * z[c].w;
  ss = wave_sum(ss);
  if ((tid & 63) == 0) s_part[tid >> 6] = ss;
  __syncthreads();
  const float tot = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
  const float r = 1.0f / sqrtf(tot / static_cast<float>(L) + eps);
#pragma unroll
  for (int c = 0; c < NC4; ++c) {
    const int gi = tid + 256 * c;
    if (live && gi < ng) {
      const uint2 gm = *reinterpret_cast<const uint2*>(gamma + 4 * gi);
      uint2 o;
      o.x = f32_to_bf16_bits((z[c].x * r) * bf16_bits_to_f32(gm.x & 0xffffu)) |
            (f32_to_bf16_bits((z[c].y * r) * bf16_bits_to_f32(gm.x >> 16)) << 16);
      o.y = f32_to_bf16_bits((z[c].z * r) * bf16_bits_to_f32(gm.y & 0xffffu)) |
            (f32_to_bf16_bits((z[c].w * r) * bf16_bits_to_f32(gm.y >> 16)) << 16);
      *reinterpret_cast<uint2*>(rn + static_cast<size_t>(t) * L + 4 * gi) = o;
    }
  }
}

template <int NC4>
__global__ __launch_bounds__(256) void k_combine_rmsnorm(const float* __restrict__ y, const float* __restrict__ topk_w,
                                                         const int32_t* __restrict__ pair_to_row,
                                                         const uint16_t* __restrict__ gamma,
                                                         uint16_t* __restrict__ rn, int L, int k, float eps) {
  __shared__ float s_part[4];
  combine_token<NC4>(y, topk_w, pair_to_row, gamma, rn, L, k, eps, blockIdx.x, threadIdx.x, s_part);
}

}  // namespace moe_tail
