// 1x128 FP8 activation quantizer and the fused top-k combine + RMSNorm.
#pragma once

#include "common.hpp"

namespace moe_tail {

// One wave per (row, 128-wide block); each lane owns two neighbouring
// elements.  s = amax / 448 (IEEE division), 1.0 for an all-zero block;
// code = e4m3(x / s).  Activations are quantized per 1x128 block with fp32
// scales, matching the 128-wide K blocks of the weights.
template <bool kBf16In>
__device__ __forceinline__ void quant_block(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                            float* __restrict__ scales, int rows, int cols, long blk, int lane) {
  const int nb = cols / 128;
  if (blk >= static_cast<long>(rows) * nb) return;
  const long r = blk / nb;
  const int b = static_cast<int>(blk % nb);
  const size_t base = static_cast<size_t>(r) * cols + 128 * b + 2 * lane;
  float v0, v1;
  if (kBf16In) {
    const uint32_t pair = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(x) + base);
    v0 = bf16_bits_to_f32(pair & 0xffffu);
    v1 = bf16_bits_to_f32(pair >> 16);
  } else {
    const float2 p = *reinterpret_cast<const float2*>(static_cast<const float*>(x) + base);
    v0 = p.x;
    v1 = p.y;
  }
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  const uint32_t q = f32_to_e4m3(v0 / s) | (f32_to_e4m3(v1 / s) << 8);
  *reinterpret_cast<uint16_t*>(codes + base) = static_cast<uint16_t>(q);
  if (lane == 0) scales[static_cast<size_t>(r) * nb + b] = s;
}

template <bool kBf16In>
__global__ __launch_bounds__(256) void k_quant_1x128(const void* __restrict__ x, uint8_t* __restrict__ codes,
                                                     float* __restrict__ scales, int rows, int cols) {
  quant_block<kBf16In>(x, codes, scales, rows, cols, static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6),
                       threadIdx.x & 63);
}

// The same quantizer of x, whose first workgroup also clears n words at
// `zero` (the completion counters of the single-launch tail that follows).
__global__ __launch_bounds__(256) void k_quant_clear(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                                     float* __restrict__ scales, int rows, int cols,
                                                     int* __restrict__ zero, int n) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < n; i += 256) zero[i] = 0;
  quant_block<true>(x, codes, scales, rows, cols, static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6),
                    threadIdx.x & 63);
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
