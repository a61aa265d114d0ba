// Router: logits, top-k + softmax, and the counting-sort permutation of
// (token, slot) pairs into per-expert row segments.
//
// The combine weights are a softmax over the k selected logits and the
// finalize step is a top-k weighted expert combine (tokenspeed PR 1062,
// Summary).  The routed rows of one expert are ordered by token so that the
// permutation is unique and reproducible ("routed dispatch", DeepGEMM PR 416
// mirror, Implementation).
#pragma once

#include "common.hpp"

namespace moe_tail {

// ---------------------------------------------------------------- logits --
// One workgroup = 4 waves; tile of kLogitTok tokens x (4 * kLogitExpPerWave)
// experts.  Lane l of a wave accumulates p[l] = fma-chain over i of
// x[64 i + l] * W[e, 64 i + l]; the 64 partials are then combined by an xor
// butterfly (32, 16, 8, 4, 2, 1), which leaves the same value in every lane.
// The x rows of the tile are staged in LDS (as fp32) one column chunk at a
// time; the chain order over i is unchanged by the chunking.
constexpr int kLogitTok = 8;
constexpr int kLogitExpPerWave = 2;
constexpr int kLogitChunk = 1024;  // columns staged per pass

__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x_lat,
                                                       const float* __restrict__ gate,
                                                       const float* __restrict__ bias, float* __restrict__ logits,
                                                       int Mr, int L, int E) {
  __shared__ float sx[kLogitTok][kLogitChunk];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kLogitTok;
  const int e0 = (blockIdx.y * 4 + wave) * kLogitExpPerWave;
  const float* wp[kLogitExpPerWave];
#pragma unroll
  for (int e = 0; e < kLogitExpPerWave; ++e) wp[e] = gate + static_cast<size_t>(min(e0 + e, E - 1)) * L + lane;

  float acc[kLogitTok][kLogitExpPerWave];
#pragma unroll
  for (int t = 0; t < kLogitTok; ++t)
#pragma unroll
    for (int e = 0; e < kLogitExpPerWave; ++e) acc[t][e] = 0.0f;

  for (int c0 = 0; c0 < L; c0 += kLogitChunk) {
    const int cw = min(kLogitChunk, L - c0);  // multiple of 256
    __syncthreads();
    // kLogitTok rows x cw columns as 8-element groups: 4 per thread
#pragma unroll
    for (int q = 0; q < kLogitTok * kLogitChunk / 8 / 256; ++q) {
      const int idx = tid + 256 * q;
      const int t = idx / (kLogitChunk / 8), c = 8 * (idx % (kLogitChunk / 8));
      const int tr = min(t0 + t, Mr - 1);
      const int cc = min(c, cw - 8);
      const uint4 v = *reinterpret_cast<const uint4*>(x_lat + static_cast<size_t>(tr) * L + c0 + cc);
      if (c < cw) {
        float* d = &sx[t][c];
        d[0] = bf16_bits_to_f32(v.x & 0xffffu);
        d[1] = bf16_bits_to_f32(v.x >> 16);
        d[2] = bf16_bits_to_f32(v.y & 0xffffu);
        d[3] = bf16_bits_to_f32(v.y >> 16);
        d[4] = bf16_bits_to_f32(v.z & 0xffffu);
        d[5] = bf16_bits_to_f32(v.z >> 16);
        d[6] = bf16_bits_to_f32(v.w & 0xffffu);
        d[7] = bf16_bits_to_f32(v.w >> 16);
      }
    }
    __syncthreads();
    // cw / 64 is a multiple of 4
    for (int i0 = 0; i0 < cw / 64; i0 += 4) {
      float wv[4][kLogitExpPerWave];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < kLogitExpPerWave; ++e) wv[u][e] = wp[e][c0 + 64 * (i0 + u)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int t = 0; t < kLogitTok; ++t) {
          const float xv = sx[t][64 * (i0 + u) + lane];
#pragma unroll
          for (int e = 0; e < kLogitExpPerWave; ++e) acc[t][e] = __builtin_fmaf(xv, wv[u][e], acc[t][e]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kLogitTok; ++t)
#pragma unroll
    for (int e = 0; e < kLogitExpPerWave; ++e) {
      float p = acc[t][e];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) p = p + __shfl_xor(p, off);
      acc[t][e] = p;
    }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < kLogitTok; ++t)
#pragma unroll
      for (int e = 0; e < kLogitExpPerWave; ++e)
        if (t0 + t < Mr && e0 + e < E)
          logits[static_cast<size_t>(t0 + t) * E + e0 + e] = acc[t][e] + (bias ? bias[e0 + e] : 0.0f);
  }
}

// ----------------------------------------------------------------- top-k --
// One wave per token: k rounds of a wave-wide argmax with key (logit desc,
// expert asc), then softmax over the k winners (sum in slot order).  Expert e
// lives in lane e % 64, slot e / 64; a lane rescans its slots only after its
// own best was taken.
constexpr int kGroup = 64;              // tokens per permutation group (one mask bit each)
constexpr int kMaxExpertsPerLane = 16;  // E <= 1024

__device__ __forceinline__ bool key_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int32_t* __restrict__ topk_ids,
                                                     float* __restrict__ topk_w, int Mr, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Mr) return;  // wave-uniform
  const int per = (E + 63) / 64;
  const float* lr = logits + static_cast<size_t>(t) * E;
  float v[kMaxExpertsPerLane];
#pragma unroll
  for (int m = 0; m < kMaxExpertsPerLane; ++m) {
    const int e = lane + 64 * m;
    v[m] = (m < per && e < E) ? lr[e] : 0.0f;
  }
  uint32_t taken = 0;
  auto lane_best = [&](float& bv, int& bi) {
    bv = 0.0f;
    bi = 0x7fffffff;
#pragma unroll
    for (int m = 0; m < kMaxExpertsPerLane; ++m) {
      const int e = lane + 64 * m;
      if (m < per && e < E && !((taken >> m) & 1u) && (bi == 0x7fffffff || key_better(v[m], e, bv, bi))) {
        bv = v[m];
        bi = e;
      }
    }
  };
  float lv;
  int li;
  lane_best(lv, li);
  float my_v = 0.0f, top_v = 0.0f;
  int my_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = lv;
    int bi = li;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || key_better(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if (j == 0) top_v = bv;
    if (lane == j) {
      my_v = bv;
      my_i = bi;
    }
    if ((bi & 63) == lane) {  // the winner's lane drops it and finds its next best
      taken |= 1u << (bi >> 6);
      lane_best(lv, li);
    }
  }
  const float u = (lane < k) ? expf(my_v - top_v) : 0.0f;
  float S = 0.0f;
  for (int j = 0; j < k; ++j) S = S + __shfl(u, j);
  if (lane < k) {
    topk_ids[static_cast<size_t>(t) * k + lane] = my_i;
    topk_w[static_cast<size_t>(t) * k + lane] = u / S;
  }
}

// --------------------------------------------------------- group masks --
// One wave per group of 64 tokens: mask[e] has bit (t mod 64) set when token t
// of the group is routed to e; its popcount is the group's row count for e.
__device__ __forceinline__ void build_group_masks(const int32_t* __restrict__ topk_ids, unsigned long long* s_mask,
                                                  int g, int Mr, int E, int k) {
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) s_mask[e] = 0ull;
  __syncthreads();
  const int t = g * kGroup + lane;
  if (t < Mr)
    for (int j = 0; j < k; ++j) atomicOr(&s_mask[topk_ids[static_cast<size_t>(t) * k + j]], 1ull << lane);
  __syncthreads();
}

__global__ __launch_bounds__(64) void k_router_hist(const int32_t* __restrict__ topk_ids, int32_t* __restrict__ hist,
                                                    int Mr, int E, int k, int ngroups) {
  __shared__ unsigned long long s_mask[1024];
  const int g = blockIdx.x;
  build_group_masks(topk_ids, s_mask, g, Mr, E, k);
  for (int e = threadIdx.x; e < E; e += 64) hist[static_cast<size_t>(e) * ngroups + g] = __popcll(s_mask[e]);
}

// ------------------------------------------------------------------ scan --
// One workgroup of 1024 threads: exclusive prefix sum of hist laid out
// [expert][group] (in place), which gives every (expert, group) its first
// row; expert_offsets[e] is the first row of expert e, expert_offsets[E] = R.
__global__ __launch_bounds__(1024) void k_router_scan(int32_t* __restrict__ hist, int32_t* __restrict__ expert_offsets,
                                                      int E, int ngroups) {
  __shared__ int s_tot[1024];
  const int n = E * ngroups;
  const int tid = threadIdx.x;
  const int chunk = (n + 1023) / 1024;
  const int b = tid * chunk;
  const int end = min(b + chunk, n);
  int sum = 0;
  for (int i = b; i < end; ++i) sum += hist[i];
  s_tot[tid] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan over the 1024 chunk totals
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = (tid >= off) ? s_tot[tid - off] : 0;
    __syncthreads();
    s_tot[tid] += add;
    __syncthreads();
  }
  int run = (tid == 0) ? 0 : s_tot[tid - 1];
  for (int i = b; i < end; ++i) {
    const int c = hist[i];
    hist[i] = run;
    run += c;
  }
  __syncthreads();
  const int total = s_tot[1023];
  for (int e = tid; e <= E; e += 1024) expert_offsets[e] = (e < E) ? (ngroups > 0 ? hist[e * ngroups] : 0) : total;
}

// --------------------------------------------------------------- scatter --
// One wave per token group: the row of pair (t, j) routed to e is the first
// row of (e, group) plus the number of earlier tokens of the group routed to
// e (a popcount of the group's mask below bit t mod 64).
__global__ __launch_bounds__(64) void k_router_scatter(const int32_t* __restrict__ topk_ids,
                                                       const int32_t* __restrict__ base,
                                                       int32_t* __restrict__ sorted_pair,
                                                       int32_t* __restrict__ pair_to_row, int Mr, int E, int k,
                                                       int ngroups) {
  __shared__ unsigned long long s_mask[1024];
  const int lane = threadIdx.x;
  const int g = blockIdx.x;
  build_group_masks(topk_ids, s_mask, g, Mr, E, k);
  const int t = g * kGroup + lane;
  if (t >= Mr) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const int p = t * k + j;
    const int e = topk_ids[p];
    const int row = base[static_cast<size_t>(e) * ngroups + g] + __popcll(s_mask[e] & below);
    sorted_pair[row] = p;
    pair_to_row[p] = row;
  }
}

}  // namespace moe_tail
