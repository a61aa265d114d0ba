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
// One workgroup = 4 waves; tile of kTok tokens x (4 * kEPW) experts
// (kLogitTok x 4 kLogitExpPerWave unless the launch is small).  Lane l of a wave accumulates p[l] = fma-chain over i of
// x[64 i + l] * W[e, 64 i + l]; the 64 partials are then combined by an xor
// butterfly (32, 16, 8, 4, 2, 1), which leaves the same value in every lane.
// The kernel is latency-bound (a few hundred KB in all), so it waits for
// memory once: the tile's x rows (bf16) go to LDS with direct loads while
// every gate value a lane needs (up to kLogitChunk columns) is loaded into
// registers, and only then does the arithmetic start.
constexpr int kLogitTok = 4;
constexpr int kLogitExpPerWave = 2;
constexpr int kLogitChunk = 4096;  // gate columns in registers at once
// dynamic LDS: the x tile, kTok x L bf16.  Few tokens (a launch of fewer than
// kLogitSmallGrid workgroups): 2 tokens x 1 expert per wave instead, four
// times the workgroups, each logit's chain unchanged (the 16-token workload:
// 4 -> 16 workgroups).
constexpr int kLogitSmallGrid = 64;

template <int kTok, int kEPW>
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x_lat,
                                                       const float* __restrict__ gate,
                                                       const float* __restrict__ bias, float* __restrict__ logits,
                                                       int Mr, int L, int E) {
  static_assert((kTok * 256 * 2) % 1024 == 0, "the x tile in whole 1 KB blocks for every L a multiple of 256");
  extern __shared__ __attribute__((aligned(16))) uint16_t sx[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int t0 = blockIdx.x * kTok;
  const int e0 = (blockIdx.y * 4 + wave) * kEPW;

  // x rows t0 .. t0 + kTok - 1 as one linear byte array: 1 KB block j is
  // loaded by wave j % 4, lane l copying bytes [16 (64 j + l), +16) (rows
  // past Mr read as zeros)
  {
    const uint32_t row_bytes = static_cast<uint32_t>(L) * 2;
    const int nrows = max(0, min(kTok, Mr - t0));
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(x_lat + static_cast<size_t>(t0) * L, static_cast<uint32_t>(nrows) * row_bytes);
    const int nblocks = (kTok * L * 2) / 1024;  // L is a multiple of 256
    for (int j = wv; j < nblocks; j += 4) dma16(r, reinterpret_cast<uint8_t*>(sx) + 1024 * j, 16u * (64 * j + lane), 0);
  }

  // gate row of each expert as a buffer (columns past L read as zeros)
  __amdgpu_buffer_rsrc_t wr[kEPW];
#pragma unroll
  for (int e = 0; e < kEPW; ++e)
    wr[e] = make_rsrc(gate + static_cast<size_t>(min(e0 + e, E - 1)) * L, static_cast<uint32_t>(L) * 4);
  constexpr int kPer = kLogitChunk / 64;  // gate values per lane and expert
  float acc[kTok][kEPW];
#pragma unroll
  for (int t = 0; t < kTok; ++t)
#pragma unroll
    for (int e = 0; e < kEPW; ++e) acc[t][e] = 0.0f;

  for (int c0 = 0; c0 < L; c0 += kLogitChunk) {  // one pass for L <= kLogitChunk
    float w[kEPW][kPer];
#pragma unroll
    for (int e = 0; e < kEPW; ++e)
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        w[e][u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(wr[e], 4 * lane, 4 * (c0 + 64 * u), 0));
    ring_barrier<0>();  // the gate values and (first pass) the x tile are in
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (c0 + 64 * u < L) {
#pragma unroll
        for (int t = 0; t < kTok; ++t) {
          const float xv = bf16_bits_to_f32(sx[t * L + c0 + 64 * u + lane]);
#pragma unroll
          for (int e = 0; e < kEPW; ++e) acc[t][e] = __builtin_fmaf(xv, w[e][u], acc[t][e]);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kTok; ++t)
#pragma unroll
    for (int e = 0; e < kEPW; ++e) {
      float p = acc[t][e];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) p = p + __shfl_xor(p, off);
      acc[t][e] = p;
    }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < kTok; ++t)
#pragma unroll
      for (int e = 0; e < kEPW; ++e)
        if (t0 + t < Mr && e0 + e < E)
          logits[static_cast<size_t>(t0 + t) * E + e0 + e] = acc[t][e] + (bias ? bias[e0 + e] : 0.0f);
  }
}

// Many tokens: the 4-token tile above re-reads every gate row once per 4
// tokens (about 1 GB of L2 traffic at 4096 tokens).  Here a workgroup of 4
// waves takes 2 kTW tokens x 2 kEW experts; wave w computes tokens kTW (w & 1)
// .. and experts kEW (w >> 1) .. .  Per chunk of kLgC columns one stage holds
// the x rows (bf16) and the gate rows (fp32), loaded with 1 KB direct loads
// (6 per wave) and double-buffered, so a lane reads per 64-column step kTW x
// values and kEW gate values from LDS for kTW x kEW fused multiply-adds.  The
// order of operations per logit is the one above: lane l's chain over i of
// x[64 i + l] * W[e, 64 i + l], i ascending, then the xor butterfly, then the
// bias.  At 2048 tokens x 384 experts: 8 x 8 per wave 142-150 us; 4 x 16 and
// 16 x 4 171-181, 8 x 16 and 16 x 8 241-260 (fewer waves per SIMD); an
// earlier form with the gate values loaded into registers (one 4-byte load
// per value and lane) 188 us.  Stages of 256 columns (48 KB of LDS for two)
// let 3 workgroups share a CU, stages of 128 columns 5 (then the registers
// limit): the launch takes 128-column stages when its workgroups need more
// than one round at 3 per CU (4096 x 64: 56.4 -> 51.6 us; 2048 x 384: 149.2
// -> 146.7), 256-column ones otherwise (half as many barriers; 1024 x 128:
// 30.4 against 34.6 us).
constexpr int kWideMinTokens = 512;
template <int kTW, int kEW, int kLgC>  // kLgC: columns per stage (128 or 256; L is a multiple of 256)
__global__ __launch_bounds__(256, kLgC == 128 ? 4 : 1) void k_router_logits_tile(const uint16_t* __restrict__ x_lat,
                                                               const float* __restrict__ gate,
                                                               const float* __restrict__ bias,
                                                               float* __restrict__ logits, int Mr, int L, int E) {
  constexpr int kRowsX = 2 * kTW, kRowsG = 2 * kEW;
  constexpr int kXBytes = kRowsX * kLgC * 2, kGBytes = kRowsG * kLgC * 4;
  constexpr int kStage = kXBytes + kGBytes;
  constexpr int kPieces = kStage / 1024;   // 1 KB direct loads per stage
  constexpr int kXRows = 1024 / (2 * kLgC);  // x rows per piece
  constexpr int kGRows = 1024 / (4 * kLgC);  // gate rows per piece
  constexpr int kXPieces = kRowsX / kXRows;
  static_assert(kGRows >= 1 && kRowsX % kXRows == 0 && kRowsG % kGRows == 0 && kPieces % 4 == 0,
                "whole rows per 1 KB piece; the same number of pieces for each of the 4 waves");
  __shared__ __attribute__((aligned(16))) uint8_t st[2][kStage];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int tw = wv & 1, ew = wv >> 1;
  const int t0 = blockIdx.x * kRowsX, e0 = blockIdx.y * kRowsG;
  const int nx = max(0, min(kRowsX, Mr - t0)), ng = max(0, min(kRowsG, E - e0));
  // rows past Mr / E read zeros
  const __amdgpu_buffer_rsrc_t rx =
      make_rsrc(x_lat + static_cast<size_t>(t0) * L, static_cast<uint32_t>(nx) * static_cast<uint32_t>(L) * 2u);
  const __amdgpu_buffer_rsrc_t rg =
      make_rsrc(gate + static_cast<size_t>(e0) * L, static_cast<uint32_t>(ng) * static_cast<uint32_t>(L) * 4u);
  // piece q of chunk c: q < kXPieces: x rows kXRows q .. (64 / kXRows lanes
  // each); else gate rows kGRows (q - kXPieces) .. (64 / kGRows lanes each)
  auto load = [&](int c, int b) {
#pragma unroll
    for (int j = 0; j < kPieces / 4; ++j) {
      const int q = wv + 4 * j;
      if (q < kXPieces) {
        constexpr int kLanes = 64 / kXRows;
        const uint32_t r = static_cast<uint32_t>(kXRows * q + lane / kLanes);
        dma16(rx, st[b] + 1024 * q,
              r * static_cast<uint32_t>(L) * 2u + static_cast<uint32_t>(c) * (kLgC * 2) + 16u * (lane % kLanes), 0);
      } else {
        constexpr int kLanes = 64 / kGRows;
        const uint32_t r = static_cast<uint32_t>(kGRows * (q - kXPieces) + lane / kLanes);
        dma16(rg, st[b] + 1024 * q,
              r * static_cast<uint32_t>(L) * 4u + static_cast<uint32_t>(c) * (kLgC * 4) + 16u * (lane % kLanes), 0);
      }
    }
  };
  float acc[kTW][kEW];
#pragma unroll
  for (int t = 0; t < kTW; ++t)
#pragma unroll
    for (int e = 0; e < kEW; ++e) acc[t][e] = 0.0f;
  const int nch = L / kLgC;
  load(0, 0);
  for (int c = 0; c < nch; ++c) {
    const int b = c & 1;
    ring_barrier<0>();  // this wave's loads of chunk c, then every wave's; every wave done with chunk c - 1
    if (c + 1 < nch) load(c + 1, b ^ 1);
    const uint16_t* xr = reinterpret_cast<const uint16_t*>(st[b]) + kTW * tw * kLgC;
    const float* gr = reinterpret_cast<const float*>(st[b] + kXBytes) + kEW * ew * kLgC;
#pragma unroll
    for (int u = 0; u < kLgC / 64; ++u) {
      float xv[kTW], gv[kEW];
#pragma unroll
      for (int t = 0; t < kTW; ++t) xv[t] = bf16_bits_to_f32(xr[t * kLgC + 64 * u + lane]);
#pragma unroll
      for (int e = 0; e < kEW; ++e) gv[e] = gr[e * kLgC + 64 * u + lane];
#pragma unroll
      for (int t = 0; t < kTW; ++t)
#pragma unroll
        for (int e = 0; e < kEW; ++e) acc[t][e] = __builtin_fmaf(xv[t], gv[e], acc[t][e]);
    }
  }
  // each logit reduced over the 64 lanes, then stored by lane t (with
  // 128-column stages, which leave fewer registers, each one as soon as it is
  // complete)
  const int tb = t0 + kTW * tw, eb = e0 + kEW * ew;
#pragma unroll
  for (int t = 0; t < kTW; ++t)
#pragma unroll
    for (int e = 0; e < kEW; ++e) {
      float p = acc[t][e];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) p = p + __shfl_xor(p, off);
      if constexpr (kLgC == 128) {
        if (lane == t && tb + t < Mr && eb + e < E)
          logits[static_cast<size_t>(tb + t) * E + eb + e] = p + (bias ? bias[eb + e] : 0.0f);
      } else {
        acc[t][e] = p;
      }
    }
  if constexpr (kLgC != 128) {
#pragma unroll
    for (int t = 0; t < kTW; ++t)
      if (lane == t && tb + t < Mr) {
#pragma unroll
        for (int e = 0; e < kEW; ++e)
          if (eb + e < E) logits[static_cast<size_t>(tb + t) * E + eb + e] = acc[t][e] + (bias ? bias[eb + e] : 0.0f);
      }
  }
}

// ----------------------------------------------------------------- top-k --
// One wave per token: k rounds of a wave-wide argmax with key (logit desc,
// expert asc), then softmax over the k winners (sum in slot order).  Expert e
// lives in lane e % 64, slot e / 64; a lane rescans its slots only after its
// own best was taken.  The argmax reduces within each 16-lane row with DPP
// lane moves (xor 1, xor 2, mirror within 8, mirror within 16: ALU ops,
// not LDS round trips) and then across the 4 rows through readlane.
constexpr int kGroup = 64;              // tokens per permutation group (one mask bit each)
constexpr int kMaxExpertsPerLane = 16;  // E <= 1024
constexpr int kNoExpert = 0x7fffffff;

__device__ __forceinline__ bool key_better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// (value, index) of the better key of this lane and the lane kCtrl names
template <int kCtrl>
__device__ __forceinline__ void argmax_dpp(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(bv), __float_as_int(bv), kCtrl, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(bi, bi, kCtrl, 0xf, 0xf, false);
  if (oi != kNoExpert && (bi == kNoExpert || key_better(ov, oi, bv, bi))) {
    bv = ov;
    bi = oi;
  }
}

// wave-wide best key; the result is the same in every lane
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
  argmax_dpp<0xB1>(bv, bi);   // quad_perm(1, 0, 3, 2): lane ^ 1
  argmax_dpp<0x4E>(bv, bi);   // quad_perm(2, 3, 0, 1): lane ^ 2
  argmax_dpp<0x141>(bv, bi);  // row_half_mirror: quads 0 <-> 1 of each 8
  argmax_dpp<0x140>(bv, bi);  // row_mirror: halves of each 16-lane row
  float cv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int ci = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float ov = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
    const int oi = __builtin_amdgcn_readlane(bi, 16 * r);
    if (oi != kNoExpert && (ci == kNoExpert || key_better(ov, oi, cv, ci))) {
      cv = ov;
      ci = oi;
    }
  }
  bv = cv;
  bi = ci;
}

// Top-k and softmax of one token whose logit of expert e sits in v[e / 64]
// of lane e % 64: lane j < k ends with slot j's expert and weight.
template <int kPer>  // experts per lane: ceil(E / 64) <= kPer
__device__ __forceinline__ void topk_token(const float (&v)[kPer], int lane, int E, int k, int& id, float& wgt) {
  uint32_t taken = 0;
  auto lane_best = [&](float& bv, int& bi) {
    bv = 0.0f;
    bi = kNoExpert;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int e = lane + 64 * m;
      if (e < E && !((taken >> m) & 1u) && (bi == kNoExpert || key_better(v[m], e, bv, bi))) {
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
    wave_argmax(bv, bi);
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
  id = my_i;
  wgt = u / S;
}

template <int kPer>
__global__ __launch_bounds__(256) void k_router_topk(const float* __restrict__ logits, int32_t* __restrict__ topk_ids,
                                                     float* __restrict__ topk_w, int Mr, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Mr) return;  // wave-uniform
  const float* lr = logits + static_cast<size_t>(t) * E;
  float v[kPer];
#pragma unroll
  for (int m = 0; m < kPer; ++m) {
    const int e = lane + 64 * m;
    v[m] = (e < E) ? lr[e] : 0.0f;
  }
  int id;
  float wgt;
  topk_token<kPer>(v, lane, E, k, id, wgt);
  if (lane < k) {
    topk_ids[static_cast<size_t>(t) * k + lane] = id;
    topk_w[static_cast<size_t>(t) * k + lane] = wgt;
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
// Up to kScanLds cells are first copied to LDS with coalesced loads, so that
// each thread's run of `chunk` cells costs LDS reads rather than one global
// round trip after another (2048 tokens x 384 experts: 12288 cells).
constexpr int kScanLds = 16384;

__global__ __launch_bounds__(1024) void k_router_scan(int32_t* __restrict__ hist, int32_t* __restrict__ expert_offsets,
                                                      int E, int ngroups) {
  __shared__ int s_tot[32];  // wave totals, then their inclusive prefixes
  __shared__ int s_h[kScanLds];
  const int n = E * ngroups;
  const int tid = threadIdx.x;
  const bool in_lds = n <= kScanLds;
  if (in_lds) {
    for (int i = tid; i < n; i += 1024) s_h[i] = hist[i];
    __syncthreads();
  }
  const int chunk = (n + 1023) / 1024;
  const int b = tid * chunk;
  const int end = min(b + chunk, n);
  int sum = 0;
  if (in_lds)
    for (int i = b; i < end; ++i) sum += s_h[i];
  else
    for (int i = b; i < end; ++i) sum += hist[i];
  // inclusive scan of the 1024 chunk totals: within each wave by lane
  // shifts, then over the 16 wave totals by wave 0
  const int lane = tid & 63, wave = tid >> 6;
  int inc = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off);
    if (lane >= off) inc += o;
  }
  if (lane == 63) s_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? s_tot[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int o = __shfl_up(w, off);
      if (lane >= off) w += o;
    }
    if (lane < 16) s_tot[16 + lane] = w;  // inclusive totals of waves 0..lane
  }
  __syncthreads();
  int run = inc - sum + (wave > 0 ? s_tot[16 + wave - 1] : 0);  // exclusive prefix of this chunk
  if (in_lds) {
    // prefixes in place in LDS, then written out with coalesced stores
    for (int i = b; i < end; ++i) {
      const int c = s_h[i];
      s_h[i] = run;
      run += c;
    }
    __syncthreads();
    for (int i = tid; i < n; i += 1024) hist[i] = s_h[i];
  } else {
    for (int i = b; i < end; ++i) {
      const int c = hist[i];
      hist[i] = run;
      run += c;
    }
    __syncthreads();
  }
  const int total = s_tot[16 + 15];
  const int* first = in_lds ? s_h : hist;
  for (int e = tid; e <= E; e += 1024) expert_offsets[e] = (e < E) ? (ngroups > 0 ? first[e * ngroups] : 0) : total;
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

// ------------------------------------------------------- fused (small) --
// The three steps above (group masks, exclusive scan over [expert][group],
// scatter) in one workgroup of 1024 threads, for up to kSortSmall (group,
// expert) cells; the same rows result.
constexpr int kSortSmall = 4096;
constexpr int kSortSmallGroups = 24;  // token groups of 64 (beyond: the grid-wide passes are faster)

// The permutation of one workgroup (group masks, exclusive scan over
// [expert][group], scatter) from the pairs' experts ids[t * k + j].
__device__ __forceinline__ void sort_small(const int32_t* ids, int32_t* __restrict__ expert_offsets,
                                           int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_to_row, int Mr,
                                           int E, int k, int ngroups) {
  __shared__ unsigned long long s_mask[kSortSmall];  // [group][expert]
  __shared__ int s_base[kSortSmall];                 // [expert][group]: first row
  __shared__ int s_tot[1024];
  const int tid = threadIdx.x;
  const int n = E * ngroups;
  for (int i = tid; i < n; i += 1024) s_mask[i] = 0ull;
  __syncthreads();
  const int npairs = Mr * k;
  for (int p = tid; p < npairs; p += 1024) {
    const int t = p / k;
    atomicOr(&s_mask[(t / kGroup) * E + ids[p]], 1ull << (t % kGroup));
  }
  __syncthreads();
  // exclusive scan of the counts in [expert][group] order
  const int chunk = (n + 1023) / 1024;
  const int b = tid * chunk, end = min(b + chunk, n);
  int sum = 0;
  for (int i = b; i < end; ++i) {
    const int e = i / ngroups, g = i - e * ngroups;
    sum += __popcll(s_mask[g * E + e]);
  }
  s_tot[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = (tid >= off) ? s_tot[tid - off] : 0;
    __syncthreads();
    s_tot[tid] += a;
    __syncthreads();
  }
  int run = (tid == 0) ? 0 : s_tot[tid - 1];
  for (int i = b; i < end; ++i) {
    const int e = i / ngroups, g = i - e * ngroups;
    s_base[i] = run;
    run += __popcll(s_mask[g * E + e]);
  }
  __syncthreads();
  for (int e = tid; e <= E; e += 1024) expert_offsets[e] = (e < E) ? (ngroups > 0 ? s_base[e * ngroups] : 0) : s_tot[1023];
  for (int p = tid; p < npairs; p += 1024) {
    const int t = p / k, g = t / kGroup, bit = t % kGroup;
    const int e = ids[p];
    const unsigned long long below = (bit == 0) ? 0ull : (~0ull >> (64 - bit));
    const int row = s_base[e * ngroups + g] + __popcll(s_mask[g * E + e] & below);
    sorted_pair[row] = p;
    pair_to_row[p] = row;
  }
}

__global__ __launch_bounds__(1024) void k_router_sort(const int32_t* __restrict__ topk_ids,
                                                      int32_t* __restrict__ expert_offsets,
                                                      int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_to_row,
                                                      int Mr, int E, int k, int ngroups) {
  sort_small(topk_ids, expert_offsets, sorted_pair, pair_to_row, Mr, E, k, ngroups);
}

// Up to 16 tokens: top-k and the permutation in one workgroup of 16 waves
// (one launch instead of two).  Every logit is staged in LDS with direct
// loads; wave t takes token t through topk_token (the same arithmetic as
// k_router_topk) and keeps its experts in LDS for sort_small.  (With more
// tokens a wave would work through several tokens one after another, whose
// argmax rounds then cost more than the launch saved: 128 tokens x 64
// experts took 62 us against 6 + 4.4 us for the two launches.)
constexpr int kTopkSortTokens = 16;

template <int kPer>
__global__ __launch_bounds__(1024) void k_router_topk_sort(const float* __restrict__ logits,
                                                           int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
                                                           int32_t* __restrict__ expert_offsets,
                                                           int32_t* __restrict__ sorted_pair,
                                                           int32_t* __restrict__ pair_to_row, int Mr, int E, int k,
                                                           int ngroups) {
  __shared__ __attribute__((aligned(16))) float s_lg[kTopkSortTokens * 64 * kMaxExpertsPerLane];
  __shared__ int32_t s_ids[kTopkSortTokens * 16];  // top_k <= 16
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  {
    // 1 KB piece j of the logits by wave j % 16 (bytes past Mr * E read as zeros)
    const uint32_t bytes = static_cast<uint32_t>(Mr) * static_cast<uint32_t>(E) * 4u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(logits, bytes);
    const int npieces = static_cast<int>((bytes + 1023u) / 1024u);
    for (int j = wv; j < npieces; j += 16)
      dma16(r, reinterpret_cast<uint8_t*>(s_lg) + 1024 * j, 16u * (64u * j + lane), 0);
  }
  ring_barrier<0>();
  const int t = wv;
  if (t < Mr) {  // wave-uniform
    const float* lr = s_lg + static_cast<size_t>(t) * E;
    float v[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int e = lane + 64 * m;
      v[m] = (e < E) ? lr[e] : 0.0f;
    }
    int id;
    float wgt;
    topk_token<kPer>(v, lane, E, k, id, wgt);
    if (lane < k) {
      topk_ids[static_cast<size_t>(t) * k + lane] = id;
      topk_w[static_cast<size_t>(t) * k + lane] = wgt;
      s_ids[t * k + lane] = id;
    }
  }
  __syncthreads();
  sort_small(s_ids, expert_offsets, sorted_pair, pair_to_row, Mr, E, k, ngroups);
}

}  // namespace moe_tail
