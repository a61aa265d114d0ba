// Routed-expert grouped GEMMs on gfx950 FP8 / FP8 x FP4 matrix cores.
//
// Routed experts are FP8 or FP4 block-scaled ("[Kimi K3][Kernel] Fuse BF16
// shared experts into latent MegaMoE tail", Summary: routed FP8/FP4 MegaMoE;
// L1 gate/up, activation, L2 down to a 3584-wide latent).
//
// Work decomposition: the rows of every expert (tokens routed to it, in the
// sorted order of the permutation) are cut into tiles of kBM rows.  Tiles are
// numbered expert after expert; a workgroup finds its (expert, first row) by a
// wave-wide prefix sum over the per-expert tile counts read from
// expert_offsets on the device, so no host read of routing data is needed and
// the grid is sized by the upper bound R / kBM + E.
//
// Each of the 4 waves of a workgroup owns its own output columns and streams
// its weight rows straight from HBM into MFMA operand registers (no weight
// byte is used by two waves); the next K step's fragments are loaded before
// the current step's MFMAs issue.  In the 16x16x128 MFMA lane l holds row
// (l % 16) of A (column (l % 16) of B); the K elements a lane holds depend on
// the operand width (see load_fp8_frag / load_weight_frag).  The f32 result
// holds rows 4 (l / 16) + i (i = 0..3) of column l % 16.
//
// Block scales: one MFMA covers one 128-wide K block, so its FP32 result is
// promoted with (activation scale of the row) x (weight scale of the 128x128
// block) and accumulated in FP32.  For MXFP4 the weight scale rides in the
// MFMA's e8m0 operand and only the activation scale is applied afterwards.
// NVFP4 (an e4m3 scale per 16 weights, which no scaled MFMA takes) runs on
// the FP16 matrix cores with the weights dequantized exactly in registers;
// the matrix's fp32 scale joins the activation scale in the promotion.
#pragma once

#include "common.hpp"

namespace moe_tail {

constexpr int kBM = 32;           // rows per routed tile (two 16-row MFMA tiles)
constexpr int kMaxKBlocks = 64;   // K <= 8192 for the LDS copy of activation scales

enum { FMT_FP8 = 0, FMT_MXFP4 = 1, FMT_NVFP4 = 2 };

// Finds the tile `mt` among the row tiles of the experts with fewer than
// `skip_at` rows (the others go to the tiled kernel).  Run by one wave;
// returns false when mt is past the last tile.
__device__ __forceinline__ bool find_routed_tile(const int32_t* __restrict__ off, int E, int mt, int skip_at,
                                                 int& e_out, int& row0_out, int& rows_out) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  const int eb = min(lane * per, E), ee = min(eb + per, E);
  auto ntile = [&](int e) {
    const int c = off[e + 1] - off[e];
    return c < skip_at ? (c + kBM - 1) / kBM : 0;
  };
  int local = 0;
  for (int e = eb; e < ee; ++e) local += ntile(e);
  int incl = local;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int n = __shfl_up(incl, d);
    if (lane >= d) incl += n;
  }
  const int total = __shfl(incl, 63);
  if (mt >= total) return false;
  const int excl = incl - local;
  int found_e = -1, found_row0 = 0, found_rows = 0;
  if (mt >= excl && mt < incl) {
    int acc = excl;
    for (int e = eb; e < ee; ++e) {
      const int n = ntile(e);
      if (mt < acc + n) {
        found_e = e;
        found_row0 = off[e] + (mt - acc) * kBM;
        found_rows = min(kBM, off[e + 1] - found_row0);
        break;
      }
      acc += n;
    }
  }
  // exactly one lane found it; broadcast
  const unsigned long long who = __ballot(found_e >= 0);
  const int src = __ffsll(static_cast<long long>(who)) - 1;
  e_out = __shfl(found_e, src);
  row0_out = __shfl(found_row0, src);
  rows_out = __shfl(found_rows, src);
  return true;
}

// FP8 operand fragment of one 128-wide K step.  The 16x16x128 MFMA takes an
// 8-bit operand's K elements as two halves: lane group g holds K [16 g, 16 g + 16)
// in its first four registers and K [64 + 16 g, 64 + 16 g + 16) in the last four.
__device__ __forceinline__ i32x8 load_fp8_frag(const uint8_t* __restrict__ row_ptr, int k0) {
  const int g = (threadIdx.x & 63) >> 4;
  const uint4 lo = *reinterpret_cast<const uint4*>(row_ptr + k0 + 16 * g);
  const uint4 hi = *reinterpret_cast<const uint4*>(row_ptr + k0 + 64 + 16 * g);
  return i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
               static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
}

// Weight fragment of one 128-wide K step of row `row` of a [N, K] matrix.
// FP8: the two-half layout above.  MXFP4: the 4-bit operand takes 32
// consecutive K elements per lane group, K [32 g, 32 g + 32) = 16 packed bytes,
// and the lane's e8m0 scale covers exactly those 32 elements.  NVFP4 (FP16
// matrix cores, mfma_fp8_nvfp4): the K of the FP8 layout, K [16 g, +16) and
// [64 + 16 g, +16) = packed bytes [8 g, +8) and [32 + 8 g, +8) of the step,
// with the e4m3 scales of those two 16-element blocks.
template <int kFmt>
__device__ __forceinline__ void load_weight_frag(const uint8_t* __restrict__ w, const void* __restrict__ ws,
                                                 size_t row, int K, int k0, i32x8& frag, int& scale) {
  if (kFmt == FMT_FP8) {
    frag = load_fp8_frag(w + row * K, k0);
    scale = 127;
  } else if (kFmt == FMT_NVFP4) {
    const int g = (threadIdx.x & 63) >> 4;
    const uint8_t* rp = w + row * (K / 2) + k0 / 2;
    const uint2 lo = *reinterpret_cast<const uint2*>(rp + 8 * g);
    const uint2 hi = *reinterpret_cast<const uint2*>(rp + 32 + 8 * g);
    frag = i32x8{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(hi.x), static_cast<int>(hi.y),
                 0, 0, 0, 0};
    const uint8_t* sp = static_cast<const uint8_t*>(ws) + row * (K / 16) + k0 / 16;
    scale = static_cast<int>(sp[g]) | (static_cast<int>(sp[4 + g]) << 8);
  } else {
    const int g = (threadIdx.x & 63) >> 4;
    const uint4 v = *reinterpret_cast<const uint4*>(w + row * (K / 2) + (k0 + 32 * g) / 2);
    frag = i32x8{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w), 0, 0, 0, 0};
    scale = static_cast<const uint8_t*>(ws)[row * (K / 32) + (k0 + 32 * g) / 32];
  }
}

__device__ __forceinline__ i32x8 load_act_frag(const uint8_t* __restrict__ row_ptr, int k0, bool valid) {
  if (!valid) return i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  return load_fp8_frag(row_ptr, k0);
}

template <int kFmt>
__device__ __forceinline__ f32x4 mfma_lowp(const i32x8& a, const i32x8& b, int scale_b) {
  if (kFmt == FMT_FP8) return mfma_fp8(a, b);
  if (kFmt == FMT_NVFP4) return mfma_fp8_nvfp4(a, b, scale_b);
  return mfma_fp8_fp4(a, b, scale_b);
}

// ------------------------------------------------------------------- L1 --
// g = x_hat . W1_hat^T for one tile of kBM rows x (128 gate + 128 up) columns,
// then h = silu(gate) * up and h -> e4m3 codes with one fp32 scale per 1x128
// block (the 128 h columns of this tile).  Grid: (R / kBM + E, I / 128).
template <int kFmt>
__global__ __launch_bounds__(256, 2) void k_routed_l1(const uint8_t* __restrict__ xq, const float* __restrict__ sx,
                                                   const int32_t* __restrict__ sorted_pair,
                                                   const int32_t* __restrict__ expert_offsets,
                                                   const uint8_t* __restrict__ w1, const void* __restrict__ w1s,
                                                   const float* __restrict__ w1t, uint8_t* __restrict__ hq,
                                                   float* __restrict__ sh, int E, int k, int L, int I, int skip_at) {
  __shared__ int s_tile[3];
  __shared__ int s_tok[kBM];
  __shared__ float s_sx[kBM * kMaxKBlocks];
  __shared__ float s_amax[4][kBM];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[kBM][128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = blockIdx.y;
  if (wave == 0) {
    int e, row0, rows;
    const bool ok = find_routed_tile(expert_offsets, E, blockIdx.x, skip_at, e, row0, rows);
    if (lane == 0) {
      s_tile[0] = ok ? e : -1;
      s_tile[1] = row0;
      s_tile[2] = rows;
    }
  }
  __syncthreads();
  // wave-uniform (scalar registers), so the per-step weight-scale loads are
  // scalar loads that do not wait behind the vector prefetch
  const int e = __builtin_amdgcn_readfirstlane(s_tile[0]);
  if (e < 0) return;  // uniform over the workgroup
  const int row0 = __builtin_amdgcn_readfirstlane(s_tile[1]), rows = __builtin_amdgcn_readfirstlane(s_tile[2]);
  const int nkb = L / 128;
  const int n_rows = expert_offsets[E];  // routed rows: the stride of sh, which is K-block-major
  if (tid < kBM) s_tok[tid] = (tid < rows) ? sorted_pair[row0 + tid] / k : -1;
  __syncthreads();
  for (int i = tid; i < kBM * nkb; i += 256) {
    const int r = i / nkb, kb = i % nkb;
    s_sx[i] = (s_tok[r] >= 0) ? sx[static_cast<size_t>(s_tok[r]) * nkb + kb] : 0.0f;
  }
  __syncthreads();

  const int l16 = lane & 15, g = lane >> 4;
  // A rows of the two 16-row tiles
  const uint8_t* arow[2];
  bool avalid[2];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int r = 16 * ms + l16;
    avalid[ms] = r < rows;
    arow[ms] = xq + static_cast<size_t>(avalid[ms] ? s_tok[r] : 0) * L;
  }
  // B rows: subtiles 0,1 gate, 2,3 up
  size_t brow[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int base = (ns < 2) ? 128 * nb : I + 128 * nb;
    brow[ns] = static_cast<size_t>(e) * (2 * I) + base + 32 * wave + 16 * (ns & 1) + l16;
  }
  const float* S1 = static_cast<const float*>(w1s) + static_cast<size_t>(e) * (2 * I / 128) * nkb;

  f32x4 acc[2][4];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Two fragment sets used in turn (no register copies, so the loads of one
  // set stay in flight while the other set's MFMAs issue).
  i32x8 fa[2][2], fb[2][4];
  int fs[2][4];
  auto load_step = [&](int set, int kb) {
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) load_weight_frag<kFmt>(w1, w1s, brow[ns], L, kb * 128, fb[set][ns], fs[set][ns]);
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) fa[set][ms] = load_act_frag(arow[ms], kb * 128, avalid[ms]);
  };
  auto mma_step = [&](int set, int kb) {
    float swg = 1.0f, swu = 1.0f;
    if (kFmt == FMT_FP8) {
      swg = S1[static_cast<size_t>(nb) * nkb + kb];
      swu = S1[static_cast<size_t>(I / 128 + nb) * nkb + kb];
    } else if (kFmt == FMT_NVFP4) {
      swg = swu = w1t[e];  // the matrix's fp32 scale
    }
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      float sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = s_sx[(16 * ms + 4 * g + i) * nkb + kb];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        const f32x4 p = mfma_lowp<kFmt>(fa[set][ms], fb[set][ns], fs[set][ns]);
        const float sw = (ns < 2) ? swg : swu;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ms][ns][i] += p[i] * (sa[i] * sw);
      }
    }
  };
  load_step(0, 0);
  for (int kb = 0; kb < nkb; kb += 2) {
    if (kb + 1 < nkb) load_step(1, kb + 1);
    mma_step(0, kb);
    if (kb + 2 < nkb) load_step(0, kb + 2);
    if (kb + 1 < nkb) mma_step(1, kb + 1);
  }

  // SwiGLU + per-row amax over this tile's 128 h columns
  float h[2][2][4];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = 0.0f;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        h[ms][c][i] = silu_mul_fast(acc[ms][c][i], acc[ms][2 + c][i]);
        m = fmaxf(m, fabsf(h[ms][c][i]));
      }
      m = group16_max(m);
      if (l16 == 0) s_amax[wave][16 * ms + 4 * g + i] = m;
    }
  }
  __syncthreads();
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * ms + 4 * g + i;
      const float amax = fmaxf(fmaxf(s_amax[0][r], s_amax[1][r]), fmaxf(s_amax[2][r], s_amax[3][r]));
      const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
      const float inv = 1.0f / s;
#pragma unroll
      for (int c = 0; c < 2; ++c) s_q[r][32 * wave + 16 * c + l16] = static_cast<uint8_t>(f32_to_e4m3(h[ms][c][i] * inv));
      if (wave == 0 && l16 == 0 && r < rows) sh[static_cast<size_t>(nb) * n_rows + row0 + r] = s;
    }
  __syncthreads();
  {
    const int r = tid >> 3, c16 = (tid & 7) * 16;
    if (r < rows)
      *reinterpret_cast<uint4*>(hq + static_cast<size_t>(row0 + r) * I + 128 * nb + c16) =
          *reinterpret_cast<const uint4*>(&s_q[r][c16]);
  }
}

// ------------------------------------------------------------------- L2 --
// y = h_hat . W2_hat^T for one tile of kBM rows x 128 latent columns, FP32
// output in sorted row order.  Grid: (R / kBM + E, L / 128).
template <int kFmt>
__global__ __launch_bounds__(256, 2) void k_routed_l2(const uint8_t* __restrict__ hq, const float* __restrict__ sh,
                                                   const int32_t* __restrict__ expert_offsets,
                                                   const uint8_t* __restrict__ w2, const void* __restrict__ w2s,
                                                   const float* __restrict__ w2t, float* __restrict__ y, int E, int L,
                                                   int I, int skip_at) {
  __shared__ int s_tile[3];
  __shared__ float s_sh[kBM * kMaxKBlocks];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = blockIdx.y;
  if (wave == 0) {
    int e, row0, rows;
    const bool ok = find_routed_tile(expert_offsets, E, blockIdx.x, skip_at, e, row0, rows);
    if (lane == 0) {
      s_tile[0] = ok ? e : -1;
      s_tile[1] = row0;
      s_tile[2] = rows;
    }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_tile[0]);
  if (e < 0) return;
  const int row0 = __builtin_amdgcn_readfirstlane(s_tile[1]), rows = __builtin_amdgcn_readfirstlane(s_tile[2]);
  const int nkb = I / 128;
  const int n_rows = expert_offsets[E];  // routed rows: the stride of sh, which is K-block-major
  for (int i = tid; i < kBM * nkb; i += 256) {
    const int r = i / nkb, kb = i % nkb;
    s_sh[i] = (r < rows) ? sh[static_cast<size_t>(kb) * n_rows + row0 + r] : 0.0f;
  }
  __syncthreads();

  const int l16 = lane & 15, g = lane >> 4;
  const uint8_t* arow[2];
  bool avalid[2];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int r = 16 * ms + l16;
    avalid[ms] = r < rows;
    arow[ms] = hq + static_cast<size_t>(row0 + (avalid[ms] ? r : 0)) * I;
  }
  size_t brow[2];
#pragma unroll
  for (int ns = 0; ns < 2; ++ns) brow[ns] = static_cast<size_t>(e) * L + 128 * nb + 32 * wave + 16 * ns + l16;
  const float* S2 = static_cast<const float*>(w2s) + (static_cast<size_t>(e) * (L / 128) + nb) * nkb;

  f32x4 acc[2][2];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  i32x8 fa[2][2], fb[2][2];
  int fs[2][2];
  auto load_step = [&](int set, int kb) {
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) load_weight_frag<kFmt>(w2, w2s, brow[ns], I, kb * 128, fb[set][ns], fs[set][ns]);
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) fa[set][ms] = load_act_frag(arow[ms], kb * 128, avalid[ms]);
  };
  auto mma_step = [&](int set, int kb) {
    const float sw = (kFmt == FMT_FP8) ? S2[kb] : (kFmt == FMT_NVFP4) ? w2t[e] : 1.0f;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      float sa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = s_sh[(16 * ms + 4 * g + i) * nkb + kb] * sw;
#pragma unroll
      for (int ns = 0; ns < 2; ++ns) {
        const f32x4 p = mfma_lowp<kFmt>(fa[set][ms], fb[set][ns], fs[set][ns]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ms][ns][i] += p[i] * sa[i];
      }
    }
  };
  load_step(0, 0);
  for (int kb = 0; kb < nkb; kb += 2) {
    if (kb + 1 < nkb) load_step(1, kb + 1);
    mma_step(0, kb);
    if (kb + 2 < nkb) load_step(0, kb + 2);
    if (kb + 1 < nkb) mma_step(1, kb + 1);
  }
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * ms + 4 * g + i;
      if (r < rows) {
        float* yr = y + static_cast<size_t>(row0 + r) * L + 128 * nb + 32 * wave + l16;
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) yr[16 * ns] = acc[ms][ns][i];
      }
    }
}

}  // namespace moe_tail
