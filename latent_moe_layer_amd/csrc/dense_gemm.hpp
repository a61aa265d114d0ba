// BF16 GEMMs of the shared expert and of the up-projection, on gfx950 BF16
// matrix cores (16x16x32), FP32 accumulation.
//
// The shared expert is a BF16 SwiGLU MLP on the 7168-wide hidden vector and
// the routed latent goes through a BF16 3584 -> 7168 up-projection whose
// epilogue adds the shared output in FP32 before the one BF16 store
// ("[Kimi K3][Kernel] Fuse BF16 shared experts into latent MegaMoE tail",
// Summary; DeepGEMM PR 416 mirror, Summary).
//
// C[M, N] = A[M, K] . B[N, K]^T, both operands K-contiguous.  A workgroup
// owns kDM rows x 4 waves x (2 x 16) B rows; each wave streams its own B rows
// from HBM into registers.  Operand layout of the 16x16x32 MFMA: lane l holds
// row l % 16 and 8 consecutive K elements of group l / 16; one 128-wide K step
// is four MFMAs, lane group g covering elements [32 g, 32 g + 32) of the step
// in both operands.  When the grid is too small to fill the chip, K is split
// over gridDim.z and FP32 partials go to a workspace that a second kernel
// reduces in split order (deterministic), applying the same epilogue.
#pragma once

#include "common.hpp"

namespace moe_tail {

constexpr int kDM = 32;  // rows per dense tile

enum { EPI_SWIGLU = 0, EPI_SHARED = 1, EPI_UPADD = 2 };

struct DenseEpi {
  int Mr;                 // EPI_SHARED: rows < Mr -> out0, rows >= Mr -> out1[row - Mr]
  int half;               // EPI_SWIGLU: I_s (up rows start here)
  uint16_t* out0;         // SWIGLU: hs [M, I_s]; SHARED: s [Mr, N]; UPADD: out [M, N]
  uint16_t* out1;         // SHARED: shared_out [M - Mr, N]
  const uint16_t* addsrc; // UPADD: s [M, N] bf16 added in FP32
};

// Column of output produced by B row `brow` (SWIGLU pairs gate row c with up
// row half + c into output column c).
template <int kEpi>
__device__ __forceinline__ void dense_epilogue(const DenseEpi& ep, int N, int row, int col, float v0, float v1) {
  if (kEpi == EPI_SWIGLU) {
    ep.out0[static_cast<size_t>(row) * ep.half + col] = static_cast<uint16_t>(f32_to_bf16_bits(silu_mul(v0, v1)));
  } else if (kEpi == EPI_SHARED) {
    const uint16_t b = static_cast<uint16_t>(f32_to_bf16_bits(v0));
    if (row < ep.Mr) ep.out0[static_cast<size_t>(row) * N + col] = b;
    else ep.out1[static_cast<size_t>(row - ep.Mr) * N + col] = b;
  } else {
    const float s = bf16_bits_to_f32(ep.addsrc[static_cast<size_t>(row) * N + col]);
    ep.out0[static_cast<size_t>(row) * N + col] = static_cast<uint16_t>(f32_to_bf16_bits(v0 + s));
  }
}

__device__ __forceinline__ void load_bf16_frag(const uint16_t* __restrict__ row_ptr, int k0, bf16x8 (&f)[4]) {
  const int g = (threadIdx.x & 63) >> 4;
  const uint4* p = reinterpret_cast<const uint4*>(row_ptr + k0 + 32 * g);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 v = p[j];
    f[j] = __builtin_bit_cast(bf16x8, v);
  }
}

// Grid: (ceil(M / kDM), n_tiles, splits).  n_tiles = N / 128, or I_s / 64 for
// SWIGLU (each tile: 64 gate + 64 up B rows).  Split z covers K steps
// [z * kps, min((z + 1) * kps, K / 128)).  With splits > 1 the raw FP32 sums go
// to partial[z][row][brow] (row stride nraw = number of B rows).
template <int kEpi>
__global__ __launch_bounds__(256) void k_dense_bf16(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                    int M, int N, int K, int kps, float* __restrict__ partial,
                                                    DenseEpi ep) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * kDM;
  const int nraw = (kEpi == EPI_SWIGLU) ? 2 * ep.half : N;
  int brow[2];
  if (kEpi == EPI_SWIGLU) {
    brow[0] = 64 * blockIdx.y + 16 * wave + l16;
    brow[1] = ep.half + brow[0];
  } else {
    brow[0] = 128 * blockIdx.y + 32 * wave + l16;
    brow[1] = brow[0] + 16;
  }
  const uint16_t* arow[2];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) arow[ms] = A + static_cast<size_t>(min(m0 + 16 * ms + l16, M - 1)) * K;
  const uint16_t* bptr[2];
#pragma unroll
  for (int ns = 0; ns < 2; ++ns) bptr[ns] = B + static_cast<size_t>(brow[ns]) * K;

  f32x4 acc[2][2];
#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / 128;
  const int kb0 = blockIdx.z * kps, kb1 = min(kb0 + kps, nk);
  for (int kb = kb0; kb < kb1; ++kb) {
    const int k0 = kb * 128;
    bf16x8 a[2][4], b[2][4];
#pragma unroll
    for (int ns = 0; ns < 2; ++ns) load_bf16_frag(bptr[ns], k0, b[ns]);
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) load_bf16_frag(arow[ms], k0, a[ms]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) acc[ms][ns] = mfma_bf16(a[ms][j], b[ns][j], acc[ms][ns]);
  }

#pragma unroll
  for (int ms = 0; ms < 2; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 16 * ms + 4 * g + i;
      if (row >= M) continue;
      if (gridDim.z > 1) {
        float* pr = partial + (static_cast<size_t>(blockIdx.z) * M + row) * nraw;
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) pr[brow[ns]] = acc[ms][ns][i];
      } else if (kEpi == EPI_SWIGLU) {
        dense_epilogue<kEpi>(ep, N, row, brow[0], acc[ms][0][i], acc[ms][1][i]);
      } else {
#pragma unroll
        for (int ns = 0; ns < 2; ++ns) dense_epilogue<kEpi>(ep, N, row, brow[ns], acc[ms][ns][i], 0.0f);
      }
    }
}

// Sums the split-K partials in split order and applies the epilogue.
// One thread per output element; grid covers M * ncols (ncols = I_s for
// SWIGLU, N otherwise).
template <int kEpi>
__global__ __launch_bounds__(256) void k_dense_reduce(const float* __restrict__ partial, int M, int N, int splits,
                                                      DenseEpi ep) {
  const int nraw = (kEpi == EPI_SWIGLU) ? 2 * ep.half : N;
  const int ncols = (kEpi == EPI_SWIGLU) ? ep.half : N;
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(M) * ncols) return;
  const int row = static_cast<int>(idx / ncols), col = static_cast<int>(idx % ncols);
  float v0 = 0.0f, v1 = 0.0f;
  for (int z = 0; z < splits; ++z) {
    const float* pr = partial + (static_cast<size_t>(z) * M + row) * nraw;
    v0 += pr[col];
    if (kEpi == EPI_SWIGLU) v1 += pr[ep.half + col];
  }
  dense_epilogue<kEpi>(ep, N, row, col, v0, v1);
}

}  // namespace moe_tail
