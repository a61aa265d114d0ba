// BF16 GEMMs of the shared expert and of the up-projection, on gfx950 BF16
// matrix cores (16x16x32), FP32 accumulation.
//
// The shared expert is a BF16 SwiGLU MLP on the 7168-wide hidden vector and
// the routed latent goes through a BF16 3584 -> 7168 up-projection whose
// epilogue adds the shared output in FP32 before the one BF16 store
// ("[Kimi K3][Kernel] Fuse BF16 shared experts into latent MegaMoE tail",
// Summary; DeepGEMM PR 416 mirror, Summary).
//
// C[M, N] = A[M, K] . B[N, K]^T, both operands K-contiguous.  Operand layout
// of the 16x16x32 MFMA: lane l holds row l % 16 and 8 consecutive K elements
// of group l / 16; one 128-wide K step is four MFMAs, lane group g covering
// elements [32 g, 32 g + 32) of the step in both operands.  Decode-sized M
// uses k_dense_small below (K split over the grid, FP32 partials reduced in
// split order by k_dense_reduce, which applies the epilogue); larger M the
// LDS-tiled kernel of tile_gemm.hpp with the epilogue fused.
#pragma once

#include "common.hpp"

namespace moe_tail {

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

// ---------------------------------------------------------- small M --
// Decode-sized M (<= 128 rows): one workgroup covers every row, so each
// weight byte is read from HBM exactly once.  The A rows of one 128-wide K
// step are staged in LDS (double-buffered, shared by the 4 waves); each wave
// streams its own 16 * NT B rows with the next K step's fragments in flight.
// K is split over gridDim.y; FP32 partial sums partial[z][row][brow] are
// reduced (in split order) by k_dense_reduce, which applies the epilogue.
constexpr int kSmallMaxM = 128;
constexpr int kAStride = 136;  // LDS row stride in bf16 (272 B: rows start 4 banks apart)

template <int NT>
__global__ __launch_bounds__(256) void k_dense_small(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                     int M, int nbrows, int K, int kps, float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kSmallMaxM * kAStride];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int mt = (M + 15) / 16;
  const int rows_pad = 16 * mt;
  const int brow0 = blockIdx.x * 64 * NT + wave * 16 * NT;
  const uint16_t* bptr[NT];
#pragma unroll
  for (int ns = 0; ns < NT; ++ns) bptr[ns] = B + static_cast<size_t>(brow0 + 16 * ns + l16) * K;
  const int nk = K / 128;
  const int kb0 = blockIdx.y * kps, kb1 = min(kb0 + kps, nk);

  // A staging: rows_pad rows x 16 uint4 per K step; thread t moves uint4s t, t + 256, ...
  constexpr int kMaxStage = kSmallMaxM * 16 / 256;  // 8
  uint4 st[kMaxStage];
  auto stage_load = [&](int kb) {
#pragma unroll
    for (int i = 0; i < kMaxStage; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, c = idx & 15;
      st[i] = (r < M) ? *reinterpret_cast<const uint4*>(A + static_cast<size_t>(r) * K + kb * 128 + 8 * c)
                      : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto stage_store = [&](int buf) {
    // laundered buffer index: keeps these stores (and the waits on their
    // global loads) after the current step's MFMAs
    int b = buf;
    asm volatile("" : "+v"(b));
#pragma unroll
    for (int i = 0; i < kMaxStage; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 4, c = idx & 15;
      if (r < rows_pad) *reinterpret_cast<uint4*>(&sA[b][r * kAStride + 8 * c]) = st[i];
    }
  };

  f32x4 acc[8][NT];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int ns = 0; ns < NT; ++ns) acc[m][ns] = f32x4{0.f, 0.f, 0.f, 0.f};

  // B fragments in two sets used in turn; the A rows of the next step are
  // loaded before the next B fragments so that storing them to LDS waits for
  // the A loads only.
  bf16x8 fb[2][NT][4];
  auto mma_step = [&](int set, int buf) {
    const uint16_t* sa = &sA[buf][0];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < mt) {
        bf16x8 a[4];
        const uint16_t* ar = sa + (16 * m + l16) * kAStride + 32 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const bf16x8*>(ar + 8 * j);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int ns = 0; ns < NT; ++ns) acc[m][ns] = mfma_bf16(a[j], fb[set][ns][j], acc[m][ns]);
      }
    }
  };
  // Pipeline: step kb's A rows are in LDS buffer (kb - kb0) & 1 and its B
  // fragments in set (kb - kb0) & 1, while the registers hold step kb + 1's
  // A rows and the other set its B fragments (loaded one step earlier).  After
  // the MFMAs of step kb and a barrier, the A registers go to the other buffer
  // and step kb + 2 is loaded into the registers and the freed B set.
  auto step = [&](int set, int kb) {
    mma_step(set, set);
    __syncthreads();
    if (kb + 1 < kb1) {
      stage_store(set ^ 1);
      const int k2 = (kb + 2 < kb1) ? kb + 2 : kb1 - 1;
      stage_load(k2);
#pragma unroll
      for (int ns = 0; ns < NT; ++ns) load_bf16_frag(bptr[ns], k2 * 128, fb[set][ns]);
    }
    __syncthreads();
  };
  if (kb0 < kb1) {
    stage_load(kb0);
    stage_store(0);
#pragma unroll
    for (int ns = 0; ns < NT; ++ns) load_bf16_frag(bptr[ns], kb0 * 128, fb[0][ns]);
    const int k1 = (kb0 + 1 < kb1) ? kb0 + 1 : kb0;
    stage_load(k1);
#pragma unroll
    for (int ns = 0; ns < NT; ++ns) load_bf16_frag(bptr[ns], k1 * 128, fb[1][ns]);
  }
  __syncthreads();
  for (int kb = kb0; kb < kb1; kb += 2) {
    step(0, kb);
    if (kb + 1 < kb1) step(1, kb + 1);
  }

#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * m + 4 * g + i;
        if (row < M) {
          float* pr = partial + (static_cast<size_t>(blockIdx.y) * M + row) * nbrows + brow0 + l16;
#pragma unroll
          for (int ns = 0; ns < NT; ++ns) pr[16 * ns] = acc[m][ns][i];
        }
      }
    }
  }
}

// Sums the split-K partials in split order and applies the epilogue.
// One thread per output element; grid covers M * ncols (ncols = I_s for
// SWIGLU, N otherwise).
template <int kEpi>
__global__ __launch_bounds__(256) void k_dense_reduce(const float* __restrict__ partial, int M, int N, int splits,
                                                      DenseEpi ep) {
  // four neighbouring output columns per thread
  const int nraw = (kEpi == EPI_SWIGLU) ? 2 * ep.half : N;
  const int ncols = (kEpi == EPI_SWIGLU) ? ep.half : N;
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(M) * (ncols / 4)) return;
  const int row = static_cast<int>(idx / (ncols / 4)), col = 4 * static_cast<int>(idx % (ncols / 4));
  float4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
  for (int z = 0; z < splits; ++z) {
    const float* pr = partial + (static_cast<size_t>(z) * M + row) * nraw;
    const float4 a = *reinterpret_cast<const float4*>(pr + col);
    v0.x += a.x;
    v0.y += a.y;
    v0.z += a.z;
    v0.w += a.w;
    if (kEpi == EPI_SWIGLU) {
      const float4 b = *reinterpret_cast<const float4*>(pr + ep.half + col);
      v1.x += b.x;
      v1.y += b.y;
      v1.z += b.z;
      v1.w += b.w;
    }
  }
  dense_epilogue<kEpi>(ep, N, row, col + 0, v0.x, v1.x);
  dense_epilogue<kEpi>(ep, N, row, col + 1, v0.y, v1.y);
  dense_epilogue<kEpi>(ep, N, row, col + 2, v0.z, v1.z);
  dense_epilogue<kEpi>(ep, N, row, col + 3, v0.w, v1.w);
}

}  // namespace moe_tail
