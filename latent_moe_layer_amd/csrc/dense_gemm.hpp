// BF16 GEMMs of the shared expert and of the up-projection, on gfx950 BF16
// matrix cores (16x16x32), FP32 accumulation.
//
// The shared expert is a BF16 SwiGLU MLP on the 7168-wide hidden vector and
// the routed latent goes through a BF16 3584 -> 7168 up-projection whose
// epilogue adds the shared output in FP32 before the one BF16 store
// ("[Kimi K3][Kernel] Fuse BF16 shared experts into latent MegaMoE tail",
// Summary; DeepGEMM PR 416 mirror, Summary).
//
// C[M, N] = A[M, K] . B[N, K]^T, both operands K-contiguous; one 64-wide K
// step of the 16x16x32 MFMA is two MFMAs, lane group g holding 8 consecutive K
// elements of each.  Decode-sized M uses k_dense_small below (K split over
// the grid, FP32 partials reduced in split order by k_dense_reduce, which
// applies the epilogue); larger M the LDS-tiled kernel of tile_gemm.hpp with
// the epilogue fused.
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

// ---------------------------------------------------------- small M --
// Decode-sized M (<= 128 rows): a workgroup covers every row and kSkinnyN
// weight rows over a range of K steps (K is split over gridDim.y), so each
// weight byte is read from HBM once.  Both operands go straight from memory
// into a kSkinnyStages-deep LDS ring (buffer loads with the LDS flag, whole
// 128-byte lines per load, rows XOR-swizzled as in the tiled kernel), so that
// five steps of weights are in flight per CU.  Each of the 8 waves (two per
// SIMD, so one can issue while the other waits) multiplies rows
// [16 w, 16 w + 16) by the kSkinnyN weight rows; FP32 partial sums
// partial[z][row][brow] are reduced in split order by k_dense_reduce, which
// applies the epilogue.
constexpr int kSmallMaxM = 128;
constexpr int kSkinnyN = 64;      // weight rows per workgroup
constexpr int kSkinnyStages = 6;  // LDS ring depth

__global__ __launch_bounds__(512) void k_dense_small(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                     int M, int nbrows, int K, int kps, float* __restrict__ partial) {
  constexpr int kABytes = kSmallMaxM * 128;  // one K step of 64 BF16: 128 rows x 128 bytes
  constexpr int kBBytes = kSkinnyN * 128;
  constexpr int kStage = kABytes + kBBytes;
  constexpr int kLoads = 3;  // per wave and stage: A blocks w + 8 i (i < 2), B block w
  __shared__ __attribute__((aligned(16))) uint8_t ring[kSkinnyStages * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int l16 = lane & 15, g = lane >> 4;
  const int brow0 = blockIdx.x * kSkinnyN;
  const int nk = K / 64;
  const int kb0 = blockIdx.y * kps, n = min(kb0 + kps, nk) - kb0;  // this workgroup's steps (>= 1)
  const size_t rowb = static_cast<size_t>(K) * 2;

  // 1 KB block b of a stage = rows 8 b .. 8 b + 7, 128 bytes each; lane l
  // carries row 8 b + (l >> 3), chunk (l & 7) ^ (l >> 3) (rows past M read zeros)
  const int q8 = lane >> 3, st_c = (lane & 7) ^ q8;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, static_cast<uint32_t>(static_cast<size_t>(M) * rowb));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + static_cast<size_t>(brow0) * K, static_cast<uint32_t>(kSkinnyN * rowb));
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(B, 0u);
  uint32_t a_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_off[i] = static_cast<uint32_t>((8 * (wave + 8 * i) + q8) * rowb) + 16u * st_c;
  const uint32_t b_off = static_cast<uint32_t>((8 * wave + q8) * rowb) + 16u * st_c;
  // The workgroups of one K range all read the same activation rows; each
  // starts at its own step (rotation by its weight tile) so that they do not
  // request the same lines at the same time.  The summation order then
  // depends on the tile only.
  const int rot = blockIdx.x % n;
  auto issue = [&](int s) {
    uint8_t* st = ring + (s % kSkinnyStages) * kStage;
    const bool live = s < n;
    const int sr = s + rot < n ? s + rot : s + rot - n;
    const int soff = (kb0 + sr) * 128;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(live ? ra : rz, st + 1024 * (wv + 8 * i), a_off[i], soff);
    dma16(live ? rb : rz, st + kABytes + 1024 * wv, b_off, soff);
  };

  // this lane's operand pieces within a 16-row block (2 KB): row l16, chunk
  // g (first MFMA of the step) and chunk 4 + g (second)
  const int fr = 1024 * (l16 >> 3) + 128 * (l16 & 7);
  const int f_lo = fr + 16 * (g ^ (l16 & 7));
  const int f_hi = fr + 16 * ((4 | g) ^ (l16 & 7));

  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Step s: wait for stage s (every wave's loads), start stage s + 5 into the
  // buffer of stage s - 1, compute stage s.
#pragma unroll
  for (int s = 0; s < kSkinnyStages - 1; ++s) issue(s);
  for (int s = 0; s < n; ++s) {
    ring_barrier<kLoads * (kSkinnyStages - 2)>();
    issue(s + kSkinnyStages - 1);
    // unconditional (a wave past M multiplies zero rows): a branch here makes
    // the compiler copy the accumulators between register files every step
    const uint8_t* st = ring + (s % kSkinnyStages) * kStage;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int fo = h ? f_hi : f_lo;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + 2048 * wave + fo);
      bf16x8 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8*>(st + kABytes + 2048 * j + fo);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = mfma_bf16(a, b[j], acc[j]);
    }
  }
  ring_barrier<0>();  // the trailing (empty) loads

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 16 * wave + 4 * g + i;
    if (row < M) {
      float* pr = partial + (static_cast<size_t>(blockIdx.y) * M + row) * nbrows + brow0 + l16;
#pragma unroll
      for (int j = 0; j < 4; ++j) pr[16 * j] = acc[j][i];
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
