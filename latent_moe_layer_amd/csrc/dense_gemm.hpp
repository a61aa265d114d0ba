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
  const uint16_t* resid;  // UPADD: residual [M, N] bf16 added in FP32 after s, or null
  // UPADD, small M, Ms == Mr: s is formed here from the shared L2's split-K
  // partials (summed in split order and rounded to bf16, as the shared L2's
  // own reduction would) and stored to out1; addsrc is then unused
  const float* s_partial = nullptr;
  int s_splits = 0;
};

// The up-projection's output element: (acc + f32(s)) + f32(residual), one
// rounding to bf16.
__device__ __forceinline__ uint16_t up_join(float acc, uint16_t s_bits, const uint16_t* resid, size_t o) {
  float v = acc + bf16_bits_to_f32(s_bits);
  if (resid != nullptr) v += bf16_bits_to_f32(resid[o]);  // residual, same single rounding
  return static_cast<uint16_t>(f32_to_bf16_bits(v));
}

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
    const size_t o = static_cast<size_t>(row) * N + col;
    ep.out0[o] = up_join(v0, ep.addsrc[o], ep.resid, o);
  }
}

// ---------------------------------------------------------- small M --
// Decode-sized M (<= 128 rows): a workgroup covers every row and kSkinnyN
// weight rows over a range of K steps (K is split over gridDim.y), so each
// weight byte is read from HBM once.  Both operands go straight from memory
// into LDS (buffer loads with the LDS flag, whole 128-byte lines per load,
// rows XOR-swizzled as in the tiled kernel).  A CU's vector-memory path moves
// about 54 bytes per clock whether a load hits L2 or not, and every
// workgroup loads all activation rows of its K range, so the weight tile is
// as wide as the activation tile (128 rows): half of what a CU loads is
// weights.  Two rings: the weights, which come from HBM, through a deeper
// one (kBSt - 1 steps in flight), the activation rows, which the workgroups
// of a K range share and so mostly hit in L2, through a shallower one
// (kASt - 1 steps ahead).  A wave's load counter retires in issue order, so
// a wave waiting for activations would also wait for every weight load it
// issued before them: waves 0-3 load only weights and waves 4-7 only
// activations, each waiting for its own ring.  All 8 waves compute: wave w
// multiplies rows [32 (w & 3), +32) by weight rows [64 (w >> 2), +64).  FP32
// partial sums partial[z][row][brow] are reduced in split order by
// k_dense_reduce, which applies the epilogue.
constexpr int kSmallMaxM = 128;
constexpr int kSkinnyN = 128;        // weight rows per workgroup
constexpr int kSkinnyBStages = 4;    // weight ring depth
constexpr int kSkinnyAStages = 3;    // activation ring depth

template <int kBSt = kSkinnyBStages, int kASt = kSkinnyAStages>
constexpr int dense_small_lds() {
  return kBSt * kSkinnyN * 128 + kASt * kSmallMaxM * 128;
}

// One workgroup's item (weight rows [bx kSkinnyN, +kSkinnyN), K range by)
// with its LDS at smem.  kPart 1 issues only the weight ring's first stages
// and returns (the weights do not depend on earlier work, so a persistent
// kernel starts them before it waits for the activations); kPart 2 is the
// rest of such an item, kPart 0 a whole item.
template <int kBSt = kSkinnyBStages, int kASt = kSkinnyAStages, int kPart = 0>
__device__ __forceinline__ void dense_small_run(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int M,
                                                int nbrows, int K, int kps, float* __restrict__ partial, uint8_t* smem,
                                                int bx, int by) {
  static_assert(kASt >= 2 && kBSt >= kASt, "the weight ring runs ahead of the activation ring");
  constexpr int kABytes = kSmallMaxM * 128;  // one K step of 64 BF16: 128 rows x 128 bytes
  constexpr int kBBytes = kSkinnyN * 128;
  constexpr int kBLoads = kBBytes / 4096;  // per weight wave and step (1 KB each)
  constexpr int kALoads = kABytes / 4096;  // per activation wave and step
  uint8_t* ring_b = smem;
  uint8_t* ring_a = smem + kBSt * kBBytes;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const bool loads_b = wv < 4;
  const int lw = wv & 3;  // index among the waves of its role
  const int l16 = lane & 15, g = lane >> 4;
  const int wr = wave & 3, wc = wave >> 2;  // this wave's 32 rows and 64 weight rows
  const int brow0 = bx * kSkinnyN;
  const int nk = K / 64;
  const int kb0 = by * kps, n = min(kb0 + kps, nk) - kb0;  // this item's steps (>= 1)
  const size_t rowb = static_cast<size_t>(K) * 2;

  // 1 KB block b of a stage = rows 8 b .. 8 b + 7, 128 bytes each; lane l
  // carries row 8 b + (l >> 3), chunk (l & 7) ^ (l >> 3) (rows past M read
  // zeros).  A wave of a role loads blocks lw, lw + 4, lw + 8, lw + 12.
  const int q8 = lane >> 3, st_c = (lane & 7) ^ q8;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, static_cast<uint32_t>(static_cast<size_t>(M) * rowb));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + static_cast<size_t>(brow0) * K, static_cast<uint32_t>(kSkinnyN * rowb));
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(B, 0u);
  const __amdgpu_buffer_rsrc_t rl = loads_b ? rb : ra;
  // The workgroups of one K range all read the same activation rows; each
  // starts at its own step (rotation by its weight tile) so that they do not
  // request the same lines at the same time.  The summation order then
  // depends on the tile only.
  const int rot = bx % n;
  // stage s of this wave's ring into `slot`: blocks lw + 4 i
  auto issue = [&](int s, uint8_t* slot, int nl) {
    const int sr = s + rot < n ? s + rot : s + rot - n;
    const int soff = (kb0 + sr) * 128;
    for (int i = 0; i < nl; ++i) {
      const int blk = lw + 4 * i;
      dma16(s < n ? rl : rz, slot + 1024 * blk, static_cast<uint32_t>((8 * blk + q8) * rowb) + 16u * st_c, soff);
    }
  };
  auto issue_b = [&](int s) { issue(s, ring_b + (s % kBSt) * kBBytes, kBLoads); };
  auto issue_a = [&](int s) { issue(s, ring_a + (s % kASt) * kABytes, kALoads); };

  // this lane's operand pieces within a 16-row block (2 KB): row l16, chunk
  // g (first MFMA of the step) and chunk 4 + g (second)
  const int fr = 1024 * (l16 >> 3) + 128 * (l16 & 7);
  const int f_lo = fr + 16 * (g ^ (l16 & 7));
  const int f_hi = fr + 16 * ((4 | g) ^ (l16 & 7));

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Step s: wait for this wave's part of stage s, barrier (stage s complete,
  // every wave done with step s - 1), start stage s + kBSt - 1 (weights) or
  // s + kASt - 1 (activations) into the slot of step s - 1, compute step s.
  if (loads_b) {
    if (kPart != 2) {
#pragma unroll
      for (int s = 0; s < kBSt - 1; ++s) issue_b(s);
    }
  } else if (kPart != 1) {
#pragma unroll
    for (int s = 0; s < kASt - 1; ++s) issue_a(s);
  }
  if (kPart == 1) return;
  for (int s = 0; s < n; ++s) {
    if (loads_b) vm_wait<kBLoads * (kBSt - 2)>();
    else vm_wait<kALoads * (kASt - 2)>();
    lds_barrier();
    if (loads_b) issue_b(s + kBSt - 1);
    else issue_a(s + kASt - 1);
    // unconditional (a wave past M multiplies zero rows): a branch here makes
    // the compiler copy the accumulators between register files every step
    const uint8_t* sa = ring_a + (s % kASt) * kABytes + 4096 * wr;
    const uint8_t* sb = ring_b + (s % kBSt) * kBBytes + 8192 * wc;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int fo = h ? f_hi : f_lo;
      bf16x8 a[2], b[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const bf16x8*>(sa + 2048 * i + fo);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8*>(sb + 2048 * j + fo);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(a[i], b[j], acc[i][j]);
    }
  }
  vm_wait<0>();  // the trailing (empty) loads

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 32 * wr + 16 * i + 4 * g + e;
      if (row < M) {
        float* pr = partial + (static_cast<size_t>(by) * M + row) * nbrows + brow0 + 64 * wc + l16;
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[16 * j] = acc[i][j][e];
      }
    }
}

template <int kBSt = kSkinnyBStages, int kASt = kSkinnyAStages>
__global__ __launch_bounds__(512) void k_dense_small(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                     int M, int nbrows, int K, int kps, float* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[dense_small_lds<kBSt, kASt>()];
  dense_small_run<kBSt, kASt>(A, B, M, nbrows, K, kps, partial, smem, blockIdx.x, blockIdx.y);
}

// Sum over z < splits of the float4 at base + z * stride, added in z order;
// the loads of kChunk splits are issued before any is added (one memory
// latency per chunk instead of one per split).
template <int kChunk = 8>
__device__ __forceinline__ float4 sum_splits(const float* base, size_t stride, int splits) {
  float4 v = {0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < splits; z0 += kChunk) {
    float4 a[kChunk];
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (z0 + i < splits) a[i] = *reinterpret_cast<const float4*>(base + (z0 + i) * stride);
#pragma unroll
    for (int i = 0; i < kChunk; ++i)
      if (z0 + i < splits) {
        v.x += a[i].x;
        v.y += a[i].y;
        v.z += a[i].z;
        v.w += a[i].w;
      }
  }
  return v;
}

// Sums the split-K partials in split order and applies the epilogue to
// output group idx (four neighbouring columns) of M * ncols / 4 (ncols = I_s
// for SWIGLU, N otherwise).
template <int kEpi>
__device__ __forceinline__ void dense_reduce_group(const float* __restrict__ partial, int M, int N, int splits,
                                                   const DenseEpi& ep, long idx) {
  const int nraw = (kEpi == EPI_SWIGLU) ? 2 * ep.half : N;
  const int ncols = (kEpi == EPI_SWIGLU) ? ep.half : N;
  const int row = static_cast<int>(idx / (ncols / 4)), col = 4 * static_cast<int>(idx % (ncols / 4));
  const size_t zs = static_cast<size_t>(M) * nraw;  // split stride
  const float* pr = partial + static_cast<size_t>(row) * nraw + col;
  const float4 v0 = sum_splits(pr, zs, splits);
  float4 v1 = {0.f, 0.f, 0.f, 0.f};
  if (kEpi == EPI_SWIGLU) v1 = sum_splits(pr + ep.half, zs, splits);
  if (kEpi == EPI_UPADD && ep.s_partial != nullptr) {
    const float4 s4 = sum_splits(ep.s_partial + static_cast<size_t>(row) * N + col, static_cast<size_t>(M) * N,
                                 ep.s_splits);
    const size_t o = static_cast<size_t>(row) * N + col;
    const uint16_t s0 = static_cast<uint16_t>(f32_to_bf16_bits(s4.x)), s1 = static_cast<uint16_t>(f32_to_bf16_bits(s4.y));
    const uint16_t s2 = static_cast<uint16_t>(f32_to_bf16_bits(s4.z)), s3 = static_cast<uint16_t>(f32_to_bf16_bits(s4.w));
    ep.out1[o + 0] = s0;
    ep.out1[o + 1] = s1;
    ep.out1[o + 2] = s2;
    ep.out1[o + 3] = s3;
    ep.out0[o + 0] = up_join(v0.x, s0, ep.resid, o + 0);
    ep.out0[o + 1] = up_join(v0.y, s1, ep.resid, o + 1);
    ep.out0[o + 2] = up_join(v0.z, s2, ep.resid, o + 2);
    ep.out0[o + 3] = up_join(v0.w, s3, ep.resid, o + 3);
    return;
  }
  dense_epilogue<kEpi>(ep, N, row, col + 0, v0.x, v1.x);
  dense_epilogue<kEpi>(ep, N, row, col + 1, v0.y, v1.y);
  dense_epilogue<kEpi>(ep, N, row, col + 2, v0.z, v1.z);
  dense_epilogue<kEpi>(ep, N, row, col + 3, v0.w, v1.w);
}

template <int kEpi>
__global__ __launch_bounds__(256) void k_dense_reduce(const float* __restrict__ partial, int M, int N, int splits,
                                                      DenseEpi ep) {
  const int ncols = (kEpi == EPI_SWIGLU) ? ep.half : N;
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<long>(M) * (ncols / 4)) return;
  dense_reduce_group<kEpi>(partial, M, N, splits, ep, idx);
}

}  // namespace moe_tail
