// The whole forward of a decode-sized tail (at most 128 routed and 128
// shared tokens) in one persistent launch.
//
// The pages' producer schedules the routed experts and the BF16 shared
// expert's L1/L2 together in one kernel with the routed RMSNorm (DeepGEMM PR
// 416 mirror, Summary; "[Kimi K3][Kernel] Fuse BF16 shared experts into latent
// MegaMoE tail", Summary).  Here one workgroup per CU runs the tail's stages
// as a fixed sequence of segments, each the device body of the stage's own
// kernel (same tiles, same summation orders, so the same bits as the
// multi-launch path):
//
//   S1   shared L1 split-K products        (no dependency)
//   L1   routed L1 + SwiGLU + h codes      (x codes: the launch before)
//   S1R  shared L1 reduction -> hs         (after every S1)
//   L2   routed L2 -> y                    (after every L1)
//   S2   shared L2 split-K products        (after every S1R)
//   CMB  top-k combine + RMSNorm -> rn     (after every L2)
//   UP   up-projection split-K products    (after every CMB)
//   FIN  s, out = bf16(up + s [+ residual]), shared_out   (after every UP)
//
// Each segment ends with the workgroup's stores complete and a release
// increment of the segment's counter (which writes this XCD's L2 back); a
// segment that needs an earlier one waits (one lane, bounded) until that
// counter reaches the grid size, then acquires (invalidating this CU's stale
// lines).  Independent work sits between a segment and its consumer (S1R
// between L1 and L2, S2 between L2 and CMB), and the weights of a
// workgroup's first S2 and UP item start loading before it waits for their
// activations.  The counters are cleared by the launch before (the x
// quantizer).
//
// Every workgroup must be resident at once (the waits are on all of them):
// the grid is at most one workgroup per CU and the kernel's LDS allows no
// second.  A wait that does not end within its poll limit sets the error
// word and goes on, so every wave always exits; the launch then fails
// closed: the last workgroup to finish (a completion count after the final
// stage) finds the error word set and overwrites out and shared_out with
// NaN, and the word stays set for the host to read.
#pragma once

#include "common.hpp"
#include "dense_gemm.hpp"
#include "quant_norm.hpp"
#include "tile_gemm.hpp"

namespace moe_tail {

enum { SEG_S1 = 0, SEG_L1, SEG_S1R, SEG_L2, SEG_S2, SEG_CMB, SEG_UP, SEG_FIN, kSegs };
constexpr int kSyncWords = 16;  // segment counters + error word (cleared before the launch)
constexpr int kSyncErr = 15;    // 0: every wait ended; 1: a wait gave up (outputs are NaN)
constexpr int kSpinLimit = 1 << 20;
constexpr uint16_t kBf16NaN = 0x7FC0;

struct DenseItems {
  int nt, splits, kps;  // weight-row blocks, K splits, K steps per split
};

struct FusedArgs {
  TileArgs l1, l2;                   // routed L1 / L2 (32-row tiles)
  const uint16_t* x_hid;             // [Ms, H]
  const uint16_t* ws1;               // [2 I_s, H]
  const uint16_t* ws2;               // [H, I_s]
  const uint16_t* w_up;              // [H, L]
  int Mr, Ms, H, Is, L, k;
  DenseItems s1, s2, up;
  float* part_s1;                    // [s1.splits, Ms, 2 I_s]   (reused by UP)
  float* part_s2;                    // [s2.splits, Ms, H]
  float* part_up;                    // [up.splits, Mr, H]
  uint16_t* hs;                      // [Ms, I_s]
  const float* y;                    // [Mr k, L]
  const float* topk_w;               // [Mr, k]
  const int32_t* pair_to_row;        // [Mr k]
  const uint16_t* gamma;             // [L]
  uint16_t* rn;                      // [Mr, L]
  float eps;
  uint16_t* out;                     // [Mr, H]
  uint16_t* s;                       // [Mr, H] (the shared output of the routed tokens)
  uint16_t* shared_out;              // [Ms - Mr, H] or null
  const uint16_t* resid;             // [Mr, H] or null
  int* sync;                         // kSyncWords words, zero at launch
  int max_polls;                     // polls of a stage wait before it gives up (0: give up at once)
};

template <int FMT>
constexpr int fused_lds() {
  constexpr int a = TileLds<TK_L1, FMT, 32>::kBytes, b = TileLds<TK_L2, FMT, 32>::kBytes, c = dense_small_lds<>();
  constexpr int ab = a > b ? a : b;
  return ab > c ? ab : c;
}

// The end of a segment: this workgroup's stores have completed (every wave
// waits for its own), then one release increment (which writes this XCD's
// L2 back, so the other XCDs see the data).
__device__ __forceinline__ void seg_done(int* ctr) {
  vm_wait<0>();
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until `target` workgroups have finished the segment of `ctr`; the
// acquire then invalidates this CU's stale lines before any wave reads.
// After max_polls polls (at once for max_polls == 0) the wait gives up and
// sets the error word.
__device__ __forceinline__ void seg_wait(const int* ctr, int target, int* err, int max_polls) {
  if (threadIdx.x == 0) {
    int n = 0;
    for (;;) {
      if (n == max_polls) {
        __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) break;
      ++n;
      __builtin_amdgcn_s_sleep(4);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
}

// The end of the launch: every workgroup counts itself out after its final
// stores; the last one (which sees every other workgroup's count) reads the
// error word and, if a wait gave up anywhere, overwrites out and shared_out
// with NaN, so that a result of an incomplete hand-off is never returned as
// numbers.
__device__ __forceinline__ void fused_fail_closed(const FusedArgs& f, int nwg, int* s_flag) {
  vm_wait<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int before = __hip_atomic_fetch_add(f.sync + SEG_FIN, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    int poison = 0;
    if (before == nwg - 1) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      poison = __hip_atomic_load(f.sync + kSyncErr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
    }
    *s_flag = poison;
  }
  __syncthreads();
  if (*s_flag == 0) return;
  const size_t n_out = static_cast<size_t>(f.Mr) * f.H, n_so = static_cast<size_t>(f.Ms - f.Mr) * f.H;
  for (size_t i = threadIdx.x; i < n_out; i += blockDim.x) f.out[i] = kBf16NaN;
  if (f.shared_out != nullptr)
    for (size_t i = threadIdx.x; i < n_so; i += blockDim.x) f.shared_out[i] = kBf16NaN;
}

template <int NC4>
__device__ __forceinline__ void fused_combine(const FusedArgs& f, float* s_part, int wg, int nwg) {
  const int tid = threadIdx.x, half = tid >> 8;
  int it = 0;
  // two tokens per workgroup and pass (one per 256 threads); the halves'
  // 4-word partial sums alternate between two buffers by pass, so a pass's
  // writes never meet the previous pass's reads (one barrier per pass)
  for (int t0 = 2 * wg; t0 < f.Mr; t0 += 2 * nwg, ++it) {
    const int t = t0 + half;
    combine_token<NC4>(f.y, f.topk_w, f.pair_to_row, f.gamma, f.rn, f.L, f.k, f.eps, t < f.Mr ? t : -1, tid & 255,
                       s_part + 8 * (it & 1) + 4 * half);
  }
}

// FIN: group idx (four columns) of [Ms, H]: s = bf16 of the shared L2's
// partials summed in split order; rows < Mr: s and out = bf16(up + s
// [+ residual]) with the up-projection's partials summed in split order;
// rows >= Mr: shared_out.
__device__ __forceinline__ void fused_final_group(const FusedArgs& f, long idx) {
  const int N = f.H;
  const int row = static_cast<int>(idx / (N / 4)), col = 4 * static_cast<int>(idx % (N / 4));
  const float4 s4 = sum_splits(f.part_s2 + static_cast<size_t>(row) * N + col, static_cast<size_t>(f.Ms) * N,
                               f.s2.splits);
  const uint16_t b0 = static_cast<uint16_t>(f32_to_bf16_bits(s4.x)), b1 = static_cast<uint16_t>(f32_to_bf16_bits(s4.y));
  const uint16_t b2 = static_cast<uint16_t>(f32_to_bf16_bits(s4.z)), b3 = static_cast<uint16_t>(f32_to_bf16_bits(s4.w));
  if (row >= f.Mr) {
    uint16_t* so = f.shared_out + static_cast<size_t>(row - f.Mr) * N + col;
    so[0] = b0;
    so[1] = b1;
    so[2] = b2;
    so[3] = b3;
    return;
  }
  const float4 v = sum_splits(f.part_up + static_cast<size_t>(row) * N + col, static_cast<size_t>(f.Mr) * N,
                              f.up.splits);
  const size_t o = static_cast<size_t>(row) * N + col;
  f.s[o + 0] = b0;
  f.s[o + 1] = b1;
  f.s[o + 2] = b2;
  f.s[o + 3] = b3;
  f.out[o + 0] = up_join(v.x, b0, f.resid, o + 0);
  f.out[o + 1] = up_join(v.y, b1, f.resid, o + 1);
  f.out[o + 2] = up_join(v.z, b2, f.resid, o + 2);
  f.out[o + 3] = up_join(v.w, b3, f.resid, o + 3);
}

// The dense split-K items i = wg, wg + nwg, ... of one segment; the first
// item's weights start loading before the wait for the segment's
// activations (dep: null for none), which the weights do not depend on.
__device__ __forceinline__ void fused_dense_items(const uint16_t* A, const uint16_t* B, int M, int nbrows, int K,
                                                  const DenseItems& it, float* part, uint8_t* smem, int wg, int nwg,
                                                  const int* dep, int* err, int max_polls) {
  const int n = it.nt * it.splits;
  if (dep != nullptr) {
    if (wg < n)
      dense_small_run<kSkinnyBStages, kSkinnyAStages, 1>(A, B, M, nbrows, K, it.kps, part, smem, wg % it.nt,
                                                         wg / it.nt);
    seg_wait(dep, nwg, err, max_polls);
  }
  for (int i = wg; i < n; i += nwg) {
    if (dep != nullptr && i == wg)
      dense_small_run<kSkinnyBStages, kSkinnyAStages, 2>(A, B, M, nbrows, K, it.kps, part, smem, i % it.nt,
                                                         i / it.nt);
    else
      dense_small_run<>(A, B, M, nbrows, K, it.kps, part, smem, i % it.nt, i / it.nt);
    lds_barrier();  // the next item's loads reuse the ring
  }
}

template <int FMT>
__global__ __launch_bounds__(512) void k_tail_small(FusedArgs f) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[fused_lds<FMT>()];
  __shared__ int s_flag;
  const int wg = blockIdx.x, nwg = gridDim.x, tid = threadIdx.x;
  int* err = f.sync + kSyncErr;
  const int mp = f.max_polls;

  // S1: shared L1 split-K items (weight block, K split)
  fused_dense_items(f.x_hid, f.ws1, f.Ms, 2 * f.Is, f.H, f.s1, f.part_s1, smem, wg, nwg, nullptr, err, mp);
  seg_done(f.sync + SEG_S1);

  // L1: routed L1 tiles (x codes quantized by the launch before)
  tile_run<TK_L1, FMT, 0, 32>(f.l1, tile_smem_in<TK_L1, FMT, 32>(smem), wg, nwg);
  seg_done(f.sync + SEG_L1);

  // S1R: hs = bf16(silu(gate) * up) from the S1 partials
  seg_wait(f.sync + SEG_S1, nwg, err, mp);
  {
    const DenseEpi ep{f.Mr, f.Is, f.hs, nullptr, nullptr, nullptr};
    const long n = static_cast<long>(f.Ms) * (f.Is / 4);
    for (long idx = static_cast<long>(wg) * 512 + tid; idx < n; idx += static_cast<long>(nwg) * 512)
      dense_reduce_group<EPI_SWIGLU>(f.part_s1, f.Ms, f.Is, f.s1.splits, ep, idx);
  }
  seg_done(f.sync + SEG_S1R);

  // L2: routed L2 tiles -> y
  seg_wait(f.sync + SEG_L1, nwg, err, mp);
  tile_run<TK_L2, FMT, 0, 32>(f.l2, tile_smem_in<TK_L2, FMT, 32>(smem), wg, nwg);
  seg_done(f.sync + SEG_L2);

  // S2: shared L2 split-K items, after every S1R
  fused_dense_items(f.hs, f.ws2, f.Ms, f.H, f.Is, f.s2, f.part_s2, smem, wg, nwg, f.sync + SEG_S1R, err, mp);
  seg_done(f.sync + SEG_S2);

  // CMB: top-k combine + RMSNorm -> rn
  seg_wait(f.sync + SEG_L2, nwg, err, mp);
  {
    float* s_part = reinterpret_cast<float*>(smem);
    const int nc4 = (f.L / 4 + 255) / 256;
    if (nc4 <= 2) fused_combine<2>(f, s_part, wg, nwg);
    else if (nc4 <= 4) fused_combine<4>(f, s_part, wg, nwg);
    else fused_combine<8>(f, s_part, wg, nwg);
  }
  seg_done(f.sync + SEG_CMB);

  // UP: up-projection split-K items (S1's partials are consumed: reuse
  // them), after every CMB
  fused_dense_items(f.rn, f.w_up, f.Mr, f.H, f.L, f.up, f.part_up, smem, wg, nwg, f.sync + SEG_CMB, err, mp);
  seg_done(f.sync + SEG_UP);

  // FIN (every workgroup finished S2 before it started UP)
  seg_wait(f.sync + SEG_UP, nwg, err, mp);
  {
    const long n = static_cast<long>(f.Ms) * (f.H / 4);
    for (long idx = static_cast<long>(wg) * 512 + tid; idx < n; idx += static_cast<long>(nwg) * 512)
      fused_final_group(f, idx);
  }
  fused_fail_closed(f, nwg, &s_flag);
}

// ----------------------------------------------------------------------
// The decode-sized forward as six launches with independent work sharing a
// launch (kernel boundaries are the only synchronization):
//   x quantizer (clears the ticket counter) | routed L1 | routed L2 + shared
//   L1 items | combine + RMSNorm + shared L1 reduction | shared L2 items +
//   up-projection items | final join
// Routed L2 gives 896 tiles to 256 workgroups at decode, so half of them
// have a tile less; they take the shared L1's split-K items by ticket
// (device-scope atomic counter) after their own tiles, filling that gap.
// Each item computes what the shared L1's own launch would, so the bits do
// not change.

// words of the counters region used by this plan
constexpr int kTicketS1 = 0;

template <int FMT>
constexpr int l2_s1_lds() {
  constexpr int a = TileLds<TK_L2, FMT, 32>::kBytes, c = dense_small_lds<>();
  return a > c ? a : c;
}

// routed L2 tiles (static, as the routed L2 launch deals them), then shared
// L1 split-K items by ticket
template <int FMT>
__global__ __launch_bounds__(512) void k_l2_shared1(FusedArgs f) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[l2_s1_lds<FMT>()];
  __shared__ int s_item;
  tile_run<TK_L2, FMT, 0, 32>(f.l2, tile_smem_in<TK_L2, FMT, 32>(smem), blockIdx.x, gridDim.x);
  __syncthreads();
  const int n = f.s1.nt * f.s1.splits;
  for (;;) {
    if (threadIdx.x == 0)
      s_item = __hip_atomic_fetch_add(f.sync + kTicketS1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int i = s_item;
    if (i >= n) break;
    dense_small_run<>(f.x_hid, f.ws1, f.Ms, 2 * f.Is, f.H, f.s1.kps, f.part_s1, smem, i % f.s1.nt, i / f.s1.nt);
    __syncthreads();  // the ring and s_item are reused
  }
}

// blocks [0, Mr): combine + RMSNorm of token b; the others: shared L1
// reduction groups (256 per block) -> hs
template <int NC4>
__global__ __launch_bounds__(256) void k_combine_shared1r(FusedArgs f) {
  __shared__ float s_part[4];
  const int b = blockIdx.x;
  if (b < f.Mr) {
    combine_token<NC4>(f.y, f.topk_w, f.pair_to_row, f.gamma, f.rn, f.L, f.k, f.eps, b, threadIdx.x, s_part);
    return;
  }
  const DenseEpi ep{f.Mr, f.Is, f.hs, nullptr, nullptr, nullptr};
  const long idx = static_cast<long>(b - f.Mr) * 256 + threadIdx.x;
  if (idx < static_cast<long>(f.Ms) * (f.Is / 4)) dense_reduce_group<EPI_SWIGLU>(f.part_s1, f.Ms, f.Is, f.s1.splits, ep, idx);
}

// blocks [0, n2): shared L2 split-K items; the others: up-projection items
__global__ __launch_bounds__(512) void k_shared2_up(FusedArgs f) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[dense_small_lds<>()];
  const int n2 = f.s2.nt * f.s2.splits;
  const int b = blockIdx.x;
  if (b < n2) {
    dense_small_run<>(f.hs, f.ws2, f.Ms, f.H, f.Is, f.s2.kps, f.part_s2, smem, b % f.s2.nt, b / f.s2.nt);
  } else {
    const int u = b - n2;
    dense_small_run<>(f.rn, f.w_up, f.Mr, f.H, f.L, f.up.kps, f.part_up, smem, u % f.up.nt, u / f.up.nt);
  }
}

// s, out = bf16(up + s [+ residual]) and shared_out, one thread per four
// columns
__global__ __launch_bounds__(256) void k_final_join(FusedArgs f) {
  const long idx = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (idx < static_cast<long>(f.Ms) * (f.H / 4)) fused_final_group(f, idx);
}

}  // namespace moe_tail
