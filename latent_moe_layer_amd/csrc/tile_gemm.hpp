// LDS-tiled MFMA GEMM for large row counts (prefill): the routed experts'
// L1 / L2 (FP8 or FP8 x MXFP4, block-scaled) and the dense BF16 GEMMs of the
// shared expert and the up-projection.
//
// Tile: kTM = 128 rows x kTN = 256 B rows, one 128-byte K step per stage (128
// FP8 / FP4 elements or 64 BF16 elements), 8 waves as 2 (M) x 4 (N), each
// wave 64 rows x 64 B rows = 4 x 4 MFMA tiles of 16 x 16 (64 accumulator
// registers, which leaves room for the FP32 promotion without spilling).  Both operands are
// staged in LDS, double-buffered, in "fragment order": a 16-row block of one
// K step is stored as [half][lane][16 bytes], so that lane l's two 16-byte
// halves of its MFMA operand sit at lane * 16 -- every LDS read is a
// contiguous, conflict-free 1 KB per wave.  (8-bit operand: lane group g
// holds K [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of the step; BF16 at
// 64 elements per step: the same bytes are two 16x16x32 MFMAs; FP4: one
// 16-byte chunk per lane, K [32g, 32g + 32).)
//
// FP8 / FP4 block scales are applied once per MFMA result in FP32 (one MFMA
// covers one 128-wide scale block): acc += P * (s_act[row] * s_w[block]).
//
// Tiles are numbered m-slot major, n fastest, and the workgroup index is
// remapped so that each of the 8 XCDs (workgroups are dealt round-robin to
// them) runs a contiguous range of tiles: neighbouring n tiles share the A
// rows and neighbouring m tiles of an expert share the weights in that XCD's
// L2.
#pragma once

#include "common.hpp"
#include "dense_gemm.hpp"
#include "routed_gemm.hpp"

namespace moe_tail {

constexpr int kTM = 128;
constexpr int kTN = 256;
constexpr int kBigMinRows = 128;  // experts with at least this many rows use the tiled kernel

enum { TK_L1 = 0, TK_L2 = 1, TK_DENSE = 2 };
enum { TF_FP8 = 0, TF_FP4 = 1, TF_BF16 = 2 };

struct TileArgs {
  const uint8_t* a;               // L1: xq [Mr, L]; L2: hq [R, I]; dense: bf16 rows [M, K]
  const float* a_scale;           // L1: sx [Mr, L/128]; L2: sh [R, I/128]
  const int32_t* sorted_pair;     // L1: row -> token * k + slot
  const int32_t* expert_offsets;  // routed
  const uint8_t* b;               // weights (bytes)
  const void* b_scale;            // FP8: [E, N/128, K/128] f32; FP4: [E, N, K/32] e8m0
  uint8_t* hq;                    // L1 out
  float* sh;                      // L1 out
  float* y;                       // L2 out [R, L]
  DenseEpi ep;                    // dense epilogue
  int E, k;                       // routed
  int M;                          // dense rows
  int K;                          // reduction length (elements)
  int N;                          // B rows per expert (routed) or output columns (dense)
  int half;                       // L1: I (up rows start), dense SWIGLU: I_s
  int ntn;                        // n tiles
  int nslots;                     // m slots in the grid
};

// Row tiles of experts with >= kBigMinRows rows, kTM rows each (last one partial).
__device__ __forceinline__ bool find_big_tile(const int32_t* __restrict__ off, int E, int mt, int& e_out,
                                              int& row0_out, int& rows_out) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) / 64;
  const int eb = min(lane * per, E), ee = min(eb + per, E);
  auto ntile = [&](int e) {
    const int c = off[e + 1] - off[e];
    return c >= kBigMinRows ? (c + kTM - 1) / kTM : 0;
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
  int fe = -1, fr0 = 0, frows = 0;
  if (mt >= excl && mt < incl) {
    int acc = excl;
    for (int e = eb; e < ee; ++e) {
      const int n = ntile(e);
      if (mt < acc + n) {
        fe = e;
        fr0 = off[e] + (mt - acc) * kTM;
        frows = min(kTM, off[e + 1] - fr0);
        break;
      }
      acc += n;
    }
  }
  const unsigned long long who = __ballot(fe >= 0);
  const int src = __ffsll(static_cast<long long>(who)) - 1;
  e_out = __shfl(fe, src);
  row0_out = __shfl(fr0, src);
  rows_out = __shfl(frows, src);
  return true;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS loads: lane l's 16 (or 4) bytes land at lds + 16 l
// (4 l); an offset outside the resource's range writes zeros.  `lds` must be
// the same for the whole wave.  Issued as inline assembly so that the
// compiler does not track them: it cannot always tell which LDS reads they
// may overlap and would then wait for every one in flight; ring_barrier
// below does the waiting instead.  (No memory clobber: volatile asm keeps
// its order against ring_barrier, and the compiler may move LDS reads of
// other stages around these.)
__device__ __forceinline__ uint32_t lds_offset(const uint8_t* lds) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t*)lds)));
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const uint8_t* lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_offset(lds)), "v"(voff), "s"(r),
               "s"(soff));
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, const uint8_t* lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds_offset(lds)), "v"(voff), "s"(r),
               "s"(soff));
}

// Wait until at most N of this wave's direct loads are in flight and its LDS
// reads are done, then meet the other waves: afterwards every load issued
// before the newest N (by any wave) has landed.  (A fenced __syncthreads
// would wait for all of them.)
template <int N>
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int KIND, int FMT, int EPI>
__global__ __launch_bounds__(512) void k_tile(TileArgs p) {
  constexpr bool kFP4 = FMT == TF_FP4;
  constexpr bool kBF16 = FMT == TF_BF16;
  constexpr bool kScaled = !kBF16;
  constexpr int kABytes = kTM * 128;                 // 16 KB
  constexpr int kBBytes = kTN * (kFP4 ? 64 : 128);   // 16 or 32 KB
  constexpr int kSOff = kABytes + kBBytes;           // scale words: activation [0, 512), FP4 e8m0 [512, 1536)
  constexpr int kStage = kSOff + (kScaled ? 2048 : 0);
  constexpr int kBChunks = kFP4 ? 2 : 4;             // 16-byte B loads per thread and stage
  constexpr int kLoads = 2 + kBChunks + (kScaled ? 1 : 0);  // direct loads per wave and stage
  // three-stage ring, one array per stage so that the compiler can tell the
  // stages apart (its own waits before LDS reads then cover just that stage)
  __shared__ __attribute__((aligned(16))) uint8_t ring0[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[kStage];
  __shared__ __attribute__((aligned(16))) uint8_t ring2[kStage];
  __shared__ int s_tile[3];
  __shared__ int s_tok[kTM];
  __shared__ float s_amax[4][kTM];
  __shared__ float s_wsc[2][kMaxKBlocks];  // FP8 weight scales of the tile's two 128-row B blocks

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int l16 = lane & 15, g = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(wave);

  // workgroup -> tile, contiguous tile ranges per XCD
  const int T = p.nslots * p.ntn;
  const int b = blockIdx.x;
  const int full = T - T % 8;
  const int t = (b < full) ? (b % 8) * (full / 8) + b / 8 : b;
  const int slot = t / p.ntn, nt = t % p.ntn;

  int e = 0, row0 = 0, rows = 0;
  if (KIND == TK_DENSE) {
    row0 = slot * kTM;
    rows = min(kTM, p.M - row0);
  } else {
    if (wave == 0) {
      int fe, fr, fn;
      const bool ok = find_big_tile(p.expert_offsets, p.E, slot, fe, fr, fn);
      if (lane == 0) {
        s_tile[0] = ok ? fe : -1;
        s_tile[1] = fr;
        s_tile[2] = fn;
      }
    }
    __syncthreads();
    e = __builtin_amdgcn_readfirstlane(s_tile[0]);
    if (e < 0) return;  // uniform
    row0 = __builtin_amdgcn_readfirstlane(s_tile[1]);
    rows = __builtin_amdgcn_readfirstlane(s_tile[2]);
  }
  const int nk = kBF16 ? p.K / 64 : p.K / 128;    // K steps of 128 bytes
  const int nkb = p.K / 128;                       // scale blocks along K (scaled formats)
  const int elem = kBF16 ? 2 : 1;                  // bytes per A element
  constexpr bool kPaired = KIND == TK_L1 || (KIND == TK_DENSE && EPI == EPI_SWIGLU);
  const int nbrows = kPaired ? 2 * p.half : p.N;  // B rows of one expert / of the dense matrix
  // B row j of the tile (0..255) -> weight row: paired kinds take 128 gate
  // rows and the matching 128 up rows, the others 256 consecutive rows
  auto wrow = [&](int j) -> int {
    if (kPaired) return (j < 128) ? 128 * nt + j : p.half + 128 * nt + (j - 128);
    return kTN * nt + j;
  };

  if (KIND == TK_L1 && tid < kTM) s_tok[tid] = (tid < rows) ? p.sorted_pair[row0 + tid] / p.k : -1;
  // FP8 weight scales [E, N/128, K/128] of tile rows [0, 128) and [128, 256)
  // for every K step, read once here
  if (FMT == TF_FP8 && tid < 2 * nkb) {
    const int q = tid / nkb, kb = tid - q * nkb;
    const int wr = wrow(128 * q);
    s_wsc[q][kb] = (wr < nbrows) ? static_cast<const float*>(p.b_scale)[(static_cast<size_t>(e) * (nbrows / 128) + wr / 128) * nkb + kb]
                                 : 0.0f;
  }
  __syncthreads();

  // ---- per-thread load assignment ----
  // Thread t fills the 16-byte LDS slots t + 512 i of an operand, so every
  // wave's load writes one contiguous kilobyte.  Slot s is 16-row block
  // s / 128 (FP4 B: s / 64), half h = (s / 64) % 2, lane' = s % 64 = 16 g + r:
  // tile row 16 * block + r, 16-byte chunk c = 4 h + g (FP4: g).  This is the
  // MFMA operand ("fragment") order, so each lane later reads its operand at
  // lane * 16 of a block's half.
  const int t_r = tid & 15, t_g = (tid >> 4) & 3, t_h = (tid >> 6) & 1;
  const int st_c = 4 * t_h + t_g;                       // chunk of an 8-bit / BF16 row step
  const int st_r0 = 16 * (tid >> 7) + t_r;              // rows st_r0 + 64 i
  // A operand: rows st_r0 + 64 i, i < 2; out-of-range rows read as zero
  // (offset past the buffer's end).
  constexpr uint32_t kNoRow = 0x80000000u;
  const size_t a_row_bytes = static_cast<size_t>(p.K) * elem;
  uint32_t a_off[2];
  const uint8_t* a_base;
  uint32_t a_records;
  if (KIND == TK_L1) {
    a_base = p.a;                                       // gathered token rows of x codes
    a_records = static_cast<uint32_t>(static_cast<size_t>(p.M) * a_row_bytes);
  } else {
    a_base = p.a + static_cast<size_t>(row0) * a_row_bytes;
    a_records = static_cast<uint32_t>(static_cast<size_t>(rows) * a_row_bytes);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = st_r0 + 64 * i;
    uint32_t o = kNoRow;
    if (row < rows) {
      const size_t rr = (KIND == TK_L1) ? static_cast<size_t>(s_tok[row]) : static_cast<size_t>(row);
      o = static_cast<uint32_t>(rr * a_row_bytes) + 16u * st_c;
    }
    a_off[i] = o;
  }
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a_base), static_cast<short>(0), a_records, 0x00020000);
  // B operand: the tile's 256 B rows map to weight rows wrow(j)
  const size_t brow_bytes = kFP4 ? static_cast<size_t>(p.K) / 2 : static_cast<size_t>(p.K) * elem;
  uint32_t b_off[kBChunks];
#pragma unroll
  for (int i = 0; i < kBChunks; ++i) {
    const int row = kFP4 ? 128 * i + 16 * (tid >> 6) + t_r : st_r0 + 64 * i;
    const int c = kFP4 ? t_g : st_c;
    b_off[i] = static_cast<uint32_t>(static_cast<size_t>(wrow(row)) * brow_bytes) + 16u * c;
  }
  const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.b + static_cast<size_t>(e) * nbrows * brow_bytes), static_cast<short>(0),
      static_cast<uint32_t>(static_cast<size_t>(nbrows) * brow_bytes), 0x00020000);
  // a resource with no valid bytes: loads through it write zeros
  const __amdgpu_buffer_rsrc_t z_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b), static_cast<short>(0), 0u, 0x00020000);
  // scale words, one 4-byte load per lane and stage: waves 0-1 the
  // activation scales of tile rows 64 w + lane, waves 2-5 (FP4) the e8m0
  // words of B rows 64 (w - 2) + lane; the other waves load zeros
  __amdgpu_buffer_rsrc_t s_rsrc = z_rsrc;
  uint32_t s_off = kNoRow;
  if (kScaled) {
    if (wv < 2) {
      const int row = 64 * wv + lane;
      const float* sbase = (KIND == TK_L1) ? p.a_scale : p.a_scale + static_cast<size_t>(row0) * nkb;
      const size_t srows = (KIND == TK_L1) ? static_cast<size_t>(p.M) : static_cast<size_t>(rows);
      s_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sbase), static_cast<short>(0),
                                                 static_cast<uint32_t>(srows * nkb * 4), 0x00020000);
      if (row < rows) {
        const size_t ar = (KIND == TK_L1) ? static_cast<size_t>(s_tok[row]) : static_cast<size_t>(row);
        s_off = static_cast<uint32_t>(ar * nkb * 4);
      }
    } else if (kFP4 && wv < 6) {
      const int j = 64 * (wv - 2) + lane;
      const size_t wpr = static_cast<size_t>(p.K) / 32;  // e8m0 bytes per weight row
      s_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(static_cast<const uint8_t*>(p.b_scale) + static_cast<size_t>(e) * nbrows * wpr),
          static_cast<short>(0), static_cast<uint32_t>(nbrows * wpr), 0x00020000);
      s_off = static_cast<uint32_t>(wrow(j) * wpr);
    }
  }

  // stage ks -> ring buffer; past the last stage the loads go through the
  // empty resource (no memory traffic) so that every stage counts kLoads
  auto issue = [&](uint8_t* ring, int ks) {
    const bool live = ks < nk;
    const __amdgpu_buffer_rsrc_t ra = live ? a_rsrc : z_rsrc;
    const __amdgpu_buffer_rsrc_t rb = live ? b_rsrc : z_rsrc;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(ra, ring + 8192 * i + 1024 * wv, a_off[i], ks * 128);
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) dma16(rb, ring + kABytes + 8192 * i + 1024 * wv, b_off[i], kFP4 ? ks * 64 : ks * 128);
    if (kScaled) dma4(live ? s_rsrc : z_rsrc, ring + kSOff + 256 * wv, s_off, 4 * ks);
  };

  // B blocks of this wave, j = 0..3 (paired: two gate blocks, then the two
  // matching up blocks)
  auto bblk = [&](int j) {
    if (kPaired) return (j < 2) ? 2 * wn + j : 8 + 2 * wn + (j - 2);
    return 4 * wn + j;
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint8_t* st, int ks) {
    // weight scales of this step (FP8): the wave's B rows lie in the tile's
    // row half 16 * bblk(0) / 128 (paired: its gate rows) and 16 * bblk(3) / 128
    float sw_lo = 1.0f, sw_hi = 1.0f;
    if (FMT == TF_FP8) {
      sw_lo = s_wsc[(16 * bblk(0)) / 128][ks];
      sw_hi = s_wsc[(16 * bblk(3)) / 128][ks];
    }
    i32x8 af[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const uint8_t* ab = st + (4 * wm + mt) * 2048 + lane * 16;
      const i32x4 lo = *reinterpret_cast<const i32x4*>(ab);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(ab + 1024);
      af[mt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // per-row promotion factors of this step: activation scale x weight scale
    float sc[2][4][4];
    if (kScaled) {
      const float* ss = reinterpret_cast<const float*>(st + kSOff);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(ss + 64 * wm + 16 * mt + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[0][mt][i] = v[i] * sw_lo;
          sc[1][mt][i] = v[i] * sw_hi;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bb = bblk(j);
      if (kBF16) {
        const uint8_t* bp = st + kABytes + bb * 2048 + lane * 16;
        const bf16x8 b0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(bp));
        const bf16x8 b1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(bp + 1024));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const i32x4 alo = __builtin_shufflevector(af[mt], af[mt], 0, 1, 2, 3);
          const i32x4 ahi = __builtin_shufflevector(af[mt], af[mt], 4, 5, 6, 7);
          acc[mt][j] = mfma_bf16(__builtin_bit_cast(bf16x8, alo), b0, acc[mt][j]);
          acc[mt][j] = mfma_bf16(__builtin_bit_cast(bf16x8, ahi), b1, acc[mt][j]);
        }
      } else {
        i32x8 bf;
        int sb = 127;
        if (kFP4) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(st + kABytes + bb * 1024 + lane * 16);
          const i32x4 z = {0, 0, 0, 0};
          bf = __builtin_shufflevector(v, z, 0, 1, 2, 3, 4, 5, 6, 7);
          sb = st[kSOff + 512 + (16 * bb + l16) * 4 + g];
        } else {
          const uint8_t* bp = st + kABytes + bb * 2048 + lane * 16;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(bp);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(bp + 1024);
          bf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        const int half_sel = (kPaired && j >= 2) ? 1 : 0;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const f32x4 pr = kFP4 ? mfma_fp8_fp4(af[mt], bf, sb) : mfma_fp8(af[mt], bf);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][j][i] += pr[i] * sc[half_sel][mt][i];
        }
      }
    }
  };

  // Pipeline: stage ks sits in ring ks % 3 while stages ks + 1 and ks + 2 are
  // in flight.  Each step: wait for stage ks (all waves), start stage ks + 2
  // into the buffer that stage ks - 1 (read by every wave before the
  // barrier) leaves free, then compute stage ks.
  issue(ring0, 0);
  issue(ring1, 1);
  for (int ks = 0; ks < nk; ks += 3) {
    ring_barrier<kLoads>();
    issue(ring2, ks + 2);
    compute(ring0, ks);
    if (ks + 1 < nk) {
      ring_barrier<kLoads>();
      issue(ring0, ks + 3);
      compute(ring1, ks + 1);
    }
    if (ks + 2 < nk) {
      ring_barrier<kLoads>();
      issue(ring1, ks + 4);
      compute(ring2, ks + 2);
    }
  }
  // drain the trailing (empty) loads before the epilogue reuses ring0
  ring_barrier<0>();

  // ---------------------------------------------------------------- epilogues
  if (KIND == TK_L1) {
    // h = silu(gate) * up for this wave's 64 rows x 32 h columns; row amax over the tile's 128 h columns
    float h[4][2][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          h[mt][j][i] = silu_mul(acc[mt][j][i], acc[mt][2 + j][i]);
          m = fmaxf(m, fabsf(h[mt][j][i]));
        }
        m = group16_max(m);
        if (l16 == 0) s_amax[wn][64 * wm + 16 * mt + 4 * g + i] = m;
      }
    __syncthreads();
    uint8_t* sq = ring0;  // [128 rows][128 codes], the ring is free now
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 64 * wm + 16 * mt + 4 * g + i;
        const float amax = fmaxf(fmaxf(s_amax[0][r], s_amax[1][r]), fmaxf(s_amax[2][r], s_amax[3][r]));
        const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
#pragma unroll
        for (int j = 0; j < 2; ++j) sq[r * 128 + 32 * wn + 16 * j + l16] = static_cast<uint8_t>(f32_to_e4m3(h[mt][j][i] / s));
        if (wn == 0 && l16 == 0 && r < rows) p.sh[static_cast<size_t>(row0 + r) * (p.half / 128) + nt] = s;
      }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 512 * i;
      const int r = q >> 3, c16 = (q & 7) * 16;
      if (r < rows)
        *reinterpret_cast<uint4*>(p.hq + static_cast<size_t>(row0 + r) * p.half + 128 * nt + c16) =
            *reinterpret_cast<const uint4*>(sq + r * 128 + c16);
    }
  } else if (KIND == TK_L2) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 64 * wm + 16 * mt + 4 * g + i;
        if (r < rows) {
          float* yr = p.y + static_cast<size_t>(row0 + r) * p.N + kTN * nt + 64 * wn + l16;
#pragma unroll
          for (int j = 0; j < 4; ++j) yr[16 * j] = acc[mt][j][i];
        }
      }
  } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 64 * wm + 16 * mt + 4 * g + i;
        if (r < rows) {
          if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int j = 0; j < 2; ++j)
              dense_epilogue<EPI>(p.ep, p.N, row0 + r, 128 * nt + 32 * wn + 16 * j + l16, acc[mt][j][i],
                                  acc[mt][2 + j][i]);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              dense_epilogue<EPI>(p.ep, p.N, row0 + r, kTN * nt + 64 * wn + 16 * j + l16, acc[mt][j][i], 0.0f);
          }
        }
      }
  }
}

}  // namespace moe_tail
