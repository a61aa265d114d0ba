// LDS-tiled MFMA GEMM for large row counts (prefill): the routed experts'
// L1 / L2 (FP8 or FP8 x MXFP4, block-scaled) and the dense BF16 GEMMs of the
// shared expert and the up-projection.
//
// Tile: TM = 256, 128 or 32 rows x kTN = 256 B rows, one 128-byte K step per
// stage (128 FP8 / FP4 elements or 64 BF16 elements), 8 waves as 2 (M) x 4
// (N), each wave 128 or 64 rows x 64 B rows (8 or 4 x 4 MFMA tiles of
// 16 x 16), or for 32-row tiles 8 waves of 32 x 32.  Both operands go
// straight from memory to LDS (buffer loads with the LDS flag) into a ring of
// two (256 rows), three (128) or four (32) stages.  Every load fetches
// whole 128-byte lines; a row's 16-byte chunks are stored XOR-swizzled so
// that the MFMA operand reads are free of bank conflicts.  (8-bit operand:
// lane group g holds K [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16) of the
// step; BF16 at 64 elements per step: the same bytes are two 16x16x32 MFMAs;
// FP4: one 16-byte chunk per lane, K [32g, 32g + 32).)
//
// FP8 / FP4 block scales are applied once per MFMA result in FP32 (one MFMA
// covers one 128-wide scale block): acc += P * (s_act[row] * s_w[block]).
//
// Tiles are numbered m-slot major, n fastest; each of the 8 XCDs works
// through a contiguous run of them (see xcd_tile).
#pragma once

#include "common.hpp"
#include "dense_gemm.hpp"
#include "routed_gemm.hpp"

namespace moe_tail {

constexpr int kTM = 128;
constexpr int kTN = 256;
constexpr int kBigMinRows = 128;  // experts with at least this many rows use 128-row tiles (by default)
constexpr int kHugeTM = 256;      // ... and from this many rows on, 256-row tiles where they pay
constexpr int kMidTM = 64;        // experts between 32 and kBigMinRows rows, when the experts average over 32

// An expert with c >= huge rows takes 256-row tiles for its first c / 256 *
// 256 rows; a tail of more than 128 rows takes one more (partly padded)
// 256-row tile, a shorter tail one 128-row tile.  Switching whole experts
// to 128-row tiles measured slower at the prefill loads (routed L1 752
// against 699 us: a 128-row tile does half a 256-row tile's work per byte it
// moves); moving only the short tails measured about neutral in kernel time
// (621 us of 256-row tiles + 102 us of tails against 722 us).
__host__ __device__ __forceinline__ bool use256(int c, int huge) { return c >= huge; }
// Such an expert's rows past its last full 256-row tile: up to 128 of them
// go to one 128-row tile (a 256-row tile would be more than half padding),
// more stay in a last, partly padded 256-row tile.
__host__ __device__ __forceinline__ int tiles256(int c) { return c / 256 + ((c % 256) > 128 ? 1 : 0); }
__host__ __device__ __forceinline__ bool tail128(int c) { return (c % 256) > 0 && (c % 256) <= 128; }
constexpr int kTileMaxE = 512;    // expert tables of the routed kinds live in LDS

enum { TK_L1 = 0, TK_L2 = 1, TK_DENSE = 2 };
enum { TF_FP8 = 0, TF_FP4 = 1, TF_BF16 = 2, TF_NV4 = 3 };  // TF_NV4: NVFP4 weights (FP16 matrix cores)

// K halves (128-wide blocks) per stage.  An MXFP4 weight row holds 64 bytes
// per 128 K, and loads of half lines run at a fraction of the rate of whole
// ones (the 1024-token MXFP4 workload's routed L1 + L2: 460 + 238 us with
// half-line weight loads, 387 + 199 us in a timing-only variant that moved
// the same bytes as whole lines), so MXFP4 tiles take two K blocks (one
// 128-byte line of every weight row) per stage.  MXFP4 tiles have 32 or 64
// rows: a larger tile's two-block stage would leave at most one stage in
// flight (every MXFP4 expert on 32- and 64-row tiles measured fastest).
// NVFP4 weights are staged like MXFP4 ones (the same e2m1 bytes) and take
// 32-row tiles only: their e4m3 block scales add 4 KB to a stage.
constexpr int tile_khalves(int FMT, int TM) { return (FMT == TF_FP4 || FMT == TF_NV4) ? 2 : 1; }
// Ring depth: kStages - 1 stages in flight.
constexpr int tile_stages(int FMT, int TM) { return TM == 256 ? 2 : (TM == 32 && FMT == TF_FP8) ? 4 : 3; }

struct TileArgs {
  const uint8_t* a;               // L1: xq [Mr, L]; L2: hq [R, I]; dense: bf16 rows [M, K]
  const float* a_scale;           // routed: scales of the A rows by routed row, K-block-major: L1 the x scales
                                  // [L/128, R] (RowScales), L2 sh [I/128, R]
  const int32_t* sorted_pair;     // L1: row -> token * k + slot
  const int32_t* expert_offsets;  // routed
  const uint8_t* b;               // weights (bytes)
  const void* b_scale;            // FP8: [E, N/128, K/128] f32; FP4: [E, N, K/32] e8m0; NV4: [E, N, K/16] e4m3
  const float* b_tscale;          // NV4: [E] the fp32 scale of each expert's matrix
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
  int nslots;                     // dense: row tiles; routed: unused (the tile count comes from expert_offsets)
  int big_rows;                   // routed: experts with >= big_rows rows take 128-row tiles, the others 32-row tiles
  int huge_rows;                  // routed: experts with >= huge_rows rows take 256-row tiles instead
  int mid_rows;                   // routed: experts with mid_rows .. big_rows - 1 rows take 64-row tiles
  int scales_packed;              // MXFP4 / NV4: block scales in the packed tile order (k_pack_e8m0 / k_pack_e4m3_16)
  int ksplit;                     // dense: K ranges (each tile's K steps split evenly; 0 or 1: none)
  float* partial;                 // dense, ksplit > 1: FP32 partials [ksplit, M, B rows], reduced by k_dense_reduce
};

// MXFP4 e8m0 scales from the natural order [E][N][K/32] into the tile order
// P[e][t][s][h][j][g] = S[e][n(t, j)][8 s + 4 h + g] (t: tile of 256 weight
// rows, s: 256-wide K step, h: 128-wide K block, j: tile row, g: 32-wide
// group), one 4-byte word (the four groups g) per thread.  Tile row j is
// weight row 256 t + j, or for the paired L1 matrix (half = I) gate row
// 128 t + j (j < 128) and up row I + 128 t + j - 128.  The scales of one
// tile's rows for one K step are then 2 KB in a row, [h][j][g] as the
// two-K-block stage holds them in LDS; with one K block per step, block
// 2 s + h is the 1 KB at offset 1024 (2 s + h).
__global__ __launch_bounds__(256) void k_pack_e8m0(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                   size_t words, int N, int K, int half) {
  const size_t w = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (w >= words) return;
  const int j = static_cast<int>(w % 256);
  size_t rest = w / 256;
  const int h = static_cast<int>(rest % 2);
  rest /= 2;
  const size_t nks = static_cast<size_t>(K) / 256, ntl = static_cast<size_t>(N) / 256;
  const int s = static_cast<int>(rest % nks);
  rest /= nks;
  const size_t t = rest % ntl, e = rest / ntl;
  const size_t n = half > 0 ? (j < 128 ? 128 * t + j : static_cast<size_t>(half) + 128 * t + (j - 128)) : 256 * t + j;
  const size_t wpr = static_cast<size_t>(K) / 32;
  reinterpret_cast<uint32_t*>(dst)[w] =
      *reinterpret_cast<const uint32_t*>(src + (e * static_cast<size_t>(N) + n) * wpr + 8 * static_cast<size_t>(s) + 4 * h);
}

// NVFP4 e4m3 scales from the natural order [E][N][K/16] into the tile order
// P[e][t][s][j][q] = S[e][n(t, j)][16 s + q] (t: tile of 256 weight rows, s:
// 256-wide K step, j: tile row, q < 16), one 16-byte run (t, s, j) per
// thread; tile rows as for k_pack_e8m0.  The scales of one tile's rows for
// one K step are then 4 KB in a row (whole-line loads instead of 16 bytes
// from each of 256 rows).
__global__ __launch_bounds__(256) void k_pack_e4m3_16(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                      size_t runs, int N, int K, int half) {
  const size_t w = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (w >= runs) return;
  const int j = static_cast<int>(w % 256);
  size_t rest = w / 256;
  const size_t nks = static_cast<size_t>(K) / 256, ntl = static_cast<size_t>(N) / 256;
  const int s = static_cast<int>(rest % nks);
  rest /= nks;
  const size_t t = rest % ntl, e = rest / ntl;
  const size_t n = half > 0 ? (j < 128 ? 128 * t + j : static_cast<size_t>(half) + 128 * t + (j - 128)) : 256 * t + j;
  const uint8_t* in = src + (e * static_cast<size_t>(N) + n) * (static_cast<size_t>(K) / 16) + 16 * static_cast<size_t>(s);
  *reinterpret_cast<uint4*>(dst + 16 * w) = *reinterpret_cast<const uint4*>(in);
}

// NVFP4 activation rows in LDS: chunk c of row r at 16-byte slot
// c ^ nv_swz(r & 7).  Lane group g reads chunks 2 g and 2 g + 1 of row l16;
// under the plain swizzle (slot c ^ (r & 7)) lane groups 2 i and 2 i + 1
// read chunks of one parity, and the LDS, serving them in one pass, finds
// pairs of them on the same banks (1.5 times the read time of a conflict-free
// pattern, measured).  This swizzle spreads the rows of each parity over
// both halves of the slots.
__host__ __device__ __forceinline__ int nv_swz(int r) { return ((r >> 1) & 1) | (r & 4); }

// Persistent: one workgroup per CU works through a list of tiles.  Tile t
// of T: XCD x (workgroups are dealt to the 8 XCDs in turn, b % 8) owns tiles
// [x * per, (x + 1) * per), per = ceil(T / 8), and its workgroups take them
// in turn, so the XCD's CUs work on neighbouring tiles together
// (neighbouring n tiles share the A rows, neighbouring slots of an expert its
// weights, in that XCD's L2).  The K steps of all of a workgroup's tiles form
// one stream through the three-stage ring: the first stages of the next tile
// are loaded while the current one finishes and while its epilogue runs.
// TM = 256: tiles of 256 rows (experts with at least huge_rows rows, the
// dense GEMMs with many rows): a quarter less LDS and L2 traffic per FLOP
// than 128 rows and half the barriers, one stage in flight.  TM = 128:
// experts with big_rows .. huge_rows - 1 rows, 8 waves as 2 (M) x 4 (N) of
// 64 x 64.  TM = 64: experts with mid_rows .. big_rows - 1 rows, 8 waves of
// 64 x 32, three stages.  TM = 32: tiles of 32 rows for the experts with
// fewer rows (decode sizes), 8 waves of 32 x 32, a deeper ring.  Either way
// 256 B rows (weight rows) per tile.
// LDS of one workgroup of the tiled kernel (ring + expert tables + per-tile
// side data), carved from one buffer so that a persistent kernel running
// several stages of the tail can reuse it.
template <int KIND, int FMT, int TM>
struct TileLds {
  static constexpr bool kFP4 = FMT == TF_FP4;
  static constexpr bool kScaled = FMT != TF_BF16;
  static constexpr bool kRouted = KIND != TK_DENSE;
  static constexpr int kKH = tile_khalves(FMT, TM);
  static constexpr int kStages = tile_stages(FMT, TM);
  static constexpr int kStage =
      TM * 128 * kKH + kTN * 128 + (kScaled ? (FMT == TF_NV4 ? 8 * TM + 4096 : kKH == 2 ? 8 * TM + 2048 : 2048) : 0);
  static constexpr int kPairRows = (TM < 64) ? 64 : TM;
  static constexpr int kWavesN = (TM <= 64) ? 8 : 4;
  static constexpr int kRing = 0;
  static constexpr int kEoff = kRing + kStages * kStage;
  static constexpr int kPre = kEoff + 4 * (kRouted ? kTileMaxE + 1 : 1);
  static constexpr int kPair = kPre + 4 * (kRouted ? kTileMaxE + 1 : 1);
  static constexpr int kWsc = kPair + 4 * 3 * kPairRows;
  static constexpr int kAmax = kWsc + 4 * 3 * 2 * kMaxKBlocks;
  static constexpr int kBytes = kAmax + 4 * kWavesN * TM;
};

// The LDS pieces of one workgroup of the tiled kernel.  The standalone
// kernel passes separate arrays (so the compiler knows they do not overlap);
// a kernel that runs several stages carves them from one buffer
// (tile_smem_in).
struct TileSmem {
  uint8_t* ring;
  int* eoff;
  int* pre;
  int* pair;
  float* wsc;
  float* amax;
};

template <int KIND, int FMT, int TM>
__device__ __forceinline__ TileSmem tile_smem_in(uint8_t* base) {
  using Lds = TileLds<KIND, FMT, TM>;
  return TileSmem{base + Lds::kRing, reinterpret_cast<int*>(base + Lds::kEoff), reinterpret_cast<int*>(base + Lds::kPre),
                  reinterpret_cast<int*>(base + Lds::kPair), reinterpret_cast<float*>(base + Lds::kWsc),
                  reinterpret_cast<float*>(base + Lds::kAmax)};
}

template <int KIND, int FMT, int EPI, int TM = kTM>
__device__ __forceinline__ void tile_run(const TileArgs& p, const TileSmem& sm, int wg, int nwg) {
  constexpr bool kFP4 = FMT == TF_FP4;
  constexpr bool kNV4 = FMT == TF_NV4;
  constexpr bool kNib = kFP4 || kNV4;                // 4-bit weights, 64 bytes per row and K block
  constexpr bool kBF16 = FMT == TF_BF16;
  constexpr bool kScaled = !kBF16;
  constexpr bool kRouted = KIND != TK_DENSE;
  constexpr bool kPaired = KIND == TK_L1 || (KIND == TK_DENSE && EPI == EPI_SWIGLU);
  static_assert(TM == 256 || TM == 128 || ((TM == 64 || TM == 32) && KIND != TK_DENSE), "tile rows");
  constexpr int kWavesM = (TM <= 64) ? 1 : 2;        // wave grid over the tile
  constexpr int kWavesN = 8 / kWavesM;
  constexpr int kMT = TM / (16 * kWavesM);           // 16-row MFMA tiles per wave
  constexpr int kNJ = kTN / (16 * kWavesN);          // 16-column MFMA tiles per wave
  constexpr int kStages = tile_stages(FMT, TM);     // ring depth (kStages - 1 steps in flight)
  constexpr int kKH = tile_khalves(FMT, TM);         // 128-wide K blocks per stage
  static_assert(!kFP4 || TM <= 64, "MXFP4 tiles: 32 or 64 rows");
  static_assert(!kNV4 || TM == 32, "NVFP4 tiles: 32 rows");
  constexpr int kABlk = TM / 8;                      // 1 KB blocks of A per stage and K block
  constexpr int kAL = (kABlk + 7) / 8;               // A blocks loaded per wave and K block
  constexpr int kABytes1 = TM * 128;                 // A bytes of one K block: 32, 16, 8 or 4 KB
  constexpr int kABytes = kABytes1 * kKH;
  constexpr int kBBytes = kTN * 128;                 // 128 bytes of each of the 256 B rows: 32 KB
  // scale words of a stage.  FP8 (one K block, 2 KB, 256 bytes per wave):
  // activation scales (one word per row) loaded by waves 0 .. kActW - 1; the
  // other waves load zeros into their part.  MXFP4 (two K blocks): activation words
  // [half][row] (8 TM bytes: every wave loads its share of them, waves
  // past the 2 TM words repeating the first ones, the same bytes to the same
  // place), then the e8m0 words [half][B row] (2 KB, wave w: half w / 4,
  // B rows 64 (w % 4) + lane).  NVFP4 (two K blocks): waves 0-3 the e4m3
  // scales of B rows 64 w + lane (16 bytes: 8 per K block), waves 4-7 the
  // activation words (each wave all 2 TM of them, to the same place).
  constexpr int kActW = (TM + 63) / 64 < 2 ? 2 : (TM + 63) / 64;
  constexpr int kActW2 = (2 * TM) / 64;              // two K blocks: waves with distinct activation words
  constexpr int kSOff = kABytes + kBBytes;
  constexpr int kE8Off = (kKH == 2) ? 8 * TM : 256 * kActW;
  static_assert(kKH == 2 || kE8Off + 1024 <= 2048, "scale words");
  constexpr int kSBytes = !kScaled ? 0 : kNV4 ? 8 * TM + 4096 : (kKH == 2) ? 8 * TM + 2048 : 2048;
  static_assert(!kNV4 || 2 * TM <= 64, "NVFP4: one wave's 64 lanes carry every activation word");
  constexpr int kStage = kSOff + kSBytes;
  constexpr int kBChunks = 4;                        // 16-byte B loads per thread and stage
  constexpr int kSLoads = kNV4 ? 1 : kScaled ? kKH : 0;  // scale loads per thread and stage
  // A pieces of a stage (1 KB each): with two K blocks of 32 rows there are
  // eight, one per wave (wave w: K block w / 4, block w % 4); otherwise wave
  // w loads blocks (w + 8 i) % kABlk of every K block (TM = 32 with one K
  // block: waves 4-7 load the same blocks as waves 0-3, the same bytes to the
  // same place)
  constexpr bool kASplit = kABlk * kKH == 8 && kKH == 2;
  constexpr int kAPerWave = kASplit ? 1 : kAL * kKH;   // A loads per wave and stage
  constexpr int kLoads = kAPerWave + kBChunks + kSLoads;  // direct loads per wave and stage
  constexpr uint32_t kNoRow = 0x80000000u;           // offset past any buffer: reads zeros
  using Lds = TileLds<KIND, FMT, TM>;
  static_assert(Lds::kStage == kStage && Lds::kStages == kStages && Lds::kWavesN == kWavesN, "LDS plan");
  uint8_t* ring = sm.ring;
  int* s_eoff = sm.eoff;  // expert row offsets
  int* s_pre = sm.pre;    // row tiles of the experts before e
  // per-tile data, buffer j % 3 for tile j: loaded while tile j - 2 still
  // computes and read until tile j's last step
  constexpr int kPairRows = Lds::kPairRows;  // one 64-lane load per 64 rows
  auto s_pair = reinterpret_cast<int(*)[kPairRows]>(sm.pair);  // L1: sorted pair ids of a tile's rows
  // aux loads of the next tile: pair ids by waves 0 .. kPairRows / 64 - 1 (L1),
  // the two weight-scale rows (FP8) by waves kWscW and kWscW + 1
  constexpr int kWscW = (kPairRows / 64 < 2) ? 2 : kPairRows / 64;
  auto s_wsc = reinterpret_cast<float(*)[2][kMaxKBlocks]>(sm.wsc);  // FP8: weight scales of a tile's two 128-row B halves
  auto s_amax = reinterpret_cast<float(*)[TM]>(sm.amax);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const int l16 = lane & 15, g = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int nsplit = (!kRouted && p.ksplit > 1) ? p.ksplit : 1;
  const int nk = kBF16 ? p.K / 64 / nsplit : p.K / (128 * kKH);  // K steps (stages of the stream) of a tile
  const int nkb = p.K / 128;                       // scale blocks along K (scaled formats)
  const int elem = kBF16 ? 2 : 1;                  // bytes per A element
  const int nbrows = kPaired ? 2 * p.half : p.N;  // B rows of one expert / of the dense matrix
  const size_t a_row_bytes = static_cast<size_t>(p.K) * elem;
  const size_t brow_bytes = kNib ? static_cast<size_t>(p.K) / 2 : static_cast<size_t>(p.K) * elem;
  const size_t wpr = static_cast<size_t>(p.K) / 32;  // FP4: e8m0 bytes per weight row

  // ---- this workgroup's tiles
  int T;
  int n_rows = 0;  // routed: rows of the sorted routed segment (the stride of the K-block-major scales)
  if (kRouted) {
    for (int i = tid; i <= p.E; i += 512) s_eoff[i] = p.expert_offsets[i];
    __syncthreads();
    if (wave == 0) {
      // exclusive prefix over the experts of their row tiles (TM = 256: the
      // experts with at least huge_rows rows; TM = 128: big_rows ..
      // huge_rows - 1; TM = 32: the others)
      const int per = (p.E + 63) / 64;
      const int eb = min(lane * per, p.E), ee = min(eb + per, p.E);
      auto ntile = [&](int e) {
        const int c = s_eoff[e + 1] - s_eoff[e];
        if (TM == 256) return use256(c, p.huge_rows) ? tiles256(c) : 0;
        if (TM == 128) {
          if (use256(c, p.huge_rows)) return tail128(c) ? 1 : 0;
          return c >= p.big_rows ? (c + TM - 1) / TM : 0;
        }
        if (TM == 64) return (c >= p.mid_rows && c < p.big_rows) ? (c + TM - 1) / TM : 0;
        return (c < p.big_rows && c < p.mid_rows) ? (c + TM - 1) / TM : 0;
      };
      int local = 0;
      for (int e = eb; e < ee; ++e) local += ntile(e);
      int incl = local;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int n = __shfl_up(incl, d);
        if (lane >= d) incl += n;
      }
      int run = incl - local;
      for (int e = eb; e < ee; ++e) {
        s_pre[e] = run;
        run += ntile(e);
      }
      if (lane == 63) s_pre[p.E] = incl;
    }
    __syncthreads();
    T = s_pre[p.E] * p.ntn;
    n_rows = __builtin_amdgcn_readfirstlane(s_eoff[p.E]);
  } else {
    T = p.nslots * p.ntn * nsplit;
  }
  const int xcd = wg & 7, lb = wg >> 3, nbx = nwg >> 3;
  const int per = (T + 7) / 8, lo = xcd * per, hi = min(T, lo + per);
  const int n_my = (lo + lb < hi) ? (hi - lo - lb + nbx - 1) / nbx : 0;
  if (n_my == 0) return;  // uniform

  struct Desc {
    int e, row0, rows, nt, kz;  // kz: the dense tile's K range
  };
  // tile j of this workgroup.  Routed tiles are numbered expert by expert;
  // within an expert (ns row slots x ntn n tiles) in blocks of kNBlk n tiles,
  // slot-major inside a block, so that the workgroups of an XCD working on
  // neighbouring tiles share both the weight rows (same n tile, different
  // slots) and the gathered activation rows (same slot, different n tiles)
  // in the XCD's L2: an expert with many row slots is streamed about ns /
  // (slots per round) times instead of once per slot.
  constexpr int kNBlk = 4;
  constexpr int kDenseGroup = 4;
  // dense 128-row tiles (up to about 2048 rows) when every tile of the launch runs at once
  const bool grouped = !kRouted && TM == 128 && T <= nwg;
  auto desc = [&](int j) -> Desc {
    const int t = lo + lb + j * nbx;
    Desc d;
    d.kz = 0;
    if (kRouted) {
      int a = 0, b = p.E;  // s_pre[a] * ntn <= t < s_pre[b] * ntn
      while (b - a > 1) {
        const int m = (a + b) >> 1;
        if (s_pre[m] * p.ntn <= t) a = m;
        else b = m;
      }
      d.e = a;
      const int ns = s_pre[a + 1] - s_pre[a];
      const int local = t - s_pre[a] * p.ntn;
      const int full = p.ntn / kNBlk;
      int blk = local / (kNBlk * ns), n0, w, rem;
      if (blk < full) {
        n0 = blk * kNBlk;
        w = kNBlk;
        rem = local - blk * kNBlk * ns;
      } else {
        n0 = full * kNBlk;
        w = p.ntn - n0;
        rem = local - full * kNBlk * ns;
      }
      const int slot = rem / w;
      d.nt = n0 + (rem - slot * w);
      // 128-row tiles of an expert with 256-row tiles cover only the rows
      // past its full 256-row tiles
      const int c = s_eoff[a + 1] - s_eoff[a];
      const int base = (TM == 128 && use256(c, p.huge_rows)) ? c / 256 * 256 : 0;
      d.row0 = s_eoff[a] + base + slot * TM;
      d.rows = min(TM, s_eoff[a + 1] - d.row0);
    } else {
      // K range slowest.  128-row launches whose tiles all run at once:
      // within a K range, groups of kDenseGroup row slots, the slots of a
      // group fastest, so the 32 tiles an XCD's workgroups take side by side
      // cover kDenseGroup slots x 8 n tiles and each activation row block
      // and each weight tile they stream serves 8 and kDenseGroup of them
      // from that XCD's L2 (slot-major runs streamed the weights again for
      // every slot: the 1024-token up-projection fetched 433 MB for 51 MB of
      // weights, 147 MB this way).  The 256-row launches (several rounds, or
      // MFMA-bound at 4096 rows) keep slot-major runs, which measured as
      // fast or faster there.
      const int per_z = p.nslots * p.ntn;
      d.kz = t / per_z;
      const int r = t - d.kz * per_z;
      int slot;
      if (grouped) {
        const int grp = r / (kDenseGroup * p.ntn);
        const int first = grp * kDenseGroup;
        const int gsize = min(kDenseGroup, p.nslots - first);
        const int within = r - grp * kDenseGroup * p.ntn;
        slot = first + within % gsize;
        d.nt = within / gsize;
      } else {
        slot = r / p.ntn;
        d.nt = r - slot * p.ntn;
      }
      d.e = 0;
      d.row0 = slot * TM;
      d.rows = min(TM, p.M - d.row0);
    }
    d.e = __builtin_amdgcn_readfirstlane(d.e);
    d.row0 = __builtin_amdgcn_readfirstlane(d.row0);
    d.rows = __builtin_amdgcn_readfirstlane(d.rows);
    d.nt = __builtin_amdgcn_readfirstlane(d.nt);
    d.kz = __builtin_amdgcn_readfirstlane(d.kz);
    return d;
  };
  // B row j of a tile (0..255) -> weight row: paired kinds take 128 gate
  // rows and the matching 128 up rows, the others 256 consecutive rows
  auto wrow = [&](int nt, int j) -> int {
    if (kPaired) return (j < 128) ? 128 * nt + j : p.half + 128 * nt + (j - 128);
    return kTN * nt + j;
  };

  // ---- per-thread load assignment ----
  // A stage holds the operands' K step as 128-byte row pieces in 1 KB blocks
  // of 8 rows.  Wave w loads blocks w + 8 i, so each of its loads fetches 8
  // whole 128-byte lines (loads of half lines run at a third of the rate).
  // Lane l lands at block + 16 l and carries row 8 * block + (l >> 3), chunk
  // (l & 7) ^ (l >> 3): chunk c of row r sits in 16-byte slot c ^ (r & 7) of
  // the row's 128 bytes, so the 8 lanes that read one chunk of 8
  // consecutive rows hit 8 different slots (no bank conflicts).  (MXFP4 B
  // rows hold two K blocks a step, so they are 128-byte pieces too.)
  // (each lane's row within a block, lane >> 3, its chunk (lane & 7) ^ (lane
  // >> 3) and its B rows 8 wave + (lane >> 3) + 64 i are recomputed where
  // the loads are set up, make_iss)
  // a resource with no valid bytes: loads through it write zeros
  const __amdgpu_buffer_rsrc_t z_rsrc = make_rsrc(p.b, 0u);

  // load offsets of one tile
  struct Iss {
    __amdgpu_buffer_rsrc_t ra, rb, rs, rs2;
    uint32_t a_off[kAL], b_off[kBChunks], s_off, s_off2;
    int s_step, s_step2;  // bytes of the scale loads' sources per K step (wave-uniform)
  };
  auto make_iss = [&](const Desc& d, int buf) -> Iss {
    // the lane's coordinates, recomputed from an opaque copy of the thread
    // index rather than held live across the K loop (the 256-row L1 tile has
    // no registers to spare, and a spilled value's reload would wait for
    // every load in flight)
    int tid_o = threadIdx.x;
    asm volatile("" : "+v"(tid_o));
    const int lane = tid_o & 63, wave = tid_o >> 6, q8 = lane >> 3, st_c = (lane & 7) ^ q8, st_r0 = 8 * wave + q8;
    const int st_ca = kNV4 ? (lane & 7) ^ nv_swz(q8) : st_c;  // A rows (NVFP4: their own swizzle)
    Iss r;
    // bytes along a row before this tile's K range (split dense tiles)
    const uint32_t kbase = kRouted ? 0u : static_cast<uint32_t>(d.kz) * static_cast<uint32_t>(nk) * 128u;
    if (KIND == TK_L1)  // gathered token rows of x codes
      r.ra = make_rsrc(p.a, static_cast<uint32_t>(static_cast<size_t>(p.M) * a_row_bytes));
    else
      r.ra = make_rsrc(p.a + static_cast<size_t>(d.row0) * a_row_bytes, static_cast<uint32_t>(static_cast<size_t>(d.rows) * a_row_bytes));
    // A block (wave + 8 i) % kABlk (see kASplit)
#pragma unroll
    for (int i = 0; i < kAL; ++i) {
      const int row = 8 * ((wave + 8 * i) % kABlk) + q8;
      uint32_t o = kNoRow;
      if (row < d.rows) {
        const size_t rr = (KIND == TK_L1) ? static_cast<size_t>(s_pair[buf][row] / p.k) : static_cast<size_t>(row);
        o = static_cast<uint32_t>(rr * a_row_bytes) + 16u * st_ca + kbase;
      }
      r.a_off[i] = o;
    }
    r.rb = make_rsrc(p.b + static_cast<size_t>(d.e) * nbrows * brow_bytes, static_cast<uint32_t>(static_cast<size_t>(nbrows) * brow_bytes));
#pragma unroll
    for (int i = 0; i < kBChunks; ++i) {
      const int row = st_r0 + 64 * i;
      const int c = st_c;
      r.b_off[i] = static_cast<uint32_t>(static_cast<size_t>(wrow(d.nt, row)) * brow_bytes) + 16u * c + kbase;
    }
    // scale words, one 4-byte load per lane and stage: waves 0-1 the
    // activation scales of tile rows 64 w + lane (w < kActW), waves kActW ..
    // kActW + 3 (FP4) the e8m0 words of B rows 64 (w - kActW) + lane; the
    // other waves load zeros
    r.rs = z_rsrc;
    r.s_off = kNoRow;
    r.rs2 = z_rsrc;
    r.s_off2 = kNoRow;
    r.s_step = kKH == 2 ? 8 : 4;
    r.s_step2 = 0;
    // packed e8m0 (k_pack_e8m0): this tile's run of K steps
    const uint32_t pk_tile = static_cast<uint32_t>(d.nt) * static_cast<uint32_t>(p.K / 256) * 2048u;
    if (kNV4) {
      if (wv < 4) {
        // e4m3 scales of B row j = 64 wv + lane: 16 bytes a row and step
        const int j = 64 * wv + lane;
        r.rs = make_rsrc(static_cast<const uint8_t*>(p.b_scale) + static_cast<size_t>(d.e) * nbrows * (p.K / 16),
                         static_cast<uint32_t>(static_cast<size_t>(nbrows) * (p.K / 16)));
        if (p.scales_packed) {  // k_pack_e4m3_16: this tile's 4 KB runs, one per K step
          r.s_off = static_cast<uint32_t>(d.nt) * static_cast<uint32_t>(p.K / 256) * 4096u + 16u * static_cast<uint32_t>(j);
          r.s_step = 4096;
        } else {
          r.s_off = static_cast<uint32_t>(wrow(d.nt, j) * (p.K / 16));
          r.s_step = 16;
        }
      } else {
        // activation word q = lane: half q / TM, row q % TM (as for MXFP4)
        const int hh = lane / TM, row = lane - hh * TM;
        r.rs = make_rsrc(p.a_scale, static_cast<uint32_t>(static_cast<size_t>(nkb) * n_rows * 4));
        if (hh < 2 && row < d.rows)
          r.s_off = static_cast<uint32_t>((static_cast<size_t>(hh) * n_rows + d.row0 + row) * 4);
        r.s_step = 8 * n_rows;
      }
    } else if (kScaled && kKH == 2) {
      // e8m0 words of half wv / 4, B row 64 (wv % 4) + lane (8 bytes a row and stage)
      const int j = 64 * (wv & 3) + lane;
      r.rs = make_rsrc(static_cast<const uint8_t*>(p.b_scale) + static_cast<size_t>(d.e) * nbrows * wpr,
                       static_cast<uint32_t>(nbrows * wpr));
      if (p.scales_packed) {
        r.s_off = pk_tile + 1024u * static_cast<uint32_t>(wv >> 2) + 4u * static_cast<uint32_t>(j);
        r.s_step = 2048;
      } else {
        r.s_off = static_cast<uint32_t>(wrow(d.nt, j) * wpr) + 4u * static_cast<uint32_t>(wv >> 2);
      }
      // activation word q: half q / TM, row q % TM (K block 2 k + hh of routed
      // row row0 + row: one contiguous run per half)
      const int q = 64 * (wv % kActW2) + lane, hh = q / TM, row = q - hh * TM;
      r.rs2 = make_rsrc(p.a_scale, static_cast<uint32_t>(static_cast<size_t>(nkb) * n_rows * 4));
      r.s_step2 = 8 * n_rows;
      if (row < d.rows) r.s_off2 = static_cast<uint32_t>((static_cast<size_t>(hh) * n_rows + d.row0 + row) * 4);
    } else if (kScaled) {
      if (wv < (TM + 63) / 64) {
        // K block k of routed rows row0 + 64 w + lane: one contiguous run
        const int row = 64 * wv + lane;
        r.rs = make_rsrc(p.a_scale, static_cast<uint32_t>(static_cast<size_t>(nkb) * n_rows * 4));
        r.s_step = 4 * n_rows;
        if (row < d.rows) r.s_off = static_cast<uint32_t>((static_cast<size_t>(d.row0) + row) * 4);
      }
    }
    return r;
  };
  // stage k of a tile -> ring slot; live == false loads zeros (no memory
  // traffic).  part: 1 = the B rows, 2 = the A rows and the scale words, 3 = all
  auto issue = [&](uint8_t* st, const Iss& r, int k, bool live, int part = 3) {
    if (part & 2) {
      if (kASplit) {
        const int h = wv / kABlk;
        dma16(live ? r.ra : z_rsrc, st + kABytes1 * h + 1024 * (wv % kABlk), r.a_off[0], (k * kKH + h) * 128);
      } else {
#pragma unroll
        for (int h = 0; h < kKH; ++h)
#pragma unroll
          for (int i = 0; i < kAL; ++i)
            dma16(live ? r.ra : z_rsrc, st + kABytes1 * h + 1024 * ((wv + 8 * i) % kABlk), r.a_off[i],
                  (k * kKH + h) * 128);
      }
    }
    if (part & 1) {
#pragma unroll
      for (int i = 0; i < kBChunks; ++i)
        dma16(live ? r.rb : z_rsrc, st + kABytes + 8192 * i + 1024 * wv, r.b_off[i], k * 128);
    }
    if (!(part & 2)) return;
    if (kNV4) {
      if (wv < 4) dma16(live ? r.rs : z_rsrc, st + kSOff + kE8Off + 1024 * wv, r.s_off, r.s_step * k);
      else dma4(live ? r.rs : z_rsrc, st + kSOff, r.s_off, r.s_step * k);
    } else if (kScaled && kKH == 2) {
      dma4(live ? r.rs : z_rsrc, st + kSOff + kE8Off + 256 * wv, r.s_off, r.s_step * k);
      dma4(live ? r.rs2 : z_rsrc, st + kSOff + 256 * (wv % kActW2), r.s_off2, r.s_step2 * k);
    } else if (kScaled) {
      dma4(live ? r.rs : z_rsrc, st + kSOff + 256 * wv, r.s_off, r.s_step * k);
    }
  };
  // load q of issue's batch alone (the same order: the A pieces, the B
  // chunks, the scale words), for tiles with one K block and one scale load
  // per stage (the routed L1's 256-row tiles, which spread their batch over
  // a step)
  auto issue_one = [&](uint8_t* st, const Iss& r, int k, bool live, int q) {
    if constexpr (kKH == 1 && !kASplit && !kNV4) {
      if (q < kAL) {
        dma16(live ? r.ra : z_rsrc, st + 1024 * ((wv + 8 * q) % kABlk), r.a_off[q], k * 128);
      } else if (q < kAL + kBChunks) {
        const int i = q - kAL;
        dma16(live ? r.rb : z_rsrc, st + kABytes + 8192 * i + 1024 * wv, r.b_off[i], k * 128);
      } else if (kScaled) {
        dma4(live ? r.rs : z_rsrc, st + kSOff + 256 * wv, r.s_off, r.s_step * k);
      }
    }
  };
  // per-tile data loaded ahead (issued first in a stage's batch, only by the
  // waves that carry it): L1 sorted pair ids (one wave per 64 rows), FP8 weight-scale
  // rows (waves kWscW, kWscW + 1)
  auto aux = [&](const Desc& d, int buf) {
    int tid_o = threadIdx.x;  // (recomputed, as in make_iss)
    asm volatile("" : "+v"(tid_o));
    const int lane = tid_o & 63;
    if (KIND == TK_L1 && wv < kPairRows / 64) {
      dma4(make_rsrc(p.sorted_pair + d.row0, static_cast<uint32_t>(d.rows) * 4u), reinterpret_cast<uint8_t*>(&s_pair[buf][64 * wv]),
           4u * (64 * wv + lane), 0);
    } else if (kNV4 && wv == kWscW) {
      // the matrix's fp32 scale into word 0 (the other lanes read zeros)
      dma4(make_rsrc(p.b_tscale + d.e, 4u), reinterpret_cast<uint8_t*>(&s_wsc[buf][0][0]), 4u * lane, 0);
    } else if (FMT == TF_FP8 && (wv == kWscW || wv == kWscW + 1)) {
      const int q = wv - kWscW;
      const int wr = wrow(d.nt, 128 * q);
      const float* src = static_cast<const float*>(p.b_scale) +
                         (static_cast<size_t>(d.e) * (nbrows / 128) + wr / 128) * nkb;
      dma4(make_rsrc(src, (wr < nbrows) ? static_cast<uint32_t>(nkb) * 4u : 0u), reinterpret_cast<uint8_t*>(&s_wsc[buf][q][0]),
           4u * lane, 0);
    }
  };

  // B blocks of this wave, j = 0..3 (paired: two gate blocks, then the two
  // matching up blocks)
  auto bblk = [&](int j) {
    if (kPaired) return (j < kNJ / 2) ? (kNJ / 2) * wn + j : 8 + (kNJ / 2) * wn + (j - kNJ / 2);
    return kNJ * wn + j;
  };
  // this lane's MFMA operand pieces within a 16-row block (2 KB): row l16,
  // chunk g (registers 0-3) and chunk 4 + g (registers 4-7)
  const int fr = 1024 * (l16 >> 3) + 128 * (l16 & 7);
  const int f_lo = fr + 16 * (g ^ (l16 & 7));
  const int f_hi = fr + 16 * ((4 | g) ^ (l16 & 7));
  // NVFP4's activation pieces: chunks 2 g and 2 g + 1 (32 consecutive K),
  // in rows swizzled by nv_swz
  const int f_nv0 = fr + 16 * ((2 * g) ^ nv_swz(l16 & 7));
  const int f_nv1 = fr + 16 * ((2 * g + 1) ^ nv_swz(l16 & 7));

  // Accumulators.  L1 (kTrans): the weight block is the MFMA's A operand
  // and the activation block its B operand, so acc[mt][j][i] is weight
  // column 16 bblk(j) + 4 g + i (of the tile's 256 B rows) for tile row
  // 16 kMT wm + 16 mt + l16: a lane holds one token row per mt, and the FP8
  // promotion factor (activation scale x weight scale) is one value per
  // (mt, weight half); its epilogue goes through LDS anyway.  L2 and the
  // dense kinds keep the activation block as A (acc[mt][j][i] is tile row
  // 16 kMT wm + 16 mt + 4 g + i, column 16 bblk(j) + l16), whose direct
  // stores put 16 lanes on one row.
  constexpr bool kTrans = KIND == TK_L1;
  f32x4 acc[kMT][kNJ];
  // `between(mt)` runs after row block mt's products are issued (routed L1
  // 256-row tiles: it issues load mt of the next stage)
  auto compute = [&](const uint8_t* st, int ks, int buf, auto&& between) {
    // weight scales of this step (FP8): the wave's B rows lie in the tile's
    // row half 16 * bblk(0) / 128 (paired: its gate rows) and 16 * bblk(3) / 128
    float sw_lo = 1.0f, sw_hi = 1.0f;
    if (FMT == TF_FP8) {
      sw_lo = s_wsc[buf][(16 * bblk(0)) / 128][ks];
      sw_hi = s_wsc[buf][(16 * bblk(kNJ - 1)) / 128][ks];
    } else if (kNV4) {
      sw_lo = sw_hi = s_wsc[buf][0][0];  // the matrix's fp32 scale
    }
    // weight fragments of K block h of the step (FP4: with their e8m0 scales)
    auto load_b = [&](int j, i32x8& bfj, int& sbj, int h = 0) {
      const int bb = bblk(j);
      if (kNV4) {
        // lane group g takes K [32 g, 32 g + 32) of K block h (for both
        // operands, see the activation fragments below): chunk 4 h + g of the
        // weight row, as for MXFP4, and the e4m3 scales of its two 16-element
        // groups, bytes 8 h + 2 g and 8 h + 2 g + 1 of the row's 16 (natural
        // and packed order alike)
        const i32x4 v = *reinterpret_cast<const i32x4*>(st + kABytes + bb * 2048 + (h ? f_hi : f_lo));
        const i32x4 z = {0, 0, 0, 0};
        bfj = __builtin_shufflevector(v, z, 0, 1, 2, 3, 4, 5, 6, 7);
        sbj = *reinterpret_cast<const uint16_t*>(st + kSOff + kE8Off + 16 * (16 * bb + l16) + 8 * h + 2 * g);
      } else if (kFP4) {
        // two K blocks of 128-byte rows in the swizzled layout of the 8-bit
        // operands: K block h in chunks 4 h .. 4 h + 3
        const i32x4 v = *reinterpret_cast<const i32x4*>(st + kABytes + bb * 2048 + (h ? f_hi : f_lo));
        const i32x4 z = {0, 0, 0, 0};
        bfj = __builtin_shufflevector(v, z, 0, 1, 2, 3, 4, 5, 6, 7);
        sbj = st[kSOff + kE8Off + 1024 * h + (16 * bb + l16) * 4 + g];
      } else {
        const uint8_t* bp = st + kABytes + bb * 2048;
        const i32x4 lo4 = *reinterpret_cast<const i32x4*>(bp + f_lo);
        const i32x4 hi4 = *reinterpret_cast<const i32x4*>(bp + f_hi);
        bfj = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        sbj = 127;
      }
    };
    // this lane's activation fragment of row block mt
    auto load_a = [&](int mt) -> i32x8 {
      const uint8_t* ab = st + (kMT * wm + mt) * 2048;
      const i32x4 lo4 = *reinterpret_cast<const i32x4*>(ab + f_lo);
      const i32x4 hi4 = *reinterpret_cast<const i32x4*>(ab + f_hi);
      return __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    if constexpr (kMT > 4) {
      // 256-row tiles: 8 row blocks per wave and 128 accumulator registers,
      // so the weight fragments are loaded once per step and the activation
      // fragments one row block at a time
      if (kBF16) {
        bf16x8 b0[kNJ], b1[kNJ];
#pragma unroll
        for (int j = 0; j < kNJ; ++j) {
          const uint8_t* bp = st + kABytes + bblk(j) * 2048;
          b0[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(bp + f_lo));
          b1[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(bp + f_hi));
        }
        // (the next row block's fragment is read while this one's products run)
        i32x8 a_cur = load_a(0);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          const i32x4 alo = __builtin_shufflevector(a_cur, a_cur, 0, 1, 2, 3);
          const i32x4 ahi = __builtin_shufflevector(a_cur, a_cur, 4, 5, 6, 7);
#pragma unroll
          for (int j = 0; j < kNJ; ++j) {
            acc[mt][j] = mfma_bf16(__builtin_bit_cast(bf16x8, alo), b0[j], acc[mt][j]);
            acc[mt][j] = mfma_bf16(__builtin_bit_cast(bf16x8, ahi), b1[j], acc[mt][j]);
          }
          between(mt);
          if (mt + 1 < kMT) a_cur = load_a(mt + 1);
        }
        return;
      }
      i32x8 bf[kNJ];
      int sb[kNJ];
#pragma unroll
      for (int j = 0; j < kNJ; ++j) load_b(j, bf[j], sb[j]);
      const float* ss = reinterpret_cast<const float*>(st + kSOff);
      if (kTrans) {
        // L1: row block mt - 1 is promoted after row block mt's products are
        // issued, so the multiply-adds find their products done (reading the
        // next block's operands ahead instead measured no faster here)
        f32x4 pr[2][kNJ];
#pragma unroll
        for (int mt = 0; mt <= kMT; ++mt) {
          if (mt < kMT) {
            const i32x8 a8 = load_a(mt);
#pragma unroll
            for (int j = 0; j < kNJ; ++j)
              pr[mt & 1][j] = kFP4 ? mfma_fp4_fp8(bf[j], sb[j], a8) : mfma_fp8(bf[j], a8);
            between(mt);
          }
          if (mt > 0) {
            const int mp = mt - 1;
            const float v = ss[16 * kMT * wm + 16 * mp + l16];
            const float s_lo = v * sw_lo, s_hi = v * sw_hi;
#pragma unroll
            for (int j = 0; j < kNJ; ++j) {
              const float f = (kPaired && j >= kNJ / 2) ? s_hi : s_lo;
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[mp][j][i] += pr[mp & 1][j][i] * f;
            }
          }
        }
      } else {
        // L2: software-pipelined by one row block: the activation fragment
        // and scales of block mt + 1 are read from LDS while block mt's
        // products run, and block mt is promoted after that (reading them
        // just before their use left two LDS round trips per block exposed,
        // which the stage loads landing in LDS lengthen: prefill routed L2
        // 400 -> 368 us)
        i32x8 a_cur = load_a(0);
        f32x4 v_cur = *reinterpret_cast<const f32x4*>(ss + 16 * kMT * wm + 4 * g);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          f32x4 pr[kNJ];
#pragma unroll
          for (int j = 0; j < kNJ; ++j) pr[j] = kFP4 ? mfma_fp8_fp4(a_cur, bf[j], sb[j]) : mfma_fp8(a_cur, bf[j]);
          between(mt);
          i32x8 a_nxt = a_cur;
          f32x4 v_nxt = v_cur;
          if (mt + 1 < kMT) {
            a_nxt = load_a(mt + 1);
            v_nxt = *reinterpret_cast<const f32x4*>(ss + 16 * kMT * wm + 16 * (mt + 1) + 4 * g);
          }
#pragma unroll
          for (int j = 0; j < kNJ; ++j) {
            const float sw = (kPaired && j >= kNJ / 2) ? sw_hi : sw_lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][j][i] += pr[j][i] * (v_cur[i] * sw);
          }
          a_cur = a_nxt;
          v_cur = v_nxt;
        }
      }
      return;
    } else {
  #pragma unroll
     for (int h = 0; h < kKH; ++h) {
      i32x8 af[kMT];
  #pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const uint8_t* ab = st + kABytes1 * h + (kMT * wm + mt) * 2048;
        // NVFP4 (FP16 matrix cores): K [32 g, 32 g + 32) of the block, chunks
        // 2 g and 2 g + 1; the FP8 MFMA's own layout otherwise
        const i32x4 lo4 = *reinterpret_cast<const i32x4*>(ab + (kNV4 ? f_nv0 : f_lo));
        const i32x4 hi4 = *reinterpret_cast<const i32x4*>(ab + (kNV4 ? f_nv1 : f_hi));
        af[mt] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      if (kBF16) {
  #pragma unroll
        for (int j = 0; j < kNJ; ++j) {
          const uint8_t* bp = st + kABytes + bblk(j) * 2048;
          const bf16x8 b0 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(bp + f_lo));
          const bf16x8 b1 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const i32x4*>(bp + f_hi));
  #pragma unroll
          for (int mt = 0; mt < kMT; ++mt) {
            const i32x4 alo = __builtin_shufflevector(af[mt], af[mt], 0, 1, 2, 3);
            const i32x4 ahi = __builtin_shufflevector(af[mt], af[mt], 4, 5, 6, 7);
            acc[mt][j] = mfma_bf16(__builtin_bit_cast(bf16x8, alo), b0, acc[mt][j]);
            acc[mt][j] = mfma_bf16(__builtin_bit_cast(bf16x8, ahi), b1, acc[mt][j]);
          }
        }
        return;
      }
      // promotion factors of this step: activation scale of the row times the
      // weight scale of the half (kTrans: the lane's row in each 16-row block;
      // else its 4 rows 4 g + i)
      constexpr int kSR = kTrans ? 1 : 4;
      float sc[2][kMT][kSR];
      {
        const float* ss = reinterpret_cast<const float*>(st + kSOff) + TM * h;
  #pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          if (kTrans) {
            const float v = ss[16 * kMT * wm + 16 * mt + l16];
            sc[0][mt][0] = v * sw_lo;
            sc[1][mt][0] = v * sw_hi;
          } else {
            const f32x4 v = *reinterpret_cast<const f32x4*>(ss + 16 * kMT * wm + 16 * mt + 4 * g);
  #pragma unroll
            for (int i = 0; i < kSR; ++i) {
              sc[0][mt][i] = v[i] * sw_lo;
              sc[1][mt][i] = v[i] * sw_hi;
            }
          }
        }
      }
      if constexpr (kNV4) {
        // FP16 matrix cores: the activation chunks converted once per K
        // block, each weight block's when it is read
        f16x8 xa[kMT][4];
  #pragma unroll
        for (int mt = 0; mt < kMT; ++mt) fp8_frag_f16(af[mt], xa[mt]);
        if (kTrans) {
          // as below: group j - 1 is promoted after group j is issued
          f32x4 pr[2][kMT];
  #pragma unroll
          for (int j = 0; j <= kNJ; ++j) {
            if (j < kNJ) {
              i32x8 bf;
              int sb;
              load_b(j, bf, sb, h);
              f16x8 wb[4];
              nvfp4_frag_f16(bf, sb, wb);
  #pragma unroll
              for (int mt = 0; mt < kMT; ++mt) pr[j & 1][mt] = mfma_f16_block(wb, xa[mt]);
            }
            if (j > 0) {
              const int jp = j - 1;
              const int hsel = (kPaired && jp >= kNJ / 2) ? 1 : 0;
  #pragma unroll
              for (int mt = 0; mt < kMT; ++mt)
  #pragma unroll
                for (int i = 0; i < 4; ++i) acc[mt][jp][i] += pr[jp & 1][mt][i] * sc[hsel][mt][0];
            }
          }
        } else {
  #pragma unroll
          for (int j = 0; j < kNJ; ++j) {
            i32x8 bf;
            int sb;
            load_b(j, bf, sb, h);
            f16x8 wb[4];
            nvfp4_frag_f16(bf, sb, wb);
            const int hsel = (kPaired && j >= kNJ / 2) ? 1 : 0;
  #pragma unroll
            for (int mt = 0; mt < kMT; ++mt) {
              const f32x4 pr = mfma_f16_block(xa[mt], wb);
  #pragma unroll
              for (int i = 0; i < 4; ++i) acc[mt][j][i] += pr[i] * sc[hsel][mt][i];
            }
          }
        }
        continue;
      }
      if (kTrans) {
        // kNJ groups of kMT block products; group j - 1 is promoted (FP32
        // multiply-add of the block product into the accumulator) after group
        // j has gone to the matrix cores, so the multiply-adds find their
        // products done
        i32x8 bf[kNJ];
        int sb[kNJ];
  #pragma unroll
        for (int j = 0; j < kNJ; ++j) load_b(j, bf[j], sb[j], h);
        f32x4 pr[2][kMT];
  #pragma unroll
        for (int j = 0; j <= kNJ; ++j) {
          if (j < kNJ) {
  #pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
              pr[j & 1][mt] = kFP4 ? mfma_fp4_fp8(bf[j], sb[j], af[mt]) : mfma_fp8(bf[j], af[mt]);
          }
          if (j > 0) {
            const int jp = j - 1;
            const int hsel = (kPaired && jp >= kNJ / 2) ? 1 : 0;
  #pragma unroll
            for (int mt = 0; mt < kMT; ++mt)
  #pragma unroll
              for (int i = 0; i < 4; ++i) acc[mt][jp][i] += pr[jp & 1][mt][i] * sc[hsel][mt][0];
          }
        }
      } else {
  #pragma unroll
        for (int j = 0; j < kNJ; ++j) {
          i32x8 bf;
          int sb;
          load_b(j, bf, sb, h);
          const int hsel = (kPaired && j >= kNJ / 2) ? 1 : 0;
  #pragma unroll
          for (int mt = 0; mt < kMT; ++mt) {
            const f32x4 pr = kFP4 ? mfma_fp8_fp4(af[mt], bf, sb) : mfma_fp8(af[mt], bf);
  #pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][j][i] += pr[i] * sc[hsel][mt][kTrans ? 0 : i];
          }
        }
      }
     }
    }
  };

  // ---------------------------------------------------------------- epilogues
  // Wave (wm, wn) holds, of the tile's 256 B rows, the kNJ 16-column blocks
  // bblk(j); lane (l16, g) holds rows 16 kMT wm + 16 mt + l16, columns
  // 4 g + i of each block (L1), or rows 16 kMT wm + 16 mt + 4 g + i, column
  // l16 (the others).
  auto epilogue = [&](const Desc& d, uint8_t* sq) {
    if (KIND == TK_L1) {
      // h = silu(gate) * up: the wave's kH 16-column blocks of h, written
      // over the gate accumulators; row amax over the tile's 128 h columns
      // (the 4 lane groups of the row, then all kWavesN waves of the row)
      constexpr int kH = kNJ / 2;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        float m = 0.0f;
#pragma unroll
        for (int j = 0; j < kH; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[mt][j][i] = silu_mul_fast(acc[mt][j][i], acc[mt][kH + j][i]);
            m = fmaxf(m, fabsf(acc[mt][j][i]));
          }
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        if (g == 0) s_amax[wn][16 * kMT * wm + 16 * mt + l16] = m;
      }
      lds_barrier();  // s_amax complete; every wave is done with the stage in sq
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) {
        const int r = 16 * kMT * wm + 16 * mt + l16;
        float amax = s_amax[0][r];
#pragma unroll
        for (int w = 1; w < kWavesN; ++w) amax = fmaxf(amax, s_amax[w][r]);
        const float s = (amax == 0.0f) ? 1.0f : amax / 448.0f;
        const float inv = 1.0f / s;
#pragma unroll
        for (int j = 0; j < kH; ++j) {
          uint32_t q4 = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            q4 |= static_cast<uint32_t>(f32_to_e4m3(acc[mt][j][i] * inv)) << (8 * i);
          *reinterpret_cast<uint32_t*>(sq + r * 128 + 16 * (kH * wn + j) + 4 * g) = q4;
        }
        if (wn == 0 && g == 0 && r < d.rows) p.sh[static_cast<size_t>(d.nt) * n_rows + d.row0 + r] = s;
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < (TM * 8 + 511) / 512; ++i) {
        const int q = tid + 512 * i;
        const int r = q >> 3, c16 = (q & 7) * 16;
        if (r < d.rows)
          *reinterpret_cast<uint4*>(p.hq + static_cast<size_t>(d.row0 + r) * p.half + 128 * d.nt + c16) =
              *reinterpret_cast<const uint4*>(sq + r * 128 + c16);
      }
    } else if (KIND == TK_L2) {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * kMT * wm + 16 * mt + 4 * g + i;
          if (r < d.rows) {
            float* yr = p.y + static_cast<size_t>(d.row0 + r) * p.N + kTN * d.nt + 16 * kNJ * wn + l16;
#pragma unroll
            for (int j = 0; j < kNJ; ++j) yr[16 * j] = acc[mt][j][i];
          }
        }
    } else if (nsplit > 1) {
      // one K range of a split dense tile: FP32 partial sums by B row
      // (k_dense_reduce adds the ranges in order and applies the epilogue)
      float* part = p.partial + static_cast<size_t>(d.kz) * p.M * nbrows;
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * kMT * wm + 16 * mt + 4 * g + i;
          if (r < d.rows) {
            float* pr = part + static_cast<size_t>(d.row0 + r) * nbrows;
#pragma unroll
            for (int j = 0; j < kNJ; ++j) pr[wrow(d.nt, 16 * bblk(j) + l16)] = acc[mt][j][i];
          }
        }
    } else {
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * kMT * wm + 16 * mt + 4 * g + i;
          if (r < d.rows) {
            if (EPI == EPI_SWIGLU) {
#pragma unroll
              for (int j = 0; j < kNJ / 2; ++j)
                dense_epilogue<EPI>(p.ep, p.N, d.row0 + r, 128 * d.nt + 16 * ((kNJ / 2) * wn + j) + l16, acc[mt][j][i],
                                    acc[mt][kNJ / 2 + j][i]);
            } else {
#pragma unroll
              for (int j = 0; j < kNJ; ++j)
                dense_epilogue<EPI>(p.ep, p.N, d.row0 + r, kTN * d.nt + 16 * kNJ * wn + 16 * j + l16, acc[mt][j][i], 0.0f);
            }
          }
        }
    }
  };

  // ---- prologue.  The weight rows of tile 0's first kStages - 1 stages
  // depend only on its expert and n tile, so they are loaded first; then,
  // once tile 0's pair ids and weight scales (direct loads issued before
  // them) have landed, the gathered A rows and the scale words of those
  // stages.  Loads in flight after the A part of stage s: the A parts of the
  // stages after it, then the full stages issued by the loop (ring_barrier
  // counts below).
  constexpr int kS = kStages - 1;        // stages in flight
  constexpr int kA = kLoads - kBChunks;  // A and scale loads per wave and stage
  static_assert(kStages >= 2 && kStages <= 4, "prologue barrier counts");
  Desc dc = desc(0);
  aux(dc, 0);

  // Stage G of the stream is K step G % nk of tile G / nk and sits in ring
  // slot G % kStages.  Step G: wait for stage G (every wave's loads), start
  // stage G + kStages - 1 into the slot that stage G - 1 (read by every wave
  // before the barrier) leaves free, compute stage G; after a tile's last
  // step its epilogue stages the h codes through that step's slot, which
  // the next step's loads only reuse after their barrier.  A tile's pair ids
  // and weight scales are loaded with the first stage of the tile before it;
  // with nk >= kStages - 1 (the launcher's condition) they have landed before
  // their first use and the buffer j % 3 they go to is no longer read.
  Iss is = make_iss(dc, 0);  // (its A offsets are not valid yet)
#pragma unroll
  for (int s = 0; s < kS; ++s) issue(ring + s * kStage, is, s, true, 1);
  vm_wait<kBChunks * kS>();  // this wave's pair-id / weight-scale loads
  lds_barrier();             // every wave's
  is = make_iss(dc, 0);
  if (n_my > 1) aux(desc(1), 1);
#pragma unroll
  for (int s = 0; s < kS; ++s) issue(ring + s * kStage, is, s, true, 2);
  int ji = 0;  // tile of `is`
  const int G = n_my * nk;
  // the stream position the next issue loads: tile ij, K step ik, ring slot
  // islot (counters instead of divisions by nk: they run every step)
  int ij = 0, ik = kS, islot = kS;
  if (ik == nk) {
    ik = 0;
    ij = 1;
  }
  // the next stage to load: its slot, K step and whether it is a real one;
  // a new tile's load offsets and the per-tile data of the tile after it
  // are set up here
  struct Pend {
    uint8_t* st;
    int k;
    bool live;
  };
  auto prep_next = [&]() -> Pend {
    Pend pd{ring + islot * kStage, 0, false};
    if (ij < n_my) {
      if (ik == 0 && ij != ji) {
        is = make_iss(desc(ij), ij % 3);
        ji = ij;
      }
      if (ik == 0 && ij + 1 < n_my) aux(desc(ij + 1), (ij + 1) % 3);
      pd.k = ik;
      pd.live = true;
    }
    if (++ik == nk) {
      ik = 0;
      ++ij;
    }
    if (++islot == kStages) islot = 0;
    return pd;
  };
  // The routed L1's 256-row tiles (one stage in flight) issue their batch
  // spread over the step, one load after each row block's products: issued
  // at once after the barrier, the batch (66 loads per workgroup) queues in
  // the vector memory unit while the waves wait to issue it.  (The same for
  // the routed L2 and the BF16 256-row tiles measured slower: their loads
  // then land too late for the next step.)
  constexpr bool kSpread = KIND == TK_L1 && kMT > 4;
  static_assert(!kSpread || (kKH == 1 && !kASplit && !kNV4 && kLoads >= kMT), "spread batch: one load per row block");
  int j = 0, ks = 0, jb = 0, cslot = 0;  // the computed stage: tile j (buffer jb = j % 3), K step ks, slot
  for (int gg = 0; gg < G; ++gg) {
    if (kStages >= 3 && gg == 0) ring_barrier<kA * (kStages - 2)>();
    else if (kStages >= 4 && gg == 1) ring_barrier<kA * (kStages - 3) + kLoads>();
    else ring_barrier<kLoads * (kStages - 2)>();
    const Pend pd = prep_next();
    if constexpr (!kSpread) issue(pd.st, is, pd.k, pd.live);
    if (ks == 0) {
      if (j > 0) dc = desc(j);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
        for (int jj = 0; jj < kNJ; ++jj) acc[mt][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    uint8_t* st = ring + cslot * kStage;
    compute(st, ks, jb, [&](int q) {
      if constexpr (kSpread)
        if (q < kLoads) issue_one(pd.st, is, pd.k, pd.live, q);
    });
    if constexpr (kSpread) {
#pragma unroll
      for (int q = kMT; q < kLoads; ++q) issue_one(pd.st, is, pd.k, pd.live, q);
    }
    if (ks == nk - 1) epilogue(dc, st);
    if (++ks == nk) {
      ks = 0;
      ++j;
      if (++jb == 3) jb = 0;
    }
    if (++cslot == kStages) cslot = 0;
  }
  // drain the trailing (empty) loads
  ring_barrier<0>();
}

template <int KIND, int FMT, int EPI, int TM = kTM>
__global__ __launch_bounds__(512) void k_tile(TileArgs p) {
  using Lds = TileLds<KIND, FMT, TM>;
  __shared__ __attribute__((aligned(16))) uint8_t ring[Lds::kStages * Lds::kStage];
  __shared__ int s_eoff[Lds::kRouted ? kTileMaxE + 1 : 1];
  __shared__ int s_pre[Lds::kRouted ? kTileMaxE + 1 : 1];
  __shared__ int s_pair[3 * Lds::kPairRows];
  __shared__ float s_wsc[3 * 2 * kMaxKBlocks];
  __shared__ float s_amax[Lds::kWavesN * TM];
  tile_run<KIND, FMT, EPI, TM>(p, TileSmem{ring, s_eoff, s_pre, s_pair, s_wsc, s_amax}, blockIdx.x, gridDim.x);
}

// The 32-row and 64-row tiles of one routed GEMM in one persistent launch:
// each workgroup takes its share of the 32-row tiles, then of the 64-row
// ones (a separate launch for a few hundred 64-row tiles paid its own ramp
// and tail).
template <int KIND, int FMT>
constexpr int small_mid_lds() {
  constexpr int a = TileLds<KIND, FMT, 32>::kBytes, b = TileLds<KIND, FMT, kMidTM>::kBytes;
  return a > b ? a : b;
}

// The 64-row tiles are dealt to the workgroups in reverse order (workgroup
// b takes the share of nwg - 1 - b, on the same XCD as b when nwg is a
// multiple of 8): the workgroups with one 32-row tile more then tend to get
// one 64-row tile less (the 1024-token MXFP4 loads: the busiest workgroup
// 1.09 -> 1.04 times the mean, modelled).
template <int KIND, int FMT>
__global__ __launch_bounds__(512) void k_tile_small_mid(TileArgs p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[small_mid_lds<KIND, FMT>()];
  tile_run<KIND, FMT, 0, 32>(p, tile_smem_in<KIND, FMT, 32>(smem), blockIdx.x, gridDim.x);
  __syncthreads();
  tile_run<KIND, FMT, 0, kMidTM>(p, tile_smem_in<KIND, FMT, kMidTM>(smem), gridDim.x - 1 - blockIdx.x, gridDim.x);
}

}  // namespace moe_tail
