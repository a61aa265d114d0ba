// Host side of the latent-MoE tail library: argument checks, workspace
// layout, launch planning.  Every check runs before the first HIP call, so a
// rejected call enqueues nothing (the pages' "fail closed" rule for
// unsupported layouts and token counts: vLLM PR 53556, "Sequence-parallel
// implementation"; DeepGEMM PR 416 mirror, Compatibility).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/moe_tail.h"
#include "dense_gemm.hpp"
#include "quant_norm.hpp"
#include "route.hpp"
#include "routed_gemm.hpp"
#include "tail_fused.hpp"
#include "tile_gemm.hpp"

using namespace moe_tail;

namespace {

constexpr int32_t kMaxTokens = 1 << 20;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// required pointer: non-null and 16-byte aligned when the tensor is non-empty
bool ptr_ok(const void* p, size_t bytes) { return bytes == 0 || (p != nullptr && aligned16(p)); }

bool is_nvfp4(const moe_tail_dims& d) { return d.wfmt == MOE_TAIL_W_NVFP4 || d.wfmt == MOE_TAIL_W_NVFP4_PACKED; }

int check_dims(const moe_tail_dims* d) {
  if (d == nullptr) return MOE_TAIL_ERR_INVALID;
  if (d->hidden <= 0 || d->latent <= 0 || d->inter <= 0 || d->shared_inter <= 0 || d->num_experts <= 0)
    return MOE_TAIL_ERR_INVALID;
  if (d->top_k < 1 || d->top_k > d->num_experts) return MOE_TAIL_ERR_INVALID;
  if (!(d->rms_eps > 0.0f) || !std::isfinite(d->rms_eps)) return MOE_TAIL_ERR_INVALID;
  if (d->wfmt != MOE_TAIL_W_FP8_BLOCK128 && d->wfmt != MOE_TAIL_W_MXFP4 && d->wfmt != MOE_TAIL_W_MXFP4_PACKED &&
      d->wfmt != MOE_TAIL_W_NVFP4 && d->wfmt != MOE_TAIL_W_NVFP4_PACKED)
    return MOE_TAIL_ERR_UNSUPPORTED;
  if (d->hidden % 256 || d->latent % 256 || d->latent > 256 * kNormMaxCols) return MOE_TAIL_ERR_UNSUPPORTED;
  if (d->inter % 128 || d->shared_inter % 128 || d->inter > 128 * kMaxKBlocks) return MOE_TAIL_ERR_UNSUPPORTED;
  if (d->latent > 128 * kMaxKBlocks) return MOE_TAIL_ERR_UNSUPPORTED;
  if (d->num_experts > 1024 || d->top_k > 16) return MOE_TAIL_ERR_UNSUPPORTED;
  // dense weights are addressed with 32-bit byte offsets
  if (static_cast<int64_t>(d->hidden) * d->latent * 2 >= (1ll << 31) ||
      static_cast<int64_t>(d->hidden) * d->shared_inter * 4 >= (1ll << 31))
    return MOE_TAIL_ERR_UNSUPPORTED;
  return MOE_TAIL_OK;
}

int check_counts(int32_t Mr, int32_t Ms) {
  if (Mr < 0 || Ms < 0 || Mr > Ms || Ms > kMaxTokens) return MOE_TAIL_ERR_INVALID;
  return MOE_TAIL_OK;
}

// Plan of one dense BF16 GEMM.  Up to kSmallMaxM rows: k_dense_small (all
// rows per workgroup, kSkinnyN B rows per workgroup) with K split until the grid
// holds about 256 workgroups, always through FP32 partials.  More rows: the
// LDS-tiled kernel (256- or 128-row tiles, epilogue fused unless K is split).
struct DensePlan {
  bool small;
  int mt, nt, splits, kps;
  int tm;  // tiled: rows per tile (256 or 128)
};

constexpr int kPlanCUs = 256;

DensePlan plan_dense(int M, int nbrows, int ntiles, int K, int cus = kPlanCUs) {
  DensePlan p;
  p.small = M <= kSmallMaxM;
  p.tm = 0;
  const int nk = p.small ? K / 64 : K / 128;  // K steps of the kernel
  int s = 1;
  if (p.small) {
    // about one workgroup per CU of an MI355X (the kernel's LDS ring allows
    // one); a fixed count keeps the workspace size independent of the device
    p.mt = 1;
    p.nt = nbrows / kSkinnyN;
    if (p.nt > 0) s = std::min(nk, std::max(1, cus / p.nt));
  } else {
    // 256-row tiles once they fill 7/8 of the chip (the 2048-row
    // up-projection's 224 tiles: 156 -> 143 us against 448 128-row tiles);
    // else 128-row tiles, and while those fill at most half of it, K split in
    // two more ranges (FP32 partials reduced in split order, as for small M)
    // down to 16 K steps a range (the 1024-token shared L1: 128 tiles of 112
    // K steps, split in 2)
    p.nt = ntiles;
    const bool huge = static_cast<long>((M + kHugeTM - 1) / kHugeTM) * ntiles * 8 >= 7L * cus;
    p.tm = huge ? kHugeTM : kTM;
    p.mt = (M + p.tm - 1) / p.tm;
    const int steps = K / 64;  // 64-wide BF16 K steps of the tiled kernel
    if (!huge)
      while (static_cast<long>(p.mt) * p.nt * s * 2 <= cus && steps % (2 * s) == 0 && steps / (2 * s) >= 16) s *= 2;
    p.kps = steps / s;
    p.splits = s;
    return p;
  }
  p.kps = (nk + s - 1) / s;
  p.splits = (nk + p.kps - 1) / p.kps;
  return p;
}

struct Plans {
  DensePlan s1, s2, up;
};

Plans plan_all(const moe_tail_dims& d, int32_t Mr, int32_t Ms) {
  Plans p;
  // at decode sizes the shared L2 and the up-projection share one launch,
  // each on its share of the workgroups (fewer, longer items than one
  // launch each would take, and fewer partial sums to write and reduce).
  // The shared expert's plan depends on Ms and the widths only, so its rows
  // come out the same whatever Mr is.
  const int pair = Ms <= kSmallMaxM ? 2 : 1;
  // (tiles of the tiled kernel: 128 gate + 128 up rows, or 256 rows)
  // (at decode sizes the shared L1's items fill the routed L2 launch's
  // ragged end: half as many K splits as one launch of its own would take,
  // half the FP32 partials to write there and to read back in the combine
  // launch; decode 351.4 -> 346.8 us)
  p.s1 = plan_dense(Ms, 2 * d.shared_inter, d.shared_inter / 128, d.hidden, pair == 2 ? kPlanCUs / 2 : kPlanCUs);
  if (pair == 2) {
    // The two share one launch, which ends with its longest item: the
    // workgroups are split between them so that the larger per-item K range
    // is as short as it can be (both have H / kSkinnyN weight-row blocks, so
    // an item's bytes follow its K range), the fewest items among equals.
    // Decode (I_s = 2048, L = 3584): 2 + 2 splits; 16 tokens with I_s = 512:
    // 1 + 3 instead of 2 + 2 (the up-projection items 448 -> 304 KB).
    const int nt = d.hidden / kSkinnyN, n2 = d.shared_inter / 64, nu = d.latent / 64;
    const int total = std::max(2, kPlanCUs / std::max(1, nt));
    int best_a = 1, best_b = 1;
    long best = -1;
    for (int a = 1; a < total && a <= n2; ++a)
      for (int b = 1; a + b <= total && b <= nu; ++b) {
        const long cost = static_cast<long>(std::max((n2 + a - 1) / a, (nu + b - 1) / b)) * 4096 + a + b;
        if (best < 0 || cost < best) {
          best = cost;
          best_a = a;
          best_b = b;
        }
      }
    p.s2 = plan_dense(Ms, d.hidden, d.hidden / kTN, d.shared_inter, best_a * nt);
    p.up = plan_dense(Mr, d.hidden, d.hidden / kTN, d.latent, best_b * nt);
  } else {
    p.s2 = plan_dense(Ms, d.hidden, d.hidden / kTN, d.shared_inter);
    p.up = plan_dense(Mr, d.hidden, d.hidden / kTN, d.latent);
  }
  return p;
}

// Small M with as many shared as routed tokens: the shared L2's split-K
// reduction is folded into the up-projection's (one launch less), which
// then also stores s.
bool fuse_shared_reduce(const Plans& p, int32_t Mr, int32_t Ms) { return Mr > 0 && Ms == Mr && p.s2.small && p.up.small; }

// Shapes of the routed tiled kernel: expert tables in LDS (E <= kTileMaxE),
// gathered x rows addressed with 32-bit offsets, a tile's side data loaded
// kStages - 1 steps ahead (K >= 384 for L1 and L2; MXFP4 and NVFP4, whose
// small tiles take two 128-wide K blocks per step: K a multiple of 256, at
// least 512).
bool tiled_ok(const moe_tail_dims& d, int32_t Mr) {
  const bool fp4_ok = d.wfmt == MOE_TAIL_W_FP8_BLOCK128 ||
                      (d.latent % 256 == 0 && d.inter % 256 == 0 && d.latent >= 512 && d.inter >= 512);
  return d.num_experts <= kTileMaxE && static_cast<size_t>(Mr) * d.latent < (1ull << 31) && d.latent >= 384 &&
         d.inter >= 384 && fp4_ok;
}

// The single-launch tail covers decode sizes: every dense GEMM on the
// small-M kernel (Ms <= 128) and every expert on 32-row tiles.
bool fused_ok(const moe_tail_dims& d, const Plans& p, int32_t Mr, int32_t Ms) {
  return Mr > 0 && Ms <= kSmallMaxM && p.s1.small && p.s2.small && p.up.small && tiled_ok(d, Mr);
}

struct Layout {
  size_t logits, hist;                              // routing scratch
  size_t xq, sx, sxr, hq, sh, y, rn, hs, s, partial;  // forward intermediates
  size_t partial_s;                                 // the shared L2's partials when a later step reduces them
  size_t sync;                                      // completion counters of the single-launch tail
  size_t sync_bytes;
  size_t total;
};

Layout layout_of(const moe_tail_dims& d, int32_t Mr, int32_t Ms) {
  const size_t L = d.latent, H = d.hidden, I = d.inter, Is = d.shared_inter, E = d.num_experts, k = d.top_k;
  const size_t R = static_cast<size_t>(Mr) * k;
  const size_t ng = (static_cast<size_t>(Mr) + kGroup - 1) / kGroup;
  const Plans p = plan_all(d, Mr, Ms);
  size_t partial = 0;
  auto need = [](const DensePlan& q) { return q.small || q.splits > 1; };
  if (need(p.s1)) partial = std::max(partial, static_cast<size_t>(p.s1.splits) * Ms * 2 * Is * 4);
  if (need(p.s2)) partial = std::max(partial, static_cast<size_t>(p.s2.splits) * Ms * H * 4);
  if (need(p.up)) partial = std::max(partial, static_cast<size_t>(p.up.splits) * Mr * H * 4);
  Layout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align_up(bytes);
    return at;
  };
  l.logits = take(static_cast<size_t>(Mr) * E * 4);
  l.hist = take(E * ng * 4);
  l.xq = take(static_cast<size_t>(Mr) * L);
  l.sx = take(static_cast<size_t>(Mr) * (L / 128) * 4);
  l.sxr = take(R * (L / 128) * 4);  // sx per routed row, K-block-major (RowScales)
  l.hq = take(R * I);
  l.sh = take(R * (I / 128) * 4);
  l.y = take(R * L * 4);
  l.rn = take(static_cast<size_t>(Mr) * L * 2);
  l.hs = take(static_cast<size_t>(Ms) * Is * 2);
  l.s = take(static_cast<size_t>(Mr) * H * 2);
  l.partial = take(partial);
  const bool keep_s2 = fuse_shared_reduce(p, Mr, Ms) || fused_ok(d, p, Mr, Ms);
  l.partial_s = take(keep_s2 ? static_cast<size_t>(p.s2.splits) * Ms * H * 4 : 0);
  l.sync_bytes = fused_ok(d, p, Mr, Ms) ? kSyncWords * 4 : 0;
  l.sync = take(l.sync_bytes);
  l.total = o;
  return l;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int launched() { return hipGetLastError() == hipSuccess ? MOE_TAIL_OK : MOE_TAIL_ERR_DEVICE; }

// The x quantizer's second copy of the scales, by routed row (read by the
// tiled routed L1)
RowScales row_scales(const moe_tail_dims& d, const Layout& lay, void* ws, const moe_tail_routing* routing, int32_t Mr) {
  RowScales rs{};
  rs.pair_to_row = routing->pair_to_row;
  rs.out = at<float>(ws, lay.sxr);
  rs.k = d.top_k;
  rs.nkb = d.latent / 128;
  rs.R = static_cast<long>(Mr) * d.top_k;
  return rs;
}

int check_weights(const moe_tail_dims& d, const moe_tail_weights* w, bool need_router, bool need_routed,
                  bool need_shared, bool need_up) {
  if (w == nullptr) return MOE_TAIL_ERR_INVALID;
  const size_t E = d.num_experts, L = d.latent, H = d.hidden, I = d.inter, Is = d.shared_inter;
  if (need_router) {
    if (!ptr_ok(w->gate, E * L * 4)) return MOE_TAIL_ERR_INVALID;
    if (w->gate_bias != nullptr && !aligned16(w->gate_bias)) return MOE_TAIL_ERR_INVALID;
  }
  if (need_routed) {
    if (!ptr_ok(w->w1, 1) || !ptr_ok(w->w1_scale, 1) || !ptr_ok(w->w2, 1) || !ptr_ok(w->w2_scale, 1))
      return MOE_TAIL_ERR_INVALID;
    if (!ptr_ok(w->rms_gamma, L * 2)) return MOE_TAIL_ERR_INVALID;
    if (is_nvfp4(d) && (!ptr_ok(w->w1_tensor_scale, E * 4) || !ptr_ok(w->w2_tensor_scale, E * 4)))
      return MOE_TAIL_ERR_INVALID;
  }
  if (need_shared && (!ptr_ok(w->ws1, 2 * Is * H * 2) || !ptr_ok(w->ws2, H * Is * 2))) return MOE_TAIL_ERR_INVALID;
  if (need_up && !ptr_ok(w->w_up, H * L * 2)) return MOE_TAIL_ERR_INVALID;
  (void)I;
  return MOE_TAIL_OK;
}

int check_routing(const moe_tail_routing* r, int32_t Mr, int k, int E) {
  if (r == nullptr) return MOE_TAIL_ERR_INVALID;
  const size_t R = static_cast<size_t>(Mr) * k;
  if (!ptr_ok(r->topk_ids, R * 4) || !ptr_ok(r->topk_weights, R * 4) || !ptr_ok(r->sorted_pair, R * 4) ||
      !ptr_ok(r->pair_to_row, R * 4) || !ptr_ok(r->expert_offsets, static_cast<size_t>(E + 1) * 4))
    return MOE_TAIL_ERR_INVALID;
  return MOE_TAIL_OK;
}

// Compute units of the current device (cached per device).
unsigned num_cus() {
  static unsigned cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = static_cast<unsigned>(n);
  }
  return cache[dev];
}

// Workgroups of a persistent launch: one per CU (the tiled kernels' LDS
// allows no second), whole rounds of 8 so that every XCD gets the same
// number; `share` > 0 caps them at that many CUs (a multiple of 8), the
// rest of the chip running a concurrent launch.
unsigned persistent_wgs(unsigned share) {
  const unsigned all = std::max(8u, num_cus() / 8 * 8);
  return share > 0 ? std::min(all, share) : all;
}

template <int KIND, int FMT, int EPI, int TM = kTM>
void launch_tile(const TileArgs& a, hipStream_t st, unsigned share = 0) {
  const unsigned T = static_cast<unsigned>(a.nslots) * static_cast<unsigned>(a.ntn) *
                     static_cast<unsigned>(KIND == TK_DENSE && a.ksplit > 1 ? a.ksplit : 1);
  if (T == 0) return;
  const unsigned wg = std::min((T + 7) / 8 * 8, persistent_wgs(share));
  hipLaunchKernelGGL((k_tile<KIND, FMT, EPI, TM>), dim3(wg), dim3(512), 0, st, a);
}

// The 32-row and 64-row tiles in one persistent launch (one workgroup per CU)
template <int KIND, int FMT>
void launch_small_mid(const TileArgs& a, hipStream_t st, unsigned share = 0) {
  hipLaunchKernelGGL((k_tile_small_mid<KIND, FMT>), dim3(persistent_wgs(share)), dim3(512), 0, st, a);
}

// A second stream of the calling host thread on the current device, with the
// two events that fork work onto it from a caller's stream and join it back
// (created on first use at the default priority and kept until the process
// ends; one per host thread, so that concurrent callers never share events).
struct SideStream {
  hipStream_t s;
  hipEvent_t fork, join;
};
const SideStream* side_stream() {
  thread_local SideStream cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  SideStream& c = cache[dev];
  if (c.s == nullptr) {
    SideStream n{};
    if (hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&n.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&n.join, hipEventDisableTiming) != hipSuccess) {
      (void)hipStreamDestroy(n.s);
      return nullptr;
    }
    c = n;
  }
  return &c;
}

template <int kEpi>
void launch_dense(const DensePlan& p, const uint16_t* A, const uint16_t* B, int M, int N, int K, float* partial,
                  const DenseEpi& ep, hipStream_t st, bool reduce = true, unsigned share = 0) {
  if (M == 0) return;
  const int nbrows = (kEpi == EPI_SWIGLU) ? 2 * ep.half : N;
  if (p.small) {
    hipLaunchKernelGGL(k_dense_small<>, dim3(p.nt, p.splits), dim3(512), 0, st, A, B, M, nbrows, K, p.kps, partial);
    if (!reduce) return;  // the partials are reduced by a later launch
    const int ncols = (kEpi == EPI_SWIGLU) ? ep.half : N;
    const long n = static_cast<long>(M) * (ncols / 4);
    hipLaunchKernelGGL(k_dense_reduce<kEpi>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                       partial, M, N, p.splits, ep);
    return;
  }
  TileArgs a{};
  a.a = reinterpret_cast<const uint8_t*>(A);
  a.b = reinterpret_cast<const uint8_t*>(B);
  a.ep = ep;
  a.M = M;
  a.K = K;
  a.N = N;
  a.half = ep.half;
  a.ntn = (kEpi == EPI_SWIGLU) ? ep.half / 128 : N / kTN;
  a.nslots = p.mt;
  a.ksplit = p.splits;
  a.partial = p.splits > 1 ? partial : nullptr;
  if (p.tm == kHugeTM) launch_tile<TK_DENSE, TF_BF16, kEpi, kHugeTM>(a, st, share);
  else launch_tile<TK_DENSE, TF_BF16, kEpi>(a, st, share);
  if (p.splits > 1) {
    const int ncols = (kEpi == EPI_SWIGLU) ? ep.half : N;
    const long n = static_cast<long>(M) * (ncols / 4);
    hipLaunchKernelGGL(k_dense_reduce<kEpi>, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st,
                       partial, M, N, p.splits, ep);
  }
}

// Arguments of the decode-sized kernels (the single-launch tail and the
// co-scheduled launches share them).
FusedArgs fused_args(const moe_tail_dims& d, const moe_tail_weights* w, int32_t Mr, const uint16_t* x_hid, int32_t Ms,
                     const moe_tail_routing* routing, const uint16_t* residual, uint16_t* out, uint16_t* shared_out,
                     void* ws, const Layout& lay, const Plans& plans) {
  const int L = d.latent, H = d.hidden, I = d.inter, Is = d.shared_inter, E = d.num_experts, k = d.top_k;
  FusedArgs f{};
  TileArgs ta{};
  ta.sorted_pair = routing->sorted_pair;
  ta.expert_offsets = routing->expert_offsets;
  ta.E = E;
  ta.k = k;
  ta.big_rows = 0x7fffffff;
  ta.huge_rows = 0x7fffffff;
  ta.mid_rows = 0x7fffffff;
  ta.scales_packed = d.wfmt == MOE_TAIL_W_MXFP4_PACKED || d.wfmt == MOE_TAIL_W_NVFP4_PACKED;
  f.l1 = ta;
  f.l1.a = at<uint8_t>(ws, lay.xq);
  f.l1.a_scale = at<float>(ws, lay.sxr);
  f.l1.M = Mr;
  f.l1.b = w->w1;
  f.l1.b_scale = w->w1_scale;
  f.l1.b_tscale = w->w1_tensor_scale;
  f.l1.hq = at<uint8_t>(ws, lay.hq);
  f.l1.sh = at<float>(ws, lay.sh);
  f.l1.K = L;
  f.l1.N = 2 * I;
  f.l1.half = I;
  f.l1.ntn = I / 128;
  f.l1.nslots = static_cast<int>(static_cast<size_t>(Mr) * k / 32 + E);  // bound on the row tiles (grid size)
  f.l2 = ta;
  f.l2.a = at<uint8_t>(ws, lay.hq);
  f.l2.a_scale = at<float>(ws, lay.sh);
  f.l2.b = w->w2;
  f.l2.b_scale = w->w2_scale;
  f.l2.b_tscale = w->w2_tensor_scale;
  f.l2.y = at<float>(ws, lay.y);
  f.l2.K = I;
  f.l2.N = L;
  f.l2.half = 0;
  f.l2.ntn = L / kTN;
  f.x_hid = x_hid;
  f.ws1 = w->ws1;
  f.ws2 = w->ws2;
  f.w_up = w->w_up;
  f.Mr = Mr;
  f.Ms = Ms;
  f.H = H;
  f.Is = Is;
  f.L = L;
  f.k = k;
  f.s1 = DenseItems{plans.s1.nt, plans.s1.splits, plans.s1.kps};
  f.s2 = DenseItems{plans.s2.nt, plans.s2.splits, plans.s2.kps};
  f.up = DenseItems{plans.up.nt, plans.up.splits, plans.up.kps};
  f.part_s1 = at<float>(ws, lay.partial);
  f.part_s2 = at<float>(ws, lay.partial_s);
  f.part_up = at<float>(ws, lay.partial);
  f.hs = at<uint16_t>(ws, lay.hs);
  f.y = at<float>(ws, lay.y);
  f.topk_w = routing->topk_weights;
  f.pair_to_row = routing->pair_to_row;
  f.gamma = w->rms_gamma;
  f.rn = at<uint16_t>(ws, lay.rn);
  f.eps = d.rms_eps;
  f.out = out;
  f.s = at<uint16_t>(ws, lay.s);
  f.shared_out = shared_out;
  f.resid = residual;
  f.sync = at<int>(ws, lay.sync);
  f.max_polls = kSpinLimit;
  return f;
}

// The host checks every forward entry point makes (before anything is
// enqueued); fills *lay on success.
int check_forward(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
                  const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing, const uint16_t* residual,
                  uint16_t* out, uint16_t* shared_out, void* ws, size_t ws_bytes, Layout* lay) {
  int rc = check_dims(dims);
  if (rc) return rc;
  rc = check_counts(Mr, Ms);
  if (rc) return rc;
  const moe_tail_dims& d = *dims;
  const int L = d.latent, H = d.hidden, E = d.num_experts, k = d.top_k;
  rc = check_weights(d, w, false, Mr > 0, Ms > 0, Mr > 0);
  if (rc) return rc;
  if (Mr > 0 && (rc = check_routing(routing, Mr, k, E))) return rc;
  if (!ptr_ok(x_lat, static_cast<size_t>(Mr) * L * 2) || !ptr_ok(x_hid, static_cast<size_t>(Ms) * H * 2) ||
      !ptr_ok(out, static_cast<size_t>(Mr) * H * 2))
    return MOE_TAIL_ERR_INVALID;
  if (residual != nullptr && !ptr_ok(residual, static_cast<size_t>(Mr) * H * 2)) return MOE_TAIL_ERR_INVALID;
  if ((Ms > Mr) != (shared_out != nullptr)) return MOE_TAIL_ERR_INVALID;
  if (shared_out != nullptr && !aligned16(shared_out)) return MOE_TAIL_ERR_INVALID;
  // packed MXFP4 scales are read by the tiled kernels only
  if ((d.wfmt == MOE_TAIL_W_MXFP4_PACKED || d.wfmt == MOE_TAIL_W_NVFP4_PACKED) && !tiled_ok(d, Mr))
    return MOE_TAIL_ERR_UNSUPPORTED;
  *lay = layout_of(d, Mr, Ms);
  if (ws_bytes < lay->total) return MOE_TAIL_ERR_WORKSPACE;
  if (lay->total > 0 && !ptr_ok(ws, 1)) return MOE_TAIL_ERR_INVALID;
  return MOE_TAIL_OK;
}

// Event modes of forward_impl: none; one launch per stage with an event
// before each stage (moe_tail_forward_profiled); the schedule moe_tail_forward
// runs with an event before each of its launch groups (moe_tail_forward_timed).
enum { EV_NONE = 0, EV_PER_STAGE = 1, EV_SCHEDULE = 2 };

// Launch groups of the schedule moe_tail_forward runs for these sizes.
const char* const kStagedNames[MOE_TAIL_NUM_STAGES] = {"quant_x", "routed_l1", "routed_l2", "combine_rmsnorm",
                                                       "shared_l1", "shared_l2", "up_proj_add"};
const char* const kDecodeNames[6] = {"quant_x",          "routed_l1",
                                     "routed_l2+shared_l1", "combine_rmsnorm+shared_l1_reduce",
                                     "shared_l2+up_proj", "final_join"};

int forward_impl(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
                 const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing, const uint16_t* residual,
                 uint16_t* out, uint16_t* shared_out, void* ws, size_t ws_bytes, void* stream, void* const* events,
                 int ev_mode = EV_NONE, bool side_ok = true) {
  Layout lay;
  int rc = check_forward(dims, w, x_lat, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, ws_bytes, &lay);
  if (rc) return rc;
  const moe_tail_dims& d = *dims;
  const int L = d.latent, H = d.hidden, I = d.inter, Is = d.shared_inter, E = d.num_experts, k = d.top_k;
  if (events != nullptr)
    for (int i = 0; i <= MOE_TAIL_NUM_STAGES; ++i)
      if (events[i] == nullptr) return MOE_TAIL_ERR_INVALID;

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // launch errors below are ours, not an earlier call's
  auto mark = [&](int i) {
    if (events) (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), st);
  };
  const Plans plans = plan_all(d, Mr, Ms);
  const size_t R = static_cast<size_t>(Mr) * k;
  uint8_t* xq = at<uint8_t>(ws, lay.xq);
  float* sx = at<float>(ws, lay.sx);
  uint8_t* hq = at<uint8_t>(ws, lay.hq);
  float* sh = at<float>(ws, lay.sh);
  float* y = at<float>(ws, lay.y);
  uint16_t* rn = at<uint16_t>(ws, lay.rn);
  uint16_t* hs = at<uint16_t>(ws, lay.hs);
  uint16_t* s = at<uint16_t>(ws, lay.s);
  float* partial = at<float>(ws, lay.partial);

  // Decode sizes (every dense GEMM small-M, every expert on 32-row tiles):
  // six launches, independent work sharing a launch (the profiled variant
  // keeps one launch per stage so that each stage can be timed)
  if (ev_mode != EV_PER_STAGE && fused_ok(d, plans, Mr, Ms)) {
    const FusedArgs f = fused_args(d, w, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, lay, plans);
    const bool fp8 = d.wfmt == MOE_TAIL_W_FP8_BLOCK128, nv4 = is_nvfp4(d);
    const long qblocks = static_cast<long>(Mr) * (L / 128);
    mark(0);
    hipLaunchKernelGGL(k_quant_clear, dim3(quant_grid(qblocks)), dim3(256), 0, st, x_lat, xq, sx, qblocks, f.sync,
                       kSyncWords, row_scales(d, lay, ws, routing, Mr));
    mark(1);
    if (fp8) launch_tile<TK_L1, TF_FP8, 0, 32>(f.l1, st);
    else if (nv4) launch_tile<TK_L1, TF_NV4, 0, 32>(f.l1, st);
    else launch_tile<TK_L1, TF_FP4, 0, 32>(f.l1, st);
    mark(2);
    const unsigned pgrid = std::max(8u, num_cus() / 8 * 8);  // persistent: one workgroup per CU
    if (fp8) hipLaunchKernelGGL(k_l2_shared1<TF_FP8>, dim3(pgrid), dim3(512), 0, st, f);
    else if (nv4) hipLaunchKernelGGL(k_l2_shared1<TF_NV4>, dim3(pgrid), dim3(512), 0, st, f);
    else hipLaunchKernelGGL(k_l2_shared1<TF_FP4>, dim3(pgrid), dim3(512), 0, st, f);
    mark(3);
    const long r_groups = static_cast<long>(Ms) * (Is / 4);
    const unsigned cgrid = static_cast<unsigned>(Mr + (r_groups + 255) / 256);
    const int nc4 = (L / 4 + 255) / 256;
    auto kc = (nc4 <= 2) ? k_combine_shared1r<2> : (nc4 <= 4) ? k_combine_shared1r<4> : k_combine_shared1r<8>;
    hipLaunchKernelGGL(kc, dim3(cgrid), dim3(256), 0, st, f);
    mark(4);
    const unsigned dgrid = static_cast<unsigned>(plans.s2.nt * plans.s2.splits + plans.up.nt * plans.up.splits);
    hipLaunchKernelGGL(k_shared2_up, dim3(dgrid), dim3(512), 0, st, f);
    mark(5);
    const long f_groups = static_cast<long>(Ms) * (H / 4);
    hipLaunchKernelGGL(k_final_join, dim3(static_cast<unsigned>((f_groups + 255) / 256)), dim3(256), 0, st, f);
    for (int i = 6; i <= MOE_TAIL_NUM_STAGES; ++i) mark(i);
    return launched();
  }

  // 1, 2: routed L1 and L2 on the persistent LDS-tiled kernel: FP8 128-row
  // tiles for experts with at least kBigMinRows rows (256-row tiles from 256
  // rows on, the rows past them in one 128-row tile when at most 128), 32-row
  // tiles for the others;
  // up to kSmallOnlyMr tokens every expert takes 32-row tiles (an expert
  // reaching 128 rows is then rare, and it saves the second launch).  When
  // the experts average more than 32 rows, those with 33 .. 127 take 64-row
  // tiles instead (two 32-row tiles of one expert stream the same weights
  // side by side, which halves the distinct weight streams in flight).  The
  // kernel keeps the expert tables in LDS (E <= kTileMaxE), addresses the
  // gathered x rows with 32-bit offsets and loads a tile's side data
  // kStages - 1 >= 3 steps ahead (K >= 384).  Shapes outside that take the
  // row-streaming kernel for every expert.
  const bool tiled = tiled_ok(d, Mr);
  constexpr int kSmallOnlyMr = 256;
  const bool fp8 = d.wfmt == MOE_TAIL_W_FP8_BLOCK128;
  const bool nvfp4 = is_nvfp4(d);
  // 128- and 256-row tiles for FP8 only.  A 256-row MXFP4 tile fits one
  // 128-wide K block per step (half-line weight loads) and a 128-row one a
  // single stage in flight; MXFP4 experts with 33 rows or more take 64-row
  // tiles (three two-block stages) instead (the 1024-token MXFP4 workload:
  // 923 -> 866 us on 128-row tiles, 851-859 us on 64-row ones).  NVFP4
  // takes 32-row tiles for every expert (its block scales leave no room for
  // a 64-row tile's three stages).
  const bool big = tiled && Mr > kSmallOnlyMr && fp8;
  const bool mid = tiled && !nvfp4 && (R > static_cast<size_t>(32) * E || (!fp8 && Mr > kSmallOnlyMr));
  // The shared expert on a second stream, beside the routed work: with FP8
  // weights and the experts averaging at most 64 rows (32/64-row tiles) the
  // routed GEMMs stream weights and keep HBM busy from fewer CUs (the
  // 2048-token, 384-expert workload's routed L1 + L2: 1580 us on 256 CUs,
  // 1726 on 192, 1923 on 160), while the shared L1 and L2 are bound by the
  // matrix cores of the CUs they run on.  So the routed launches take 10/16
  // of the CUs and the shared L1 and L2 the rest, concurrently; the
  // up-projection, which needs both, runs after the join on the whole chip.
  // Every tile computes what it computes in one stream, so the result is the
  // same bit for bit.  (That workload: 2571 -> 2475 us.  The shared GEMMs
  // then run 1.3-1.4 times slower than their share of the CUs predicts,
  // their one-stage 256-row tiles waiting longer for loads beside the routed
  // stream; 80, 104 or 112 CUs for them, or 128-row tiles, measured slower.)
  const SideStream* side = nullptr;
  unsigned r_share = 0, d_share = 0;
  if (side_ok && ev_mode == EV_NONE && Mr > 0 && fp8 && mid && R <= static_cast<size_t>(64) * E && Ms >= 2 * Mr &&
      !plans.s1.small && !plans.s2.small && (side = side_stream()) != nullptr) {
    const unsigned cus = persistent_wgs(0);
    d_share = std::max(8u, cus * 6 / 16 / 8 * 8);
    r_share = cus - d_share;
    if (r_share < 8 || hipEventRecord(side->fork, st) != hipSuccess ||
        hipStreamWaitEvent(side->s, side->fork, 0) != hipSuccess)
      side = nullptr;
  }
  const bool fuse_s = fuse_shared_reduce(plans, Mr, Ms);
  float* partial_s = at<float>(ws, lay.partial_s);
  // 4: shared L1 + SwiGLU, 5: shared L2 -> s (rows < Mr) and shared_out
  // (rows >= Mr), on `sst`
  auto shared_l1_l2 = [&](hipStream_t sst, unsigned share) {
    mark(4);
    {
      DenseEpi ep{Mr, Is, hs, nullptr, nullptr, nullptr};
      launch_dense<EPI_SWIGLU>(plans.s1, x_hid, w->ws1, Ms, Is, H, partial, ep, sst, true, share);
    }
    mark(5);
    DenseEpi ep{Mr, Is, s, shared_out, nullptr, nullptr};
    if (fuse_s) launch_dense<EPI_SHARED>(plans.s2, hs, w->ws2, Ms, H, Is, partial_s, ep, sst, false, share);
    else launch_dense<EPI_SHARED>(plans.s2, hs, w->ws2, Ms, H, Is, partial, ep, sst, true, share);
  };
  if (side != nullptr) {
    shared_l1_l2(side->s, d_share);
    if (hipEventRecord(side->join, side->s) != hipSuccess) return MOE_TAIL_ERR_DEVICE;
  }

  // 0: quantize x_lat
  mark(0);
  if (Mr > 0) {
    const long blocks = static_cast<long>(Mr) * (L / 128);
    hipLaunchKernelGGL(k_quant_1x128<true>, dim3(quant_grid(blocks)), dim3(256), 0, st, x_lat, xq, sx, blocks,
                       tiled_ok(d, Mr) ? row_scales(d, lay, ws, routing, Mr) : RowScales{});
  }
  const unsigned max_tiles = static_cast<unsigned>((R + kBM - 1) / kBM + E);
  TileArgs ta{};
  ta.sorted_pair = routing ? routing->sorted_pair : nullptr;
  ta.expert_offsets = routing ? routing->expert_offsets : nullptr;
  ta.E = E;
  ta.k = k;
  ta.scales_packed = d.wfmt == MOE_TAIL_W_MXFP4_PACKED || d.wfmt == MOE_TAIL_W_NVFP4_PACKED;
  ta.big_rows = big ? kBigMinRows : 0x7fffffff;
  ta.huge_rows = big ? kHugeTM : 0x7fffffff;
  ta.mid_rows = mid ? 33 : 0x7fffffff;
  // bounds on the row tiles, which size the grids: ceil(c / 128) <= c / 64
  // for c >= 128, and ceil(c / 32) <= c / 32 + 1 (the launch of the 32- and
  // 64-row tiles together takes one workgroup per CU)
  const int slots_big = static_cast<int>(R / (kTM / 2));
  const int slots_huge = static_cast<int>(R / (kHugeTM / 2));  // ceil(c / 256) <= c / 128 for c >= 256
  const int slots_small = static_cast<int>(R / 32 + E);
  mark(1);
  if (Mr > 0) {
    if (!tiled) {
      auto kl1 = fp8 ? k_routed_l1<FMT_FP8> : nvfp4 ? k_routed_l1<FMT_NVFP4> : k_routed_l1<FMT_MXFP4>;
      hipLaunchKernelGGL(kl1, dim3(max_tiles, I / 128), dim3(256), 0, st, xq, sx, routing->sorted_pair,
                         routing->expert_offsets, w->w1, w->w1_scale, w->w1_tensor_scale, hq, sh, E, k, L, I,
                         0x7fffffff);
    } else {
      TileArgs a1 = ta;
      a1.a = xq;
      a1.a_scale = at<float>(ws, lay.sxr);
      a1.M = Mr;
      a1.b = w->w1;
      a1.b_scale = w->w1_scale;
      a1.b_tscale = w->w1_tensor_scale;
      a1.hq = hq;
      a1.sh = sh;
      a1.K = L;
      a1.N = 2 * I;
      a1.half = I;
      a1.ntn = I / 128;
      a1.nslots = slots_small;
      if (mid) {
        if (fp8) launch_small_mid<TK_L1, TF_FP8>(a1, st, r_share);
        else launch_small_mid<TK_L1, TF_FP4>(a1, st, r_share);
      } else {
        if (fp8) launch_tile<TK_L1, TF_FP8, 0, 32>(a1, st);
        else if (nvfp4) launch_tile<TK_L1, TF_NV4, 0, 32>(a1, st);
        else launch_tile<TK_L1, TF_FP4, 0, 32>(a1, st);
      }
      if (big) {
        a1.nslots = slots_big;
        launch_tile<TK_L1, TF_FP8, 0>(a1, st, r_share);
        a1.nslots = slots_huge;
        launch_tile<TK_L1, TF_FP8, 0, kHugeTM>(a1, st, r_share);
      }
    }
  }
  mark(2);
  if (Mr > 0) {
    if (!tiled) {
      auto kl2 = fp8 ? k_routed_l2<FMT_FP8> : nvfp4 ? k_routed_l2<FMT_NVFP4> : k_routed_l2<FMT_MXFP4>;
      hipLaunchKernelGGL(kl2, dim3(max_tiles, L / 128), dim3(256), 0, st, hq, sh, routing->expert_offsets, w->w2,
                         w->w2_scale, w->w2_tensor_scale, y, E, L, I, 0x7fffffff);
    } else {
      TileArgs a2 = ta;
      a2.a = hq;
      a2.a_scale = sh;
      a2.b = w->w2;
      a2.b_scale = w->w2_scale;
      a2.b_tscale = w->w2_tensor_scale;
      a2.y = y;
      a2.K = I;
      a2.N = L;
      a2.half = 0;
      a2.ntn = L / kTN;
      a2.nslots = slots_small;
      if (mid) {
        if (fp8) launch_small_mid<TK_L2, TF_FP8>(a2, st, r_share);
        else launch_small_mid<TK_L2, TF_FP4>(a2, st, r_share);
      } else {
        if (fp8) launch_tile<TK_L2, TF_FP8, 0, 32>(a2, st);
        else if (nvfp4) launch_tile<TK_L2, TF_NV4, 0, 32>(a2, st);
        else launch_tile<TK_L2, TF_FP4, 0, 32>(a2, st);
      }
      if (big) {
        a2.nslots = slots_big;
        launch_tile<TK_L2, TF_FP8, 0>(a2, st, r_share);
        a2.nslots = slots_huge;
        launch_tile<TK_L2, TF_FP8, 0, kHugeTM>(a2, st, r_share);
      }
    }
  }
  // 3: combine + RMSNorm
  mark(3);
  if (Mr > 0) {
    const int nc4 = (L / 4 + 255) / 256;  // 4-column groups per thread
    auto kern = (nc4 <= 2) ? k_combine_rmsnorm<2> : (nc4 <= 4) ? k_combine_rmsnorm<4> : k_combine_rmsnorm<8>;
    hipLaunchKernelGGL(kern, dim3(Mr), dim3(256), 0, st, y, routing->topk_weights, routing->pair_to_row,
                       w->rms_gamma, rn, L, k, d.rms_eps);
  }
  // 4, 5: shared L1 and L2 (already on the second stream, or here)
  if (side == nullptr) shared_l1_l2(st, 0);
  else if (hipStreamWaitEvent(st, side->join, 0) != hipSuccess) return MOE_TAIL_ERR_DEVICE;
  // 6: up-projection + FP32 shared add (+ FP32 residual add)
  mark(6);
  {
    DenseEpi ep{Mr, Is, out, nullptr, s, residual};
    if (fuse_s) {
      ep.out1 = s;
      ep.s_partial = partial_s;
      ep.s_splits = plans.s2.splits;
    }
    launch_dense<EPI_UPADD>(plans.up, rn, w->w_up, Mr, H, L, partial, ep, st);
  }
  mark(7);
  return launched();
}

// Workgroups of the single-launch tail: one per CU, whole rounds of 8 (one
// per XCD), provided the kernel fits one workgroup per CU at all.
template <int FMT>
unsigned fused_grid() {
  static int fits[64] = {};  // per device: 0 unknown, 1 yes, 2 no
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (fits[dev] == 0) {
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(k_tail_small<FMT>), 512, 0);
    fits[dev] = (e == hipSuccess && n >= 1) ? 1 : 2;
  }
  return fits[dev] == 1 ? num_cus() / 8 * 8 : 0;
}

int fused_impl(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
               const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing, const uint16_t* residual,
               uint16_t* out, uint16_t* shared_out, void* ws, size_t ws_bytes, void* stream, int32_t max_polls) {
  if (max_polls < 0) return MOE_TAIL_ERR_INVALID;
  Layout lay;
  int rc = check_forward(dims, w, x_lat, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, ws_bytes, &lay);
  if (rc) return rc;
  const moe_tail_dims& d = *dims;
  const int L = d.latent;
  const Plans plans = plan_all(d, Mr, Ms);
  if (Mr == 0 && Ms <= kSmallMaxM)  // no routed work: the shared expert alone, as moe_tail_forward runs it
    return forward_impl(dims, w, x_lat, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, ws_bytes, stream,
                        nullptr);
  if (!fused_ok(d, plans, Mr, Ms)) return MOE_TAIL_ERR_UNSUPPORTED;
  const bool fp8 = d.wfmt == MOE_TAIL_W_FP8_BLOCK128, nv4 = is_nvfp4(d);
  const unsigned grid = fp8 ? fused_grid<TF_FP8>() : nv4 ? fused_grid<TF_NV4>() : fused_grid<TF_FP4>();
  if (grid < 8) return MOE_TAIL_ERR_UNSUPPORTED;

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // launch errors below are ours, not an earlier call's
  FusedArgs f = fused_args(d, w, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, lay, plans);
  f.max_polls = max_polls;
  {
    const long blocks = static_cast<long>(Mr) * (L / 128);
    hipLaunchKernelGGL(k_quant_clear, dim3(quant_grid(blocks)), dim3(256), 0, st, x_lat, at<uint8_t>(ws, lay.xq),
                       at<float>(ws, lay.sx), blocks, f.sync, kSyncWords, row_scales(d, lay, ws, routing, Mr));
  }
  if (fp8) hipLaunchKernelGGL(k_tail_small<TF_FP8>, dim3(grid), dim3(512), 0, st, f);
  else if (nv4) hipLaunchKernelGGL(k_tail_small<TF_NV4>, dim3(grid), dim3(512), 0, st, f);
  else hipLaunchKernelGGL(k_tail_small<TF_FP4>, dim3(grid), dim3(512), 0, st, f);
  return launched();
}

// Scratch of moe_tail_forward_noalloc: the workspace of one call, held by
// the library in device memory for as long as the process runs (one copy per
// GPU, each at its own address).  Host code never uses the array's name as
// an address: scratch_base() asks the runtime for this device's copy.
constexpr size_t kScratchBytes = MOE_TAIL_NOALLOC_MAX_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

// The current device's copy of `scratch`, looked up once per device (with
// that device current); nullptr if the runtime cannot give it.
void* scratch_base() {
  static std::mutex mu;
  static void* base[64] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (base[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    base[dev] = p;
  }
  return base[dev];
}

}  // namespace

extern "C" {

const char* moe_tail_strerror(int status) {
  switch (status) {
    case MOE_TAIL_OK: return "ok";
    case MOE_TAIL_ERR_INVALID: return "invalid argument";
    case MOE_TAIL_ERR_UNSUPPORTED: return "unsupported dims or format";
    case MOE_TAIL_ERR_WORKSPACE: return "workspace too small";
    case MOE_TAIL_ERR_DEVICE: return "device launch failed";
    default: return "unknown status";
  }
}

size_t moe_tail_workspace_bytes(const moe_tail_dims* dims, int32_t Mr, int32_t Ms) {
  if (check_dims(dims) || check_counts(Mr, Ms)) return 0;
  return layout_of(*dims, Mr, Ms).total;
}

int moe_tail_workspace_layout(const moe_tail_dims* dims, int32_t Mr, int32_t Ms, size_t offsets[MOE_TAIL_WS_NUM]) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if ((rc = check_counts(Mr, Ms))) return rc;
  if (offsets == nullptr) return MOE_TAIL_ERR_INVALID;
  const Layout l = layout_of(*dims, Mr, Ms);
  offsets[MOE_TAIL_WS_XQ] = l.xq;
  offsets[MOE_TAIL_WS_SX] = l.sx;
  offsets[MOE_TAIL_WS_HQ] = l.hq;
  offsets[MOE_TAIL_WS_SH] = l.sh;
  offsets[MOE_TAIL_WS_Y] = l.y;
  offsets[MOE_TAIL_WS_RN] = l.rn;
  offsets[MOE_TAIL_WS_HS] = l.hs;
  offsets[MOE_TAIL_WS_S] = l.s;
  offsets[MOE_TAIL_WS_STATUS] = l.sync_bytes > 0 ? l.sync + 4 * kSyncErr : SIZE_MAX;
  return MOE_TAIL_OK;
}

int moe_tail_route(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
                   const moe_tail_routing* out, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  if (Mr < 0 || Mr > kMaxTokens) return MOE_TAIL_ERR_INVALID;
  const moe_tail_dims& d = *dims;
  const int L = d.latent, E = d.num_experts, k = d.top_k;
  if ((rc = check_weights(d, w, true, false, false, false))) return rc;
  if ((rc = check_routing(out, Mr, k, E))) return rc;
  if (!ptr_ok(x_lat, static_cast<size_t>(Mr) * L * 2)) return MOE_TAIL_ERR_INVALID;
  // the routing scratch sits at the front of the workspace and depends on Mr only
  const Layout lay = layout_of(d, Mr, Mr);
  if (ws_bytes < lay.xq) return MOE_TAIL_ERR_WORKSPACE;
  if (lay.xq > 0 && !ptr_ok(ws, 1)) return MOE_TAIL_ERR_INVALID;

  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // launch errors below are ours, not an earlier call's
  const int ng = (Mr + kGroup - 1) / kGroup;
  float* logits = at<float>(ws, lay.logits);
  int32_t* hist = at<int32_t>(ws, lay.hist);
  if (Mr > 0) {
    const int egroups = (E + 4 * kLogitExpPerWave - 1) / (4 * kLogitExpPerWave);
    const size_t xtile = static_cast<size_t>(kLogitTok) * L * 2;  // dynamic LDS of the logits kernel
    const bool few = static_cast<long>((Mr + kLogitTok - 1) / kLogitTok) * egroups < kLogitSmallGrid;
    static bool lds_raised = false;
    if (!lds_raised) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_router_logits<kLogitTok, kLogitExpPerWave>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLogitTok * 8192 * 2);
      lds_raised = true;
    }
    if (Mr >= kWideMinTokens) {
      const dim3 grid((Mr + 15) / 16, (E + 15) / 16);
      auto lg = (static_cast<long>(grid.x) * grid.y > 3L * num_cus()) ? k_router_logits_tile<8, 8, 128>
                                                                        : k_router_logits_tile<8, 8, 256>;
      hipLaunchKernelGGL(lg, grid, dim3(256), 0, st, x_lat, w->gate, w->gate_bias, logits, Mr, L, E);
    }
    else if (few)
      hipLaunchKernelGGL((k_router_logits<2, 1>), dim3((Mr + 1) / 2, (E + 3) / 4), dim3(256),
                         static_cast<size_t>(2) * L * 2, st, x_lat, w->gate, w->gate_bias, logits, Mr, L, E);
    else
      hipLaunchKernelGGL((k_router_logits<kLogitTok, kLogitExpPerWave>), dim3((Mr + kLogitTok - 1) / kLogitTok, egroups),
                         dim3(256), xtile, st, x_lat, w->gate, w->gate_bias, logits, Mr, L, E);
  }
  // one workgroup for the whole permutation while it is short (it walks the
  // token groups one wave at a time), with the top-k too for up to 16
  // tokens (one per wave); three grid-wide passes beyond that
  const bool small_sort = static_cast<int64_t>(ng) * E <= kSortSmall && ng <= kSortSmallGroups;
  if (Mr > 0 && Mr <= kTopkSortTokens && small_sort) {
    auto ts = (E <= 64) ? k_router_topk_sort<1> : (E <= 128) ? k_router_topk_sort<2> : (E <= 384) ? k_router_topk_sort<6>
                                                                                       : k_router_topk_sort<kMaxExpertsPerLane>;
    hipLaunchKernelGGL(ts, dim3(1), dim3(1024), 0, st, logits, out->topk_ids, out->topk_weights, out->expert_offsets,
                       out->sorted_pair, out->pair_to_row, Mr, E, k, ng);
    return launched();
  }
  if (Mr > 0) {
    auto topk = (E <= 64) ? k_router_topk<1> : (E <= 128) ? k_router_topk<2> : (E <= 384) ? k_router_topk<6>
                                                                                 : k_router_topk<kMaxExpertsPerLane>;
    hipLaunchKernelGGL(topk, dim3((Mr + 3) / 4), dim3(256), 0, st, logits, out->topk_ids, out->topk_weights, Mr, E, k);
  }
  if (small_sort) {
    hipLaunchKernelGGL(k_router_sort, dim3(1), dim3(1024), 0, st, out->topk_ids, out->expert_offsets,
                       out->sorted_pair, out->pair_to_row, Mr, E, k, ng);
    return launched();
  }
  if (Mr > 0) hipLaunchKernelGGL(k_router_hist, dim3(ng), dim3(64), 0, st, out->topk_ids, hist, Mr, E, k, ng);
  hipLaunchKernelGGL(k_router_scan, dim3(1), dim3(1024), 0, st, hist, out->expert_offsets, E, ng);
  if (Mr > 0)
    hipLaunchKernelGGL(k_router_scatter, dim3(ng), dim3(64), 0, st, out->topk_ids, hist, out->sorted_pair,
                       out->pair_to_row, Mr, E, k, ng);
  return launched();
}

int moe_tail_forward(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
                     const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing, uint16_t* out,
                     uint16_t* shared_out, void* ws, size_t ws_bytes, void* stream) {
  return forward_impl(dims, w, x_lat, Mr, x_hid, Ms, routing, nullptr, out, shared_out, ws, ws_bytes, stream, nullptr);
}

int moe_tail_forward_noalloc(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
                             const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing, uint16_t* out,
                             uint16_t* shared_out, void* stream) {
  // every check first, with a stand-in for the scratch address (nothing is
  // dereferenced on the host), then the one runtime lookup
  Layout lay;
  void* const stand_in = reinterpret_cast<void*>(kAlign);
  int rc = check_forward(dims, w, x_lat, Mr, x_hid, Ms, routing, nullptr, out, shared_out, stand_in, kScratchBytes,
                         &lay);
  if (rc) return rc;
  void* base = scratch_base();
  if (base == nullptr) return MOE_TAIL_ERR_DEVICE;
  return forward_impl(dims, w, x_lat, Mr, x_hid, Ms, routing, nullptr, out, shared_out, base, kScratchBytes, stream,
                      nullptr, EV_NONE, false);
}

int moe_tail_forward_add3(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
                          const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing, const uint16_t* residual,
                          uint16_t* out, uint16_t* shared_out, void* ws, size_t ws_bytes, void* stream) {
  if (Mr > 0 && residual == nullptr) return MOE_TAIL_ERR_INVALID;
  return forward_impl(dims, w, x_lat, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, ws_bytes, stream, nullptr);
}

int moe_tail_forward_fused(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
                           const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing, const uint16_t* residual,
                           uint16_t* out, uint16_t* shared_out, void* ws, size_t ws_bytes, void* stream) {
  return fused_impl(dims, w, x_lat, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, ws_bytes, stream,
                    kSpinLimit);
}

int moe_tail_forward_fused_bounded(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat,
                                   int32_t Mr, const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing,
                                   const uint16_t* residual, uint16_t* out, uint16_t* shared_out, void* ws,
                                   size_t ws_bytes, void* stream, int32_t max_polls) {
  return fused_impl(dims, w, x_lat, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, ws_bytes, stream,
                    max_polls);
}

int moe_tail_forward_profiled(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat,
                              int32_t Mr, const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing,
                              uint16_t* out, uint16_t* shared_out, void* ws, size_t ws_bytes, void* stream,
                              void* const* stage_events) {
  if (stage_events == nullptr) return MOE_TAIL_ERR_INVALID;
  return forward_impl(dims, w, x_lat, Mr, x_hid, Ms, routing, nullptr, out, shared_out, ws, ws_bytes, stream,
                      stage_events, EV_PER_STAGE);
}

int moe_tail_forward_timed(const moe_tail_dims* dims, const moe_tail_weights* w, const uint16_t* x_lat, int32_t Mr,
                           const uint16_t* x_hid, int32_t Ms, const moe_tail_routing* routing,
                           const uint16_t* residual, uint16_t* out, uint16_t* shared_out, void* ws, size_t ws_bytes,
                           void* stream, void* const* events) {
  if (events == nullptr) return MOE_TAIL_ERR_INVALID;
  return forward_impl(dims, w, x_lat, Mr, x_hid, Ms, routing, residual, out, shared_out, ws, ws_bytes, stream, events,
                      EV_SCHEDULE);
}

const char* moe_tail_stage_name(const moe_tail_dims* dims, int32_t Mr, int32_t Ms, int32_t i) {
  if (check_dims(dims) || check_counts(Mr, Ms) || i < 0) return nullptr;
  const Plans plans = plan_all(*dims, Mr, Ms);
  if (fused_ok(*dims, plans, Mr, Ms)) return i < 6 ? kDecodeNames[i] : nullptr;
  return i < MOE_TAIL_NUM_STAGES ? kStagedNames[i] : nullptr;
}

int moe_tail_pack_mxfp4_scales(const moe_tail_dims* dims, const uint8_t* w1_scale, const uint8_t* w2_scale,
                               uint8_t* w1_scale_packed, uint8_t* w2_scale_packed, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  const moe_tail_dims& d = *dims;
  if (d.wfmt != MOE_TAIL_W_MXFP4 && d.wfmt != MOE_TAIL_W_MXFP4_PACKED) return MOE_TAIL_ERR_INVALID;
  if (d.latent % 256 || d.inter % 256) return MOE_TAIL_ERR_UNSUPPORTED;
  const size_t E = d.num_experts, L = d.latent, I = d.inter;
  const size_t n1 = E * 2 * I * (L / 32), n2 = E * L * (I / 32);  // bytes of each scale array
  if ((w1_scale == nullptr) != (w1_scale_packed == nullptr) || (w2_scale == nullptr) != (w2_scale_packed == nullptr))
    return MOE_TAIL_ERR_INVALID;
  if ((w1_scale && (!ptr_ok(w1_scale, n1) || !ptr_ok(w1_scale_packed, n1))) ||
      (w2_scale && (!ptr_ok(w2_scale, n2) || !ptr_ok(w2_scale_packed, n2))))
    return MOE_TAIL_ERR_INVALID;
  auto overlap = [](const uint8_t* a, const uint8_t* b, size_t n) { return a < b + n && b < a + n; };
  if ((w1_scale && overlap(w1_scale, w1_scale_packed, n1)) || (w2_scale && overlap(w2_scale, w2_scale_packed, n2)))
    return MOE_TAIL_ERR_INVALID;
  if (w1_scale == nullptr && w2_scale == nullptr) return MOE_TAIL_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (w1_scale) {
    const size_t words = n1 / 4;
    hipLaunchKernelGGL(k_pack_e8m0, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, st, w1_scale,
                       w1_scale_packed, words, static_cast<int>(2 * I), static_cast<int>(L), static_cast<int>(I));
  }
  if (w2_scale) {
    const size_t words = n2 / 4;
    hipLaunchKernelGGL(k_pack_e8m0, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0, st, w2_scale,
                       w2_scale_packed, words, static_cast<int>(L), static_cast<int>(I), 0);
  }
  return launched();
}

int moe_tail_pack_nvfp4_scales(const moe_tail_dims* dims, const uint8_t* w1_scale, const uint8_t* w2_scale,
                               uint8_t* w1_scale_packed, uint8_t* w2_scale_packed, void* stream) {
  int rc = check_dims(dims);
  if (rc) return rc;
  const moe_tail_dims& d = *dims;
  if (!is_nvfp4(d)) return MOE_TAIL_ERR_INVALID;
  if (d.latent % 256 || d.inter % 256) return MOE_TAIL_ERR_UNSUPPORTED;
  const size_t E = d.num_experts, L = d.latent, I = d.inter;
  const size_t n1 = E * 2 * I * (L / 16), n2 = E * L * (I / 16);  // bytes of each scale array
  if ((w1_scale == nullptr) != (w1_scale_packed == nullptr) || (w2_scale == nullptr) != (w2_scale_packed == nullptr))
    return MOE_TAIL_ERR_INVALID;
  if ((w1_scale && (!ptr_ok(w1_scale, n1) || !ptr_ok(w1_scale_packed, n1))) ||
      (w2_scale && (!ptr_ok(w2_scale, n2) || !ptr_ok(w2_scale_packed, n2))))
    return MOE_TAIL_ERR_INVALID;
  auto overlap = [](const uint8_t* a, const uint8_t* b, size_t n) { return a < b + n && b < a + n; };
  if ((w1_scale && overlap(w1_scale, w1_scale_packed, n1)) || (w2_scale && overlap(w2_scale, w2_scale_packed, n2)))
    return MOE_TAIL_ERR_INVALID;
  if (w1_scale == nullptr && w2_scale == nullptr) return MOE_TAIL_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (w1_scale) {
    const size_t runs = n1 / 16;
    hipLaunchKernelGGL(k_pack_e4m3_16, dim3(static_cast<unsigned>((runs + 255) / 256)), dim3(256), 0, st, w1_scale,
                       w1_scale_packed, runs, static_cast<int>(2 * I), static_cast<int>(L), static_cast<int>(I));
  }
  if (w2_scale) {
    const size_t runs = n2 / 16;
    hipLaunchKernelGGL(k_pack_e4m3_16, dim3(static_cast<unsigned>((runs + 255) / 256)), dim3(256), 0, st, w2_scale,
                       w2_scale_packed, runs, static_cast<int>(L), static_cast<int>(I), 0);
  }
  return launched();
}

int moe_tail_quant_fp8_1x128(const void* x, int32_t x_is_bf16, int32_t rows, int32_t cols, uint8_t* codes,
                             float* scales, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 128) return MOE_TAIL_ERR_INVALID;
  const size_t n = static_cast<size_t>(rows) * cols;
  if (!ptr_ok(x, n) || !ptr_ok(codes, n) || !ptr_ok(scales, n / 32)) return MOE_TAIL_ERR_INVALID;
  if (rows == 0) return MOE_TAIL_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const long blocks = static_cast<long>(rows) * (cols / 128);
  const dim3 grid(quant_grid(blocks));
  if (x_is_bf16)
    hipLaunchKernelGGL(k_quant_1x128<true>, grid, dim3(256), 0, st, x, codes, scales, blocks, RowScales{});
  else
    hipLaunchKernelGGL(k_quant_1x128<false>, grid, dim3(256), 0, st, x, codes, scales, blocks, RowScales{});
  return launched();
}

}  // extern "C"
