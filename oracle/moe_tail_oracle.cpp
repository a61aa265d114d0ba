// CPU oracle for the latent-MoE layer tail.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
// benchmark's CPU-baseline leg may load this library.  The product path (the
// HIP library) shares no code, header, table or helper with it.
//
// What it computes, step by step, in plain FP32 loops (the method's own
// precision: FP32 accumulation of block-scaled FP8/FP4 products, FP32 norm,
// BF16 storage of BF16 tensors):
//
//   router    logits -> top-k -> softmax over the k selected logits
//             ("top-k weighted expert combine", tokenspeed PR 1062, Summary)
//   permute   histogram -> exclusive scan -> stable scatter by (expert, token)
//   routed    x_lat quantized to e4m3 with one fp32 scale per 1x128 block;
//             L1 gate/up with 128x128 block-scaled e4m3 weights (or MXFP4, or
//             NVFP4: tokenspeed recipe, Allocation and launch);
//             SwiGLU; h re-quantized per 1x128; L2 down to the 3584-wide latent
//             ("[Kimi K3][Kernel] Fuse BF16 shared experts into latent MegaMoE
//             tail", Summary: routed FP8/FP4 MegaMoE producing a 3584-wide latent)
//   combine   sum_j w_j * y_j in FP32, then RMSNorm of the latent, stored bf16
//             (same page, Summary: the routed result needs RMSNorm before the
//             up-projection)
//   shared    BF16 SwiGLU MLP on the 7168-wide hidden; its intermediate and its
//             output are BF16 tensors
//   tail      up-projection 3584 -> 7168 accumulated in FP32, plus the shared
//             output added in FP32, one rounding to bf16 (same page, Summary:
//             the tail reduces the shared fragments in FP32 and adds them in
//             the epilogue)
//
// Readings where the pages are silent are listed with the design notes; the
// ones that change arithmetic are restated at the function that takes them.
//
// Parity pins: every function here is checked by the CPU tests against closed
// forms, exhaustive format tables, library casts, brute force on tiny shapes
// and invariants.  The FP32 summation order of the GPU's matrix cores and the
// GPU's expf/sqrt ulps are not pinned by this file (parity unpinned): the
// output tolerance covers them.
//
// Build: g++ -O2 -std=c++17 -fopenmp -fno-fast-math -ffp-contract=off -fPIC -shared

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// ---------------------------------------------------------------- formats --

float bf16_to_f32(uint16_t b) {
  uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Round to nearest even on the 16 dropped bits; NaN stays a quiet NaN.
uint16_t f32_to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40);
  uint32_t keep = u >> 16;
  uint32_t rest = u & 0xffffu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1;
  return static_cast<uint16_t>(keep);
}

// OCP 8-bit FP e4m3 ("fn"): bias 7, no infinities, S.1111.111 is NaN, max 448.
float e4m3_decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  float v = (e == 0) ? std::ldexp(static_cast<float>(m), -9)             // subnormal m * 2^-9
                     : std::ldexp(static_cast<float>(8 + m), e - 10);    // (1 + m/8) * 2^(e-7)
  return s ? -v : v;
}

// Decoded value of every code, and the magnitudes of the 127 finite
// non-negative codes (ascending by code), both filled from the closed form.
struct E4m3Table {
  float val[256];
  float mag[127];
  E4m3Table() {
    for (int c = 0; c < 256; ++c) val[c] = e4m3_decode(static_cast<uint8_t>(c));
    for (int c = 0; c < 127; ++c) mag[c] = val[c];
  }
};
const E4m3Table kE4m3;
inline float e4m3_value(uint8_t c) { return kE4m3.val[c]; }

// Round-to-nearest, ties to the even code, saturating to +-448 ("satfinite");
// the sign bit of the input is kept, also for results that round to zero.
uint8_t e4m3_encode(float v) {
  const uint8_t sign = std::signbit(v) ? 0x80 : 0x00;
  const float a = std::fabs(v);
  if (!(a < kE4m3.mag[126])) return sign | 126;  // >= 448 (and NaN, which is never fed)
  // first code whose magnitude is >= a
  int hi = static_cast<int>(std::lower_bound(kE4m3.mag, kE4m3.mag + 127, a) - kE4m3.mag);
  if (kE4m3.mag[hi] == a) return sign | static_cast<uint8_t>(hi);
  int lo = hi - 1;
  // distances are exact: both neighbours and a lie on a grid no finer than 2^-10
  float dlo = a - kE4m3.mag[lo], dhi = kE4m3.mag[hi] - a;
  int c;
  if (dlo < dhi) c = lo;
  else if (dhi < dlo) c = hi;
  else c = (lo % 2 == 0) ? lo : hi;
  return sign | static_cast<uint8_t>(c);
}

// OCP MX v1.0 e2m1: bias 1, codes 0..7 = 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign.
float e2m1_decode(uint8_t nib) {
  static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  float v = mag[nib & 7];
  return (nib & 8) ? -v : v;
}

// e8m0 scale: 2^(e - 127); 255 is NaN.
float e8m0_decode(uint8_t e) {
  if (e == 255) return NAN;
  return std::ldexp(1.0f, static_cast<int>(e) - 127);
}

struct E8m0Table {
  float val[256];
  E8m0Table() {
    for (int e = 0; e < 256; ++e) val[e] = e8m0_decode(static_cast<uint8_t>(e));
  }
};
const E8m0Table kE8m0;

// ------------------------------------------------------------ primitives --

// One row, 1x128 blocks: s = amax / 448 (IEEE division), q = e4m3(x / s);
// an all-zero block gets s = 1.  (Reading: plain amax scaling, no power-of-two
// rounding of the scale.)
void quant_row_1x128(const float* x, int cols, uint8_t* q, float* s) {
  for (int b = 0; b < cols / 128; ++b) {
    const float* xb = x + 128 * b;
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i) amax = std::max(amax, std::fabs(xb[i]));
    float scale = (amax == 0.0f) ? 1.0f : amax / 448.0f;
    s[b] = scale;
    for (int i = 0; i < 128; ++i) q[128 * b + i] = e4m3_encode(xb[i] / scale);
  }
}

// Sequential FP32 dot product, index ascending, multiply then add.
float dot(const float* a, const float* b, int n) {
  float acc = 0.0f;
  for (int i = 0; i < n; ++i) acc = acc + a[i] * b[i];
  return acc;
}

float silu_mul(float gate, float up) { return (gate / (1.0f + std::exp(-gate))) * up; }

// Dequantized routed weight row n of expert e of a [N, K] matrix.
//   FP8: W = RN(e4m3(code) * S[n/128, c/128])
//   MXFP4: W = e2m1(nibble) * 2^(e8m0 - 127)   (exact)
//   NVFP4: W = RN((e2m1(nibble) * e4m3(S[n, c/16])) * g[e]), the inner product
//          exact (at most five significant bits), g the matrix's fp32 scale.
//          (Reading: the pages name NVFP4 only as the served quantization;
//          this is the format as published: e2m1 elements, an e4m3 scale per
//          16 along K, an fp32 scale per tensor, here per expert matrix.)
void dequant_row(int wfmt, const uint8_t* w, const void* ws, const float* tscale, int e, int N, int K, int n,
                 float* out) {
  if (wfmt == 3) {
    const uint8_t* row = w + (static_cast<size_t>(e) * N + n) * (K / 2);
    const uint8_t* S = static_cast<const uint8_t*>(ws) + (static_cast<size_t>(e) * N + n) * (K / 16);
    const float g = tscale[e];
    for (int c = 0; c < K; ++c) {
      uint8_t byte = row[c / 2];
      uint8_t nib = (c % 2 == 0) ? (byte & 0xf) : (byte >> 4);
      out[c] = (e2m1_decode(nib) * e4m3_value(S[c / 16])) * g;
    }
    return;
  }
  if (wfmt == 0) {
    const uint8_t* row = w + (static_cast<size_t>(e) * N + n) * K;
    const float* S = static_cast<const float*>(ws) + static_cast<size_t>(e) * (N / 128) * (K / 128) +
                     static_cast<size_t>(n / 128) * (K / 128);
    for (int c = 0; c < K; ++c) out[c] = e4m3_value(row[c]) * S[c / 128];
  } else {
    const uint8_t* row = w + (static_cast<size_t>(e) * N + n) * (K / 2);
    const uint8_t* S = static_cast<const uint8_t*>(ws) + (static_cast<size_t>(e) * N + n) * (K / 32);
    for (int c = 0; c < K; ++c) {
      uint8_t byte = row[c / 2];
      uint8_t nib = (c % 2 == 0) ? (byte & 0xf) : (byte >> 4);
      out[c] = e2m1_decode(nib) * kE8m0.val[S[c / 32]];
    }
  }
}

}  // namespace

extern "C" {

// ---------------------------------------------------- exported primitives --

void oracle_bf16_from_f32(const float* x, int64_t n, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16(x[i]);
}

void oracle_e4m3_decode(const uint8_t* c, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_decode(c[i]);
}

void oracle_e4m3_encode(const float* x, int64_t n, uint8_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_encode(x[i]);
}

void oracle_e2m1_decode(const uint8_t* nib, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e2m1_decode(nib[i]);
}

void oracle_e8m0_decode(const uint8_t* e, int64_t n, float* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = e8m0_decode(e[i]);
}

// 1x128 FP8 quantization of fp32 rows [rows, cols] (cols % 128 == 0).
void oracle_quant_1x128(const float* x, int rows, int cols, uint8_t* q, float* s) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r)
    quant_row_1x128(x + static_cast<size_t>(r) * cols, cols, q + static_cast<size_t>(r) * cols,
                    s + static_cast<size_t>(r) * (cols / 128));
}

// RMSNorm of fp32 rows: ms = (sum z^2) / n in FP32, r = 1 / sqrt(ms + eps),
// out = bf16((z * r) * gamma).  (Reading: FP32-internal norm, eps inside the
// root, gamma after normalisation.)
void oracle_rmsnorm(const float* z, int rows, int n, const uint16_t* gamma, float eps, uint16_t* out) {
  for (int t = 0; t < rows; ++t) {
    const float* zr = z + static_cast<size_t>(t) * n;
    float ss = 0.0f;
    for (int c = 0; c < n; ++c) ss = ss + zr[c] * zr[c];
    float ms = ss / static_cast<float>(n);
    float r = 1.0f / std::sqrt(ms + eps);
    for (int c = 0; c < n; ++c) out[static_cast<size_t>(t) * n + c] = f32_to_bf16((zr[c] * r) * bf16_to_f32(gamma[c]));
  }
}

// ------------------------------------------------------------------ router --

// Router logits with a fixed FP32 summation order, so that the argmax they
// feed is reproducible bit for bit on a 64-lane wavefront:
//   p[l] = fma-chain over i of x[64 i + l] * W[e, 64 i + l]   (l = 0..63)
//   xor butterfly: for off in 32,16,8,4,2,1: p[l] = p[l] + p[l ^ off]
//   logit = p[0] + bias[e]
// (Reading: the pages give no order; this is the contract both sides keep.)
void oracle_router_logits(int L, int E, int Mr, const uint16_t* x_lat, const float* gate, const float* bias,
                          float* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < Mr; ++t) {
    for (int e = 0; e < E; ++e) {
      float p[64];
      for (int l = 0; l < 64; ++l) {
        float acc = 0.0f;
        for (int i = 0; i < L / 64; ++i) {
          size_t c = static_cast<size_t>(64) * i + l;
          acc = std::fma(bf16_to_f32(x_lat[static_cast<size_t>(t) * L + c]), gate[static_cast<size_t>(e) * L + c], acc);
        }
        p[l] = acc;
      }
      for (int off = 32; off >= 1; off /= 2) {
        float q[64];
        for (int l = 0; l < 64; ++l) q[l] = p[l] + p[l ^ off];
        std::memcpy(p, q, sizeof(p));
      }
      logits[static_cast<size_t>(t) * E + e] = p[0] + (bias ? bias[e] : 0.0f);
    }
  }
}

// Top-k by repeated argmax, key (logit descending, expert index ascending);
// softmax over the k selected logits: m = top logit, u_j = exp(l_j - m),
// S = sum of u_j in j order, w_j = u_j / S.
void oracle_topk_softmax(int E, int k, int Mr, const float* logits, int32_t* ids, float* w) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < Mr; ++t) {
    const float* l = logits + static_cast<size_t>(t) * E;
    std::vector<char> taken(E, 0);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;  // strict: equal logits keep the lower index
      }
      taken[best] = 1;
      ids[static_cast<size_t>(t) * k + j] = best;
    }
    const float m = l[ids[static_cast<size_t>(t) * k]];
    float u[64];
    float S = 0.0f;
    for (int j = 0; j < k; ++j) {
      u[j] = std::exp(l[ids[static_cast<size_t>(t) * k + j]] - m);
      S = S + u[j];
    }
    for (int j = 0; j < k; ++j) w[static_cast<size_t>(t) * k + j] = u[j] / S;
  }
}

void oracle_route(int L, int E, int k, int Mr, const uint16_t* x_lat, const float* gate, const float* bias,
                  int32_t* ids, float* w, float* logits_out) {
  std::vector<float> logits(static_cast<size_t>(Mr) * E);
  oracle_router_logits(L, E, Mr, x_lat, gate, bias, logits.data());
  oracle_topk_softmax(E, k, Mr, logits.data(), ids, w);
  if (logits_out) std::memcpy(logits_out, logits.data(), logits.size() * sizeof(float));
}

// Counting sort of the (token, slot) pairs by expert, stable in token order:
//   cnt[e] = #pairs routed to e; offsets = exclusive prefix sum (offsets[E] = Mr*k)
//   sorted_pair[offsets[e] + n] = t*k + j for the n-th token (ascending) routed to e
//   pair_to_row[t*k + j] = that position
void oracle_permute(int E, int k, int Mr, const int32_t* ids, int32_t* offsets, int32_t* sorted_pair,
                    int32_t* pair_to_row) {
  std::vector<int32_t> cnt(E, 0);
  for (int p = 0; p < Mr * k; ++p) cnt[ids[p]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + cnt[e];
  std::vector<int32_t> fill(offsets, offsets + E);
  for (int t = 0; t < Mr; ++t)
    for (int j = 0; j < k; ++j) {
      int p = t * k + j;
      int row = fill[ids[p]]++;
      sorted_pair[row] = p;
      pair_to_row[p] = row;
    }
}

// ----------------------------------------------------------------- forward --

// Forward pass for the tokens listed in `sel` (indices into 0..Ms-1).
// Token t < Mr produces the combined output row; t >= Mr only the shared row.
// Per selected token s (outputs are [n_sel, ...], optional ones may be NULL):
//   out_f32[s, H]  t < Mr: up(rn) + f32(s_bf) before rounding, then + f32(residual[t])
//                  when a residual is given ("add3": tokenspeed PR, commit log); t >= Mr: f32(s_bf)
//   out_bf16[s, H] t < Mr: bf16(out_f32); t >= Mr: s_bf (the shared_out row)
//   xq[s, L], sx[s, L/128]                  x_lat codes and scales (t < Mr)
//   hq[s, k, I], sh[s, k, I/128], h[s, k, I] h codes, scales, pre-quantization h
//   y[s, k, L]                               routed L2 output per slot
//   rn[s, L]                                 normalised latent (bf16)
//   hs[s, Is], sbf[s, H]                     shared intermediate and output (bf16)
// w1_tscale / w2_tscale: [E] fp32 scales of the NVFP4 matrices (wfmt 3; NULL
// otherwise).
// hq_in / sh_in (optional, [n_sel, k, I] codes and [n_sel, k, I/128] scales,
// rows in sel order): h codes and scales given instead of computed; the
// routed L1 and SwiGLU are then skipped (h_out reads 0) and every later step
// runs on the given codes.  This is how a test checks the steps after the h
// quantization on exactly the codes another implementation produced.
int oracle_forward(int H, int L, int E, int k, int I, int Is, int wfmt, float eps,
                   const uint8_t* w1, const void* w1s, const uint8_t* w2, const void* w2s,
                   const uint16_t* gamma, const uint16_t* w_up, const uint16_t* ws1, const uint16_t* ws2,
                   const uint16_t* x_lat, int Mr, const uint16_t* x_hid, int Ms,
                   const int32_t* topk_ids, const float* topk_w, const uint16_t* residual,
                   int n_sel, const int32_t* sel,
                   float* out_f32, uint16_t* out_bf16,
                   uint8_t* xq_out, float* sx_out, uint8_t* hq_out, float* sh_out, float* h_out,
                   float* y_out, uint16_t* rn_out, uint16_t* hs_out, uint16_t* sbf_out,
                   const uint8_t* hq_in, const float* sh_in, const float* w1_tscale, const float* w2_tscale) {
  if ((hq_in == nullptr) != (sh_in == nullptr)) return 1;
  if (wfmt != 0 && wfmt != 1 && wfmt != 3) return 1;
  if (wfmt == 3 && (w1_tscale == nullptr || w2_tscale == nullptr)) return 1;
  if (L % 128 || H % 128 || I % 128 || Is % 128 || k < 1 || k > E || Mr < 0 || Mr > Ms) return 1;
  for (int s = 0; s < n_sel; ++s)
    if (sel[s] < 0 || sel[s] >= Ms) return 1;
  const size_t nsel = static_cast<size_t>(n_sel);

  // token lists: routed (t < Mr) positions in sel
  std::vector<int> rsel;
  for (int s = 0; s < n_sel; ++s)
    if (sel[s] < Mr) rsel.push_back(s);
  const int nr = static_cast<int>(rsel.size());

  // --- routed: quantize x, dequantize it back (x_hat = RN(e4m3(q) * s)) ---
  std::vector<uint8_t> xq(static_cast<size_t>(nr) * L);
  std::vector<float> sx(static_cast<size_t>(nr) * (L / 128));
  std::vector<float> xhat(static_cast<size_t>(nr) * L);
#pragma omp parallel for schedule(static)
  for (int a = 0; a < nr; ++a) {
    const int t = sel[rsel[a]];
    std::vector<float> xf(L);
    for (int c = 0; c < L; ++c) xf[c] = bf16_to_f32(x_lat[static_cast<size_t>(t) * L + c]);
    quant_row_1x128(xf.data(), L, &xq[static_cast<size_t>(a) * L], &sx[static_cast<size_t>(a) * (L / 128)]);
    for (int c = 0; c < L; ++c)
      xhat[static_cast<size_t>(a) * L + c] = e4m3_value(xq[static_cast<size_t>(a) * L + c]) * sx[static_cast<size_t>(a) * (L / 128) + c / 128];
  }

  // --- routed L1: g[a, j, n] = sum_c x_hat[a, c] * W1_hat[e, n, c] ---
  std::vector<float> g(hq_in ? 0 : static_cast<size_t>(nr) * k * 2 * I);
  if (!hq_in)
#pragma omp parallel
  {
    std::vector<float> wrow(L);
#pragma omp for schedule(dynamic, 16) collapse(2)
    for (int aj = 0; aj < nr * k; ++aj)
      for (int n = 0; n < 2 * I; ++n) {
        const int a = aj / k, j = aj % k;
        const int t = sel[rsel[a]];
        const int e = topk_ids[static_cast<size_t>(t) * k + j];
        dequant_row(wfmt, w1, w1s, w1_tscale, e, 2 * I, L, n, wrow.data());
        g[static_cast<size_t>(aj) * 2 * I + n] = dot(&xhat[static_cast<size_t>(a) * L], wrow.data(), L);
      }
  }

  // --- SwiGLU, then 1x128 quantization of h and its dequantized value ---
  std::vector<float> h(static_cast<size_t>(nr) * k * I), hhat(static_cast<size_t>(nr) * k * I);
  std::vector<uint8_t> hq(static_cast<size_t>(nr) * k * I);
  std::vector<float> sh(static_cast<size_t>(nr) * k * (I / 128));
#pragma omp parallel for schedule(static)
  for (int aj = 0; aj < nr * k; ++aj) {
    float* ha = &h[static_cast<size_t>(aj) * I];
    if (hq_in) {
      // the given codes of selected token rsel[aj / k], slot aj % k
      const size_t src = static_cast<size_t>(rsel[aj / k]) * k + aj % k;
      std::memcpy(&hq[static_cast<size_t>(aj) * I], hq_in + src * I, I);
      std::memcpy(&sh[static_cast<size_t>(aj) * (I / 128)], sh_in + src * (I / 128), (I / 128) * 4);
    } else {
      const float* ga = &g[static_cast<size_t>(aj) * 2 * I];
      for (int n = 0; n < I; ++n) ha[n] = silu_mul(ga[n], ga[I + n]);
      quant_row_1x128(ha, I, &hq[static_cast<size_t>(aj) * I], &sh[static_cast<size_t>(aj) * (I / 128)]);
    }
    for (int n = 0; n < I; ++n)
      hhat[static_cast<size_t>(aj) * I + n] = e4m3_value(hq[static_cast<size_t>(aj) * I + n]) * sh[static_cast<size_t>(aj) * (I / 128) + n / 128];
  }

  // --- routed L2: y[a, j, n] = sum_i h_hat[a, j, i] * W2_hat[e, n, i] ---
  std::vector<float> y(static_cast<size_t>(nr) * k * L);
#pragma omp parallel
  {
    std::vector<float> wrow(I);
#pragma omp for schedule(dynamic, 16) collapse(2)
    for (int aj = 0; aj < nr * k; ++aj)
      for (int n = 0; n < L; ++n) {
        const int a = aj / k, j = aj % k;
        const int t = sel[rsel[a]];
        const int e = topk_ids[static_cast<size_t>(t) * k + j];
        dequant_row(wfmt, w2, w2s, w2_tscale, e, L, I, n, wrow.data());
        y[static_cast<size_t>(aj) * L + n] = dot(&hhat[static_cast<size_t>(aj) * I], wrow.data(), I);
      }
  }

  // --- combine z = sum_j w_j * y_j (j ascending), RMSNorm -> rn (bf16) ---
  std::vector<float> z(static_cast<size_t>(nr) * L);
  for (int a = 0; a < nr; ++a) {
    const int t = sel[rsel[a]];
    for (int n = 0; n < L; ++n) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) acc = acc + topk_w[static_cast<size_t>(t) * k + j] * y[(static_cast<size_t>(a) * k + j) * L + n];
      z[static_cast<size_t>(a) * L + n] = acc;
    }
  }
  std::vector<uint16_t> rn(static_cast<size_t>(nr) * L);
  oracle_rmsnorm(z.data(), nr, L, gamma, eps, rn.data());

  // --- shared expert on every selected token ---
  std::vector<uint16_t> hs(nsel * Is), sbf(nsel * H);
#pragma omp parallel
  {
    std::vector<float> xr(H), wr(H), gs(2 * Is);
#pragma omp for schedule(dynamic, 1)
    for (int s = 0; s < n_sel; ++s) {
      const int t = sel[s];
      for (int c = 0; c < H; ++c) xr[c] = bf16_to_f32(x_hid[static_cast<size_t>(t) * H + c]);
      for (int n = 0; n < 2 * Is; ++n) {
        for (int c = 0; c < H; ++c) wr[c] = bf16_to_f32(ws1[static_cast<size_t>(n) * H + c]);
        gs[n] = dot(xr.data(), wr.data(), H);
      }
      for (int n = 0; n < Is; ++n) hs[static_cast<size_t>(s) * Is + n] = f32_to_bf16(silu_mul(gs[n], gs[Is + n]));
    }
  }
#pragma omp parallel
  {
    std::vector<float> hr(Is), wr(Is);
#pragma omp for schedule(dynamic, 1)
    for (int s = 0; s < n_sel; ++s) {
      for (int i = 0; i < Is; ++i) hr[i] = bf16_to_f32(hs[static_cast<size_t>(s) * Is + i]);
      for (int n = 0; n < H; ++n) {
        for (int i = 0; i < Is; ++i) wr[i] = bf16_to_f32(ws2[static_cast<size_t>(n) * Is + i]);
        sbf[static_cast<size_t>(s) * H + n] = f32_to_bf16(dot(hr.data(), wr.data(), Is));
      }
    }
  }

  // --- up-projection + FP32 shared add, one rounding ---
  std::vector<float> of(nsel * H);
#pragma omp parallel
  {
    std::vector<float> rr(L), wr(L);
#pragma omp for schedule(dynamic, 1)
    for (int s = 0; s < n_sel; ++s) {
      const int t = sel[s];
      if (t >= Mr) {
        for (int n = 0; n < H; ++n) of[static_cast<size_t>(s) * H + n] = bf16_to_f32(sbf[static_cast<size_t>(s) * H + n]);
        continue;
      }
      const int a = static_cast<int>(std::find(rsel.begin(), rsel.end(), s) - rsel.begin());
      for (int c = 0; c < L; ++c) rr[c] = bf16_to_f32(rn[static_cast<size_t>(a) * L + c]);
      for (int n = 0; n < H; ++n) {
        for (int c = 0; c < L; ++c) wr[c] = bf16_to_f32(w_up[static_cast<size_t>(n) * L + c]);
        float v = dot(rr.data(), wr.data(), L) + bf16_to_f32(sbf[static_cast<size_t>(s) * H + n]);
        if (residual) v = v + bf16_to_f32(residual[static_cast<size_t>(t) * H + n]);
        of[static_cast<size_t>(s) * H + n] = v;
      }
    }
  }

  // --- outputs ---
  for (int s = 0; s < n_sel; ++s) {
    const int t = sel[s];
    for (int n = 0; n < H; ++n) {
      const size_t o = static_cast<size_t>(s) * H + n;
      if (out_f32) out_f32[o] = of[o];
      if (out_bf16) out_bf16[o] = (t < Mr) ? f32_to_bf16(of[o]) : sbf[o];
    }
    if (hs_out) std::memcpy(hs_out + static_cast<size_t>(s) * Is, &hs[static_cast<size_t>(s) * Is], Is * 2);
    if (sbf_out) std::memcpy(sbf_out + static_cast<size_t>(s) * H, &sbf[static_cast<size_t>(s) * H], H * 2);
  }
  for (int a = 0; a < nr; ++a) {
    const size_t s = static_cast<size_t>(rsel[a]);
    if (xq_out) std::memcpy(xq_out + s * L, &xq[static_cast<size_t>(a) * L], L);
    if (sx_out) std::memcpy(sx_out + s * (L / 128), &sx[static_cast<size_t>(a) * (L / 128)], (L / 128) * 4);
    if (hq_out) std::memcpy(hq_out + s * k * I, &hq[static_cast<size_t>(a) * k * I], static_cast<size_t>(k) * I);
    if (sh_out) std::memcpy(sh_out + s * k * (I / 128), &sh[static_cast<size_t>(a) * k * (I / 128)], static_cast<size_t>(k) * (I / 128) * 4);
    if (h_out) std::memcpy(h_out + s * k * I, &h[static_cast<size_t>(a) * k * I], static_cast<size_t>(k) * I * 4);
    if (y_out) std::memcpy(y_out + s * k * L, &y[static_cast<size_t>(a) * k * L], static_cast<size_t>(k) * L * 4);
    if (rn_out) std::memcpy(rn_out + s * L, &rn[static_cast<size_t>(a) * L], L * 2);
  }
  return 0;
}

}  // extern "C"
