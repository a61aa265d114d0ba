// Runs the CPU oracle's entry points on small random inputs under the
// address and undefined-behaviour sanitizers (built by
// tests/test_sanitizers.py): the decoders over every code, the quantizer,
// routing, the permutation and the forward pass for FP8, MXFP4 and NVFP4 weights,
// with token subsets, shared-only rows, the residual join and given h codes.
// Exit status 0 when every call accepted its arguments; a sanitizer report
// aborts the process.
#include "../../oracle/moe_tail_oracle.cpp"

#include <cstdio>
#include <random>
#include <vector>

namespace {

std::mt19937 rng(7);

float unif(float a, float b) { return std::uniform_real_distribution<float>(a, b)(rng); }
float gauss() { return std::normal_distribution<float>(0.0f, 1.0f)(rng); }
uint16_t bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>(u >> 16);
}
uint8_t e4m3_code() {  // any finite code
  uint8_t c;
  do c = static_cast<uint8_t>(rng() & 0xFF); while ((c & 0x7F) == 0x7F);
  return c;
}

int run(int wfmt) {
  const int L = 256, H = 384, I = 128, Is = 128, E = 4, k = 2, Mr = 5, Ms = 7;
  const float eps = 1e-6f;
  std::vector<uint16_t> x_lat(Mr * L), x_hid(Ms * H), gamma(L), w_up(H * L), ws1(2 * Is * H), ws2(H * Is),
      resid(Mr * H);
  for (auto& v : x_lat) v = bf16(gauss());
  for (auto& v : x_hid) v = bf16(gauss());
  for (auto& v : gamma) v = bf16(unif(0.5f, 1.5f));
  for (auto& v : w_up) v = bf16(0.05f * gauss());
  for (auto& v : ws1) v = bf16(0.05f * gauss());
  for (auto& v : ws2) v = bf16(0.08f * gauss());
  for (auto& v : resid) v = bf16(gauss());
  std::vector<float> gate(E * L), bias(E);
  for (auto& v : gate) v = 0.02f * gauss();
  for (int e = 0; e < E; ++e) bias[e] = -1.2f * std::log(static_cast<float>(e + 1));

  // routed weights
  std::vector<uint8_t> w1, w2, w1s8, w2s8;
  std::vector<float> w1s, w2s, tsc(E);
  for (auto& v : tsc) v = unif(1e-4f, 1e-3f);
  if (wfmt == 0) {
    w1.resize(static_cast<size_t>(E) * 2 * I * L);
    w2.resize(static_cast<size_t>(E) * L * I);
    for (auto& v : w1) v = e4m3_code();
    for (auto& v : w2) v = e4m3_code();
    w1s.resize(static_cast<size_t>(E) * (2 * I / 128) * (L / 128));
    w2s.resize(static_cast<size_t>(E) * (L / 128) * (I / 128));
    for (auto& v : w1s) v = unif(1e-4f, 1e-2f);
    for (auto& v : w2s) v = unif(1e-4f, 1e-2f);
  } else {
    w1.resize(static_cast<size_t>(E) * 2 * I * L / 2);
    w2.resize(static_cast<size_t>(E) * L * I / 2);
    for (auto& v : w1) v = static_cast<uint8_t>(rng() & 0xFF);
    for (auto& v : w2) v = static_cast<uint8_t>(rng() & 0xFF);
    const int grp = wfmt == 3 ? 16 : 32;  // NVFP4: e4m3 scale per 16, MXFP4: e8m0 per 32
    w1s8.resize(static_cast<size_t>(E) * 2 * I * L / grp);
    w2s8.resize(static_cast<size_t>(E) * L * I / grp);
    for (auto& v : w1s8) v = wfmt == 3 ? static_cast<uint8_t>(rng() & 0x7E) : static_cast<uint8_t>(118 + rng() % 8);
    for (auto& v : w2s8) v = wfmt == 3 ? static_cast<uint8_t>(rng() & 0x7E) : static_cast<uint8_t>(118 + rng() % 8);
  }
  const void* w1s_p = wfmt == 0 ? static_cast<const void*>(w1s.data()) : w1s8.data();
  const void* w2s_p = wfmt == 0 ? static_cast<const void*>(w2s.data()) : w2s8.data();

  // routing
  std::vector<int32_t> ids(Mr * k), off(E + 1), sp(Mr * k), p2r(Mr * k);
  std::vector<float> w(Mr * k), logits(Mr * E);
  oracle_router_logits(L, E, Mr, x_lat.data(), gate.data(), bias.data(), logits.data());
  oracle_route(L, E, k, Mr, x_lat.data(), gate.data(), bias.data(), ids.data(), w.data(), nullptr);
  oracle_permute(E, k, Mr, ids.data(), off.data(), sp.data(), p2r.data());

  // forward on every token, then on a subset with the residual and given h codes
  const int n_all = Ms;
  std::vector<int32_t> sel_all(n_all);
  for (int i = 0; i < n_all; ++i) sel_all[i] = i;
  std::vector<float> out_f32(n_all * H), h(n_all * k * I), y(n_all * k * L), sx(n_all * (L / 128)),
      sh(n_all * k * (I / 128));
  std::vector<uint16_t> out_bf16(n_all * H), rn(n_all * L), hs(n_all * Is), sbf(n_all * H);
  std::vector<uint8_t> xq(n_all * L), hq(n_all * k * I);
  int rc = oracle_forward(H, L, E, k, I, Is, wfmt, eps, w1.data(), w1s_p, w2.data(), w2s_p, gamma.data(), w_up.data(),
                          ws1.data(), ws2.data(), x_lat.data(), Mr, x_hid.data(), Ms, ids.data(), w.data(), nullptr,
                          n_all, sel_all.data(), out_f32.data(), out_bf16.data(), xq.data(), sx.data(), hq.data(),
                          sh.data(), h.data(), y.data(), rn.data(), hs.data(), sbf.data(), nullptr, nullptr,
                          tsc.data(), tsc.data());
  if (rc) return 10 + rc;
  const std::vector<int32_t> sel = {6, 0, 3};
  const int n = static_cast<int>(sel.size());
  std::vector<uint8_t> hq_in(n * k * I);
  std::vector<float> sh_in(n * k * (I / 128));
  for (int s = 0; s < n; ++s) {
    std::memcpy(&hq_in[s * k * I], &hq[sel[s] * k * I], k * I);
    std::memcpy(&sh_in[s * k * (I / 128)], &sh[sel[s] * k * (I / 128)], k * (I / 128) * 4);
  }
  std::vector<float> o2(n * H);
  rc = oracle_forward(H, L, E, k, I, Is, wfmt, eps, w1.data(), w1s_p, w2.data(), w2s_p, gamma.data(), w_up.data(),
                      ws1.data(), ws2.data(), x_lat.data(), Mr, x_hid.data(), Ms, ids.data(), w.data(), resid.data(),
                      n, sel.data(), o2.data(), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                      nullptr, nullptr, hq_in.data(), sh_in.data(), tsc.data(), tsc.data());
  if (rc) return 20 + rc;
  // a rejected call: h codes without scales
  if (oracle_forward(H, L, E, k, I, Is, wfmt, eps, w1.data(), w1s_p, w2.data(), w2s_p, gamma.data(), w_up.data(),
                     ws1.data(), ws2.data(), x_lat.data(), Mr, x_hid.data(), Ms, ids.data(), w.data(), nullptr, n,
                     sel.data(), o2.data(), nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr, nullptr, hq_in.data(), nullptr, tsc.data(), tsc.data()) == 0)
    return 30;
  return 0;
}

}  // namespace

int main() {
  // every code of the element decoders, the encoder and bf16 rounding
  std::vector<uint8_t> codes(256);
  for (int i = 0; i < 256; ++i) codes[i] = static_cast<uint8_t>(i);
  std::vector<float> dec(256), vals(4096);
  oracle_e4m3_decode(codes.data(), 256, dec.data());
  oracle_e2m1_decode(codes.data(), 16, dec.data());
  oracle_e8m0_decode(codes.data(), 255, dec.data());
  for (auto& v : vals) v = 100.0f * gauss();
  std::vector<uint8_t> enc(4096);
  std::vector<uint16_t> b16(4096);
  oracle_e4m3_encode(vals.data(), 4096, enc.data());
  oracle_bf16_from_f32(vals.data(), 4096, b16.data());
  std::vector<uint8_t> q(4096);
  std::vector<float> s(32);
  oracle_quant_1x128(vals.data(), 4, 1024, q.data(), s.data());
  for (int wfmt : {0, 1, 3}) {
    const int rc = run(wfmt);
    if (rc) {
      std::printf("oracle driver: format %d failed (%d)\n", wfmt, rc);
      return rc;
    }
  }
  std::printf("oracle driver: ok\n");
  return 0;
}
