// Runs the host side of the tail's C ABI under the address and
// undefined-behaviour sanitizers (built by tests/test_sanitizers.py together
// with the library source): workspace sizing and layout over many shapes,
// the stage names, and every argument rejection of every entry point, with
// placeholder addresses that are never dereferenced (each call below fails
// its host checks before any runtime call).  Exit status 0 when every call
// returned what the header states.
#include <cstdio>
#include <cstdint>

#include "../../include/moe_tail.h"
#include "../../include/moe_tail_probes.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what) {
  if (got != want) {
    std::printf("abi driver: %s returned %d, expected %d\n", what, got, want);
    ++failures;
  }
}

moe_tail_dims dims(int E = 64, int k = 8, int I = 2048, int Is = 2048, int wfmt = MOE_TAIL_W_FP8_BLOCK128,
                   int H = 7168, int L = 3584, float eps = 1e-6f) {
  return moe_tail_dims{H, L, E, k, I, Is, wfmt, eps};
}

void* addr(uint64_t a) { return reinterpret_cast<void*>(a); }

}  // namespace

int main() {
  const uint64_t base = 1ull << 40;
  moe_tail_weights w{};
  w.gate = static_cast<const float*>(addr(base));
  w.gate_bias = static_cast<const float*>(addr(base + (1ull << 30)));
  w.w1 = static_cast<const uint8_t*>(addr(base + (2ull << 30)));
  w.w1_scale = addr(base + (3ull << 30));
  w.w2 = static_cast<const uint8_t*>(addr(base + (4ull << 30)));
  w.w2_scale = addr(base + (5ull << 30));
  w.rms_gamma = static_cast<const uint16_t*>(addr(base + (6ull << 30)));
  w.w_up = static_cast<const uint16_t*>(addr(base + (7ull << 30)));
  w.ws1 = static_cast<const uint16_t*>(addr(base + (8ull << 30)));
  w.ws2 = static_cast<const uint16_t*>(addr(base + (9ull << 30)));
  moe_tail_routing r{};
  r.topk_ids = static_cast<int32_t*>(addr(base + (10ull << 30)));
  r.topk_weights = static_cast<float*>(addr(base + (11ull << 30)));
  r.expert_offsets = static_cast<int32_t*>(addr(base + (12ull << 30)));
  r.sorted_pair = static_cast<int32_t*>(addr(base + (13ull << 30)));
  r.pair_to_row = static_cast<int32_t*>(addr(base + (14ull << 30)));
  auto X = static_cast<const uint16_t*>(addr(1ull << 42));
  auto OUT = static_cast<uint16_t*>(addr(1ull << 43));
  auto SOUT = static_cast<uint16_t*>(addr(1ull << 44));
  void* WS = addr(1ull << 45);

  // sizing and layout over shapes (including the workloads and edge counts)
  const int shapes[][4] = {{8, 2, 16, 16}, {64, 8, 128, 128}, {64, 8, 4096, 4096}, {128, 8, 1024, 1024},
                           {384, 8, 2048, 8192}, {1024, 16, 200, 300}, {5, 5, 0, 70}, {9, 3, 1, 1}};
  for (const auto& sh : shapes) {
    for (int wfmt = 0; wfmt <= 4; ++wfmt) {
      const moe_tail_dims d = dims(sh[0], sh[1], 2048, 2048, wfmt);
      const size_t need = moe_tail_workspace_bytes(&d, sh[2], sh[3]);
      size_t off[MOE_TAIL_WS_NUM];
      expect(moe_tail_workspace_layout(&d, sh[2], sh[3], off), MOE_TAIL_OK, "workspace_layout");
      for (int i = 0; i < MOE_TAIL_WS_STATUS; ++i)
        if (off[i] > need) expect(1, 0, "layout offset past the workspace");
      for (int i = 0; moe_tail_stage_name(&d, sh[2], sh[3], i) != nullptr; ++i)
        if (i > MOE_TAIL_NUM_STAGES) expect(1, 0, "too many stage names");
    }
  }
  // invalid and unsupported dims
  moe_tail_dims bad = dims();
  bad.top_k = 0;
  expect(static_cast<int>(moe_tail_workspace_bytes(&bad, 16, 16)), 0, "workspace_bytes(top_k 0)");
  bad = dims(64, 8, 2000);
  size_t off[MOE_TAIL_WS_NUM];
  expect(moe_tail_workspace_layout(&bad, 16, 16, off), MOE_TAIL_ERR_UNSUPPORTED, "layout(I 2000)");
  expect(moe_tail_workspace_layout(nullptr, 16, 16, off), MOE_TAIL_ERR_INVALID, "layout(null dims)");
  bad = dims();
  bad.rms_eps = 0.0f;
  expect(moe_tail_workspace_layout(&bad, 16, 16, off), MOE_TAIL_ERR_INVALID, "layout(eps 0)");

  // every entry point's rejections
  const moe_tail_dims d = dims();
  const size_t need = moe_tail_workspace_bytes(&d, 16, 32), need16 = moe_tail_workspace_bytes(&d, 16, 16);
  expect(moe_tail_route(&d, &w, X, 16, &r, WS, 0, nullptr), MOE_TAIL_ERR_WORKSPACE, "route(ws 0)");
  expect(moe_tail_route(&d, &w, nullptr, 16, &r, WS, need16, nullptr), MOE_TAIL_ERR_INVALID, "route(null x)");
  expect(moe_tail_route(&d, &w, X, -1, &r, WS, need16, nullptr), MOE_TAIL_ERR_INVALID, "route(Mr -1)");
  expect(moe_tail_forward(&d, &w, X, 16, X, 32, &r, OUT, nullptr, WS, need, nullptr), MOE_TAIL_ERR_INVALID,
         "forward(no shared_out)");
  expect(moe_tail_forward(&d, &w, X, 17, X, 16, &r, OUT, nullptr, WS, need16, nullptr), MOE_TAIL_ERR_INVALID,
         "forward(Mr > Ms)");
  expect(moe_tail_forward(&d, &w, X, 16, X, 32, &r, OUT, SOUT, WS, need - 1, nullptr), MOE_TAIL_ERR_WORKSPACE,
         "forward(ws short)");
  expect(moe_tail_forward(&d, &w, X, 16, X, 32, &r, OUT + 4, SOUT, WS, need, nullptr), MOE_TAIL_ERR_INVALID,
         "forward(misaligned out)");
  expect(moe_tail_forward_add3(&d, &w, X, 16, X, 16, &r, nullptr, OUT, nullptr, WS, need16, nullptr),
         MOE_TAIL_ERR_INVALID, "add3(no residual)");
  expect(moe_tail_forward_fused(&d, &w, X, 16, X, 129, &r, nullptr, OUT, SOUT,
                                WS, moe_tail_workspace_bytes(&d, 16, 129), nullptr),
         MOE_TAIL_ERR_UNSUPPORTED, "fused(Ms 129)");
  expect(moe_tail_forward_fused_bounded(&d, &w, X, 16, X, 16, &r, nullptr, OUT, nullptr, WS, need16, nullptr, -1),
         MOE_TAIL_ERR_INVALID, "fused_bounded(-1)");
  expect(moe_tail_forward_profiled(&d, &w, X, 16, X, 16, &r, OUT, nullptr, WS, need16, nullptr, nullptr),
         MOE_TAIL_ERR_INVALID, "profiled(no events)");
  expect(moe_tail_forward_timed(&d, &w, X, 16, X, 16, &r, nullptr, OUT, nullptr, WS, need16, nullptr, nullptr),
         MOE_TAIL_ERR_INVALID, "timed(no events)");
  const moe_tail_dims big = dims(8, 8, 512, 256);
  expect(moe_tail_forward_noalloc(&big, &w, X, 512, X, 512, &r, OUT, nullptr, nullptr), MOE_TAIL_ERR_WORKSPACE,
         "noalloc(beyond its scratch)");
  expect(moe_tail_forward_noalloc(&d, &w, X, 17, X, 16, &r, OUT, nullptr, nullptr), MOE_TAIL_ERR_INVALID,
         "noalloc(Mr > Ms)");
  const moe_tail_dims d4 = dims(64, 8, 2048, 2048, MOE_TAIL_W_MXFP4);
  const uint8_t* A = static_cast<const uint8_t*>(addr(1ull << 44));
  uint8_t* P = static_cast<uint8_t*>(addr(1ull << 45));
  expect(moe_tail_pack_mxfp4_scales(&d, A, nullptr, P, nullptr, nullptr), MOE_TAIL_ERR_INVALID, "pack(fp8 dims)");
  expect(moe_tail_pack_mxfp4_scales(&d4, A, nullptr, nullptr, nullptr, nullptr), MOE_TAIL_ERR_INVALID,
         "pack(no output)");
  expect(moe_tail_pack_mxfp4_scales(&d4, nullptr, nullptr, nullptr, nullptr, nullptr), MOE_TAIL_OK,
         "pack(nothing)");
  const moe_tail_dims dn = dims(64, 8, 2048, 2048, MOE_TAIL_W_NVFP4);
  expect(moe_tail_pack_nvfp4_scales(&d4, A, nullptr, P, nullptr, nullptr), MOE_TAIL_ERR_INVALID, "pack_nv(mxfp4 dims)");
  expect(moe_tail_pack_nvfp4_scales(&dn, P, nullptr, P + 64, nullptr, nullptr), MOE_TAIL_ERR_INVALID,
         "pack_nv(overlap)");
  expect(moe_tail_pack_nvfp4_scales(&dn, nullptr, nullptr, nullptr, nullptr, nullptr), MOE_TAIL_OK, "pack_nv(nothing)");
  expect(moe_tail_quant_fp8_1x128(X, 1, 4, 100, static_cast<uint8_t*>(addr(1ull << 43)),
                                  static_cast<float*>(addr(1ull << 44)), nullptr),
         MOE_TAIL_ERR_INVALID, "quant(cols 100)");
  expect(moe_tail_probe_mfma_fp8(A, A, static_cast<float*>(addr(1ull << 43)), 0, nullptr), 1, "probe_mfma(n 0)");
  expect(moe_tail_probe_copy(P, P + 16, 4096, nullptr), 1, "probe_copy(overlap)");
  expect(moe_tail_probe_stream_read(A, 4000, static_cast<uint32_t*>(addr(1ull << 43)), 0, nullptr), 1,
         "probe_stream_read(size)");
  for (int s = -1; s <= 5; ++s)
    if (moe_tail_strerror(s) == nullptr) expect(1, 0, "strerror");

  std::printf("abi driver: %s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
