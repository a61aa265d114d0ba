// Measurement probes beside the tail library (include/moe_tail_probes.h):
// the routed GEMMs' FP8 block product on given operands, a copy of known
// size for calibrating the HBM byte counters, a streaming read, and the
// per-workgroup rates of the load paths the GEMMs use.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/moe_tail_probes.h"
#include "common.hpp"

using namespace moe_tail;

namespace {

// One wave per product.  Lane (r = lane % 16, g = lane / 16) holds, of row r
// of each operand, the K elements [16 g, 16 g + 16) and [64 + 16 g, +16):
// the 8-bit operand layout the routed GEMMs use.  Result register i of lane
// (r, g) is c[4 g + i][r].
__global__ __launch_bounds__(64) void k_probe_mfma_fp8(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                      float* __restrict__ c) {
  const int lane = threadIdx.x, r = lane & 15, g = lane >> 4;
  const size_t base = static_cast<size_t>(blockIdx.x) * 16 * 128;
  const uint8_t* ar = a + base + r * 128;
  const uint8_t* br = b + base + r * 128;
  const i32x4 alo = *reinterpret_cast<const i32x4*>(ar + 16 * g);
  const i32x4 ahi = *reinterpret_cast<const i32x4*>(ar + 64 + 16 * g);
  const i32x4 blo = *reinterpret_cast<const i32x4*>(br + 16 * g);
  const i32x4 bhi = *reinterpret_cast<const i32x4*>(br + 64 + 16 * g);
  const i32x8 a8 = __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7);
  const i32x8 b8 = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
  const f32x4 v = mfma_fp8(a8, b8);
  float* cr = c + static_cast<size_t>(blockIdx.x) * 256;
#pragma unroll
  for (int i = 0; i < 4; ++i) cr[(4 * g + i) * 16 + r] = v[i];
}

__global__ __launch_bounds__(256) void k_probe_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// Workgroup b reads 4 KB rows b, b + grid, ...; each thread one 16-byte piece
// of a row, eight rows' loads in flight before any is used.
constexpr int kReadUnroll = 8;

__global__ __launch_bounds__(256) void k_probe_stream_read(const i32x4* __restrict__ src, size_t rows,
                                                           uint32_t* __restrict__ sink, uint32_t magic) {
  int acc = 0;
  const size_t g = gridDim.x;
  size_t row = blockIdx.x;
  for (; row + (kReadUnroll - 1) * g < rows; row += kReadUnroll * g) {
    i32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + (row + u * g) * 256 + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; row < rows; row += g) {
    const i32x4 v = __builtin_nontemporal_load(src + row * 256 + threadIdx.x);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (static_cast<uint32_t>(acc) == magic) sink[0] = magic;
}

// ------------------------------------------------------ load paths --
// Per-workgroup streaming through the load paths the GEMMs use, nothing
// computed: workgroup b reads its run of `per` bytes (src + b per, or all the
// same run when `shared`).  The LDS ring has kPathStages stages of 32 KB
// (kPathStages - 1 in flight): each wave issues 4 direct loads of 1 KB per
// stage, waits for the oldest stage of its own and meets the other waves
// before reusing a slot, as the tiled kernels do.
constexpr int kPathStages = 4;
constexpr int kPathStage = 32 * 1024;
constexpr int kPathRegs = 16;  // register ring: loads in flight per lane

// mode 0: stage s = bytes [32 KB s, +32 KB); mode 1: stage s = bytes
// [128 k, +128) of each of the 256 rows (of row_bytes bytes) of matrix m,
// s = m (row_bytes / 128) + k, load i of wave w rows 8 (w + 8 i) ..
// 8 (w + 8 i) + 7 (the weight-tile pattern).
template <int kMode>
__global__ __launch_bounds__(512) void k_probe_path_lds(const uint8_t* __restrict__ src, uint32_t per, int shared,
                                                        int row_bytes, uint32_t* __restrict__ sink, uint32_t magic) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kPathStages * kPathStage];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint8_t* base = src + (shared ? 0 : static_cast<size_t>(blockIdx.x) * per);
  const int ksteps = row_bytes / 128;
  const int nst = static_cast<int>(per / kPathStage);
  const int q8 = lane >> 3, c = lane & 7;
  auto issue = [&](int s) {
    uint8_t* st = ring + (s % kPathStages) * kPathStage;
    const bool live = s < nst;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, live ? per : 0u);  // past the run: no bytes, zeros
    int soff = 0;
    if (live) soff = (kMode == 0) ? s * kPathStage : (s / ksteps) * 256 * row_bytes + 128 * (s % ksteps);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int blk = wv + 8 * i;
      const uint32_t voff = (kMode == 0) ? 1024u * blk + 16u * lane
                                         : static_cast<uint32_t>((8 * blk + q8) * row_bytes + 16 * c);
      dma16(r, st + 1024 * blk, voff, soff);
    }
  };
  for (int s = 0; s < kPathStages - 1; ++s) issue(s);
  for (int s = 0; s < nst; ++s) {
    ring_barrier<4 * (kPathStages - 2)>();
    issue(s + kPathStages - 1);
  }
  ring_barrier<0>();
  // word t of the last stage that read bytes (the trailing stages read none)
  const uint32_t v = reinterpret_cast<const uint32_t*>(ring + ((nst - 1) % kPathStages) * kPathStage)[threadIdx.x];
  if (v == magic) sink[0] = magic;
}

// mode 2: step s = bytes [8 KB s, +8 KB), lane t of the workgroup bytes
// [16 t, +16); mode 3: the same 8 KB as 64 rows of 128 bytes, wave w taking
// rows 16 (w / 2) .. + 15, half w % 2: 16 rows x 64 bytes per load (half
// lines).  kPathRegs loads in flight per lane.
template <int kMode>
__global__ __launch_bounds__(512) void k_probe_path_regs(const uint8_t* __restrict__ src, uint32_t per, int shared,
                                                         uint32_t* __restrict__ sink, uint32_t magic) {
  const uint8_t* base = src + (shared ? 0 : static_cast<size_t>(blockIdx.x) * per);
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, per);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t lo = (kMode == 2) ? 16u * threadIdx.x
                                   : static_cast<uint32_t>((16 * (wave >> 1) + (lane & 15)) * 128 + 64 * (wave & 1) +
                                                           16 * (lane >> 4));
  const int nsteps = static_cast<int>(per / 8192);
  constexpr uint32_t kPast = 0x80000000u;  // past any run: reads zeros
  i32x4 v[kPathRegs];
#pragma unroll
  for (int u = 0; u < kPathRegs; ++u)
    v[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, u < nsteps ? lo + 8192u * u : kPast, 0, 0));
  int acc = 0;
  for (int s = kPathRegs; s < nsteps + kPathRegs; s += kPathRegs) {
#pragma unroll
    for (int u = 0; u < kPathRegs; ++u) {
      acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
      const uint32_t off = (s + u < nsteps) ? lo + 8192u * static_cast<uint32_t>(s + u) : kPast;
      v[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
  }
  if (static_cast<uint32_t>(acc) == magic) sink[0] = magic;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? 0 : 4; }

}  // namespace

extern "C" {

int moe_tail_probe_mfma_fp8(const uint8_t* a, const uint8_t* b, float* c, int32_t n, void* stream) {
  if (n < 1 || n > 65536 || a == nullptr || b == nullptr || c == nullptr) return 1;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return 1;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_probe_mfma_fp8, dim3(static_cast<unsigned>(n)), dim3(64), 0, static_cast<hipStream_t>(stream),
                     a, b, c);
  return launched();
}

int moe_tail_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes % 16 || (bytes > 0 && (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst)))) return 1;
  const char *s = static_cast<const char*>(src), *d = static_cast<const char*>(dst);
  if (bytes > 0 && s < d + bytes && d < s + bytes) return 1;
  if (bytes == 0) return 0;
  (void)hipGetLastError();
  const size_t n = bytes / 16;
  const unsigned grid = static_cast<unsigned>(n / 256 < 8192 ? (n + 255) / 256 : 8192);
  hipLaunchKernelGGL(k_probe_copy, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return launched();
}

int moe_tail_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, uint32_t magic, void* stream) {
  if (bytes % 4096 || sink == nullptr || (bytes > 0 && (src == nullptr || !aligned16(src)))) return 1;
  if (bytes == 0) return 0;
  (void)hipGetLastError();
  const size_t rows = bytes / 4096;
  const unsigned grid = static_cast<unsigned>(rows < 4096 ? rows : 4096);
  hipLaunchKernelGGL(k_probe_stream_read, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const i32x4*>(src), rows, sink, magic);
  return launched();
}

int moe_tail_probe_stream_paths(const void* src, size_t per_wg, int32_t grid, int32_t shared, int32_t mode,
                                int32_t row_bytes, uint32_t* sink, uint32_t magic, void* stream) {
  if (src == nullptr || sink == nullptr || !aligned16(src) || grid < 1 || grid > 65535 || mode < 0 || mode > 3)
    return 1;
  if (per_wg == 0 || per_wg % kPathStage != 0 || per_wg >= (size_t{1} << 31)) return 1;
  if (mode == 1 && (row_bytes < 128 || row_bytes % 128 != 0 || per_wg % (size_t{256} * row_bytes) != 0)) return 1;
  (void)hipGetLastError();
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t per = static_cast<uint32_t>(per_wg);
  const int sh = shared ? 1 : 0;
  if (mode == 0)
    hipLaunchKernelGGL(k_probe_path_lds<0>, dim3(grid), dim3(512), 0, st, static_cast<const uint8_t*>(src), per, sh,
                       128, sink, magic);
  else if (mode == 1)
    hipLaunchKernelGGL(k_probe_path_lds<1>, dim3(grid), dim3(512), 0, st, static_cast<const uint8_t*>(src), per, sh,
                       static_cast<int>(row_bytes), sink, magic);
  else if (mode == 2)
    hipLaunchKernelGGL(k_probe_path_regs<2>, dim3(grid), dim3(512), 0, st, static_cast<const uint8_t*>(src), per, sh,
                       sink, magic);
  else
    hipLaunchKernelGGL(k_probe_path_regs<3>, dim3(grid), dim3(512), 0, st, static_cast<const uint8_t*>(src), per, sh,
                       sink, magic);
  return launched();
}

}  // extern "C"
