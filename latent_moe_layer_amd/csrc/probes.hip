// Measurement probes beside the tail library (include/moe_tail_probes.h):
// the routed GEMMs' FP8 block product on given operands, a copy of known
// size for calibrating the HBM byte counters, and a streaming read.
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

}  // extern "C"
