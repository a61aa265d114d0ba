// Device helpers shared by the tail's kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe_tail {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> e4m3 ("fn": bias 7, max 448, no infinities) code: the gfx950
// conversion instruction, which rounds to nearest even, saturates to +-448
// and keeps the sign bit of the input (including -0).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false)) & 0xffu;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// max over the 16 lanes that share lane / 16
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float silu_mul(float gate, float up) { return (gate / (1.0f + expf(-gate))) * up; }

// silu(gate) * up with the hardware exp2 and reciprocal (about one ulp each),
// for values that are re-quantized to FP8 right after
__device__ __forceinline__ float silu_mul_fast(float gate, float up) {
  const float e = __builtin_amdgcn_exp2f(gate * -1.44269504088896341f);
  return gate * __builtin_amdgcn_rcpf(1.0f + e) * up;
}

// 16x16x128 FP8 x FP8 block product (e4m3 both sides, unit scales).
__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}

// 16x16x128 FP8 (A) x FP4 e2m1 (B) with one e8m0 scale per lane on B.
__device__ __forceinline__ f32x4 mfma_fp8_fp4(const i32x8& a, const i32x8& b, int scale_b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 4, 0, 127, 0, scale_b);
}

// 16x16x128 FP4 e2m1 (A, one e8m0 scale per lane) x FP8 e4m3 (B).
__device__ __forceinline__ f32x4 mfma_fp4_fp8(const i32x8& a, int scale_a, const i32x8& b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 0, 0, scale_a, 0, 127);
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// FP8 x NVFP4 on the FP16 matrix cores (16x16x32, FP32 accumulation).  The
// FP8 fragment `a` is the 8-bit operand layout (lane group g: K [16 g,
// 16 g + 16) in registers 0-3, K [64 + 16 g, +16) in 4-7); the weight
// fragment `b` holds the same K of the lane's weight row as e2m1 pairs
// (registers 0-1: K [16 g, +16), 2-3: K [64 + 16 g, +16), the even K in the
// low nibble) and `scales` the e4m3 scales of those two 16-element blocks
// (bytes 0 and 1).  Every conversion is exact: e4m3 and e2m1 values are FP16
// values, and an e2m1 times an e4m3 has at most six significant bits, within
// the FP16 range (2^-10 .. 2688).  Chunk m (eight K elements, registers 2m
// and 2m + 1 of `a`, register m of `b`) of the block is the m-th MFMA for
// both operands.

// the four FP16 chunks of an FP8 fragment
__device__ __forceinline__ void fp8_frag_f16(const i32x8& a, f16x8 x[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const unsigned a0 = static_cast<unsigned>(a[2 * m]), a1 = static_cast<unsigned>(a[2 * m + 1]);
    const f16x2 x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a0, 1.0f, false);
    const f16x2 x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a0, 1.0f, true);
    const f16x2 x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a1, 1.0f, false);
    const f16x2 x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a1, 1.0f, true);
    x[m] = f16x8{x0.x, x0.y, x1.x, x1.y, x2.x, x2.y, x3.x, x3.y};
  }
}

// the four FP16 chunks of an NVFP4 fragment: e2m1 times its e4m3 block scale
__device__ __forceinline__ void nvfp4_frag_f16(const i32x8& b, int scales, f16x8 w[4]) {
  const f16x2 s_lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<unsigned>(scales) & 0xffu, 1.0f, false);
  const f16x2 s_hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((static_cast<unsigned>(scales) >> 8) & 0xffu, 1.0f, false);
  const f16x2 slo = {s_lo.x, s_lo.x}, shi = {s_hi.x, s_hi.x};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const unsigned v = static_cast<unsigned>(b[m]);
    const f16x2 s = (m < 2) ? slo : shi;
    const f16x2 w0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 0) * s;
    const f16x2 w1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 1) * s;
    const f16x2 w2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 2) * s;
    const f16x2 w3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, 3) * s;
    w[m] = f16x8{w0.x, w0.y, w1.x, w1.y, w2.x, w2.y, w3.x, w3.y};
  }
}

// one 128-wide K block from converted chunks, the activation block as A
// (acc[i]: activation row 4 g + i, weight row l16) or, with the operands
// swapped, the weight block as A (weight row 4 g + i, activation row l16);
// no activation or matrix scale
__device__ __forceinline__ f32x4 mfma_f16_block(const f16x8 a[4], const f16x8 b[4]) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < 4; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[m], b[m], acc, 0, 0, 0);
  return acc;
}

// FP8 activations (A) x NVFP4 weights (B) for one 128-wide K block
__device__ __forceinline__ f32x4 mfma_fp8_nvfp4(const i32x8& a, const i32x8& b, int scales) {
  f16x8 x[4], w[4];
  fp8_frag_f16(a, x);
  nvfp4_frag_f16(b, scales, w);
  return mfma_f16_block(x, w);
}

// ------------------------------------------------ direct global -> LDS loads

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
// (soff is wave-uniform by construction; readfirstlane keeps it in a scalar
// register where the compiler cannot prove that.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const uint8_t* lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds_offset(lds)), "v"(voff), "s"(r),
               "s"(__builtin_amdgcn_readfirstlane(soff)));
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, const uint8_t* lds, uint32_t voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds_offset(lds)), "v"(voff), "s"(r),
               "s"(__builtin_amdgcn_readfirstlane(soff)));
}

// Wait until at most N of this wave's direct loads are in flight and its LDS
// reads are done, then meet the other waves: afterwards every load issued
// before the newest N (by any wave) has landed.  (A fenced __syncthreads
// would wait for all of them.)
template <int N>
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only (a fenced __syncthreads would also
// wait for the direct loads in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Buffer resource for `bytes` bytes at `base` (wave-uniform; read through
// readfirstlane so that it lives in scalar registers, as the loads need).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // (readfirstlane returns int: convert through uint32_t, never sign-extend)
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32))));
  const uint32_t n = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(bytes)));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo),
                                           static_cast<short>(0), n, 0x00020000);
}

}  // namespace moe_tail
