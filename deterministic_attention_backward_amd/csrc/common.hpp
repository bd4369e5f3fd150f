// Device types and small helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

// v_mfma_f32_32x32x16_bf16. Lane l of the wave (h = l / 32):
//   A (32 x 16): row l % 32, k = 8h + e (e = element 0..7 of the bf16x8)
//   B (16 x 32): col l % 32, k = 8h + e
//   C (32 x 32): col l % 32, row 8 (i / 4) + 4h + (i % 4) for accumulator i = 0..15
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// Round-to-nearest-even float -> bfloat16 (gfx950 converts in hardware).
__device__ __forceinline__ bf16 to_bf16(float x) { return (bf16)x; }

// Eight consecutive accumulators (a 16-wide k-chunk of a C tile) as an MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = to_bf16(v[base + e]);
  return r;
}

__device__ __forceinline__ bf16x8 cat44(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// base + a 32-bit byte offset: with a wave-uniform base this lets the compiler
// use SGPR-base addressing instead of building a 64-bit address per lane.
template <class T>
__device__ __forceinline__ T* at_bytes(T* base, unsigned byte_off) {
  return (T*)((char*)base + byte_off);
}
template <class T>
__device__ __forceinline__ const T* at_bytes(const T* base, unsigned byte_off) {
  return (const T*)((const char*)base + byte_off);
}

// Wait until every vector memory operation this wave issued has completed
// (s_waitcnt vmcnt(0); expcnt and lgkmcnt left unconstrained).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace attn
