// gfx950 matrix-core helpers (CDNA4, wave64).
//
// v_mfma_f32_32x32x16_bf16 computes C[32x32] += A[32x16] * B[16x32] per wave:
//   A: lane l holds A[l % 32][(l / 32) * 8 + e], e = 0..7 (8 bf16, 16 bytes)
//   B: lane l holds B[(l / 32) * 8 + e][l % 32], e = 0..7
//   C: lane l holds C[(i / 4) * 8 + (l / 32) * 4 + (i % 4)][l % 32], i = 0..15
// Every kernel that relies on this layout is checked against the CPU oracle by
// the GPU parity tests.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ab {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace ab
