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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Instruction classes of __builtin_amdgcn_sched_group_barrier (LLVM AMDGPU): a
// group of matrix-core instructions and a group of LDS reads.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ f32x16_t mfma32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// v_permlane32_swap with the same value in both operands: result[0] holds
// x[l % 32] and result[1] holds x[l % 32 + 32] in every lane l, so a commutative
// combine of the two is the pair result of lanes l and l ^ 32 (identical in both).
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// (i % 4) of the 4-element (8-byte) chunks addressed by lanes i/4, i/4 + 4,
// i/4 + 8 and i/4 + 12 of its group (verified on gfx950).
__device__ __forceinline__ uint2 lds_read_tr16(const void* lds_ptr) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_t*)((__attribute__((address_space(3))) char*)(lds_ptr)));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Asynchronous 16-byte buffer load straight into LDS: lane L's bytes land at
// lds_base + 16 * L (lds_base must be wave-uniform); an offset past the buffer's
// size loads zeros (verified on gfx950).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) char*)lds_base), 16, voffset, 0,
      0, 0);
}

// 16-byte chunk permutation of an unpadded [key][d] bf16 tile in LDS that makes the
// MFMA fragment read (32 consecutive rows, same chunk, 16 bytes per lane)
// conflict-free on gfx950 (measured).
template <int D>
__device__ __forceinline__ int kfrag_swz(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

}  // namespace ab
