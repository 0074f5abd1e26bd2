// IBCS clustering: fixed-iteration k-means of the queries of every query block.
//
// AB-Attention abstract (paperdot search page, query "Xing Ma"), IBCS sentence:
// the queries of each query block are clustered on their own, tokens stay in
// place. The clustering is specified operation by operation in fp32 so that the
// result is reproducible bit for bit on any implementation:
//   * a query x is compared with centroid mu through |mu|^2 - 2 x.mu (the squared
//     distance less |x|^2, so the nearest centroid is the same): |mu|^2, then one
//     fused multiply-add of x_k * (-2 mu_k) per dimension in ascending k;
//   * |mu|^2 = products mu_k^2 rounded one by one, summed by the halving tree
//     (k with k+32, then k+16, ..., k+1) inside each group of 64 dimensions, the
//     group sums then added in order;
//   * assignment to the nearest centroid, ties to the lowest cluster index;
//   * centroid = fp32 sum of its members in ascending row order, divided by the
//     member count with one correctly rounded division; an empty cluster keeps
//     its centroid and gets size 0;
//   * initial centroids are the strided queries x[floor(c*n/C')], C' = min(C, n).
//
// One workgroup per (b, h, query block), two threads per query row: each keeps
// its query in VGPRs and scans four of every eight clusters with four fused
// multiply-add chains whose centroid operand, -2 mu, comes from registers by a
// DPP broadcast (each wave holds its clusters' -2 mu for dims 16g + lane % 16 in
// every 16-lane row), so the loop reads no LDS; the two halves then merge their
// minima (lower index wins ties). The update uses per-cluster member lists built
// with wave ballots; a wave owns whole clusters and sums their members for its
// lane's dims in ascending row order from the block's copy in LDS (bf16 rows of
// 128 dims: one 32-bit read of a dim pair per member), and the norm tree is a
// butterfly of xor shuffles (the adds commute exactly, so the lane holding the
// tree's root ends with its value).
#include "ab_internal.h"

namespace ab {
namespace {

// Separately rounded fp32 operations. HIP's __fmul_rn and __fadd_rn are plain
// operators defined in its headers, where contraction is allowed, so once
// inlined they can still be fused into an FMA; these helpers carry the
// no-contraction setting of their own bodies instead.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}
__device__ __forceinline__ float add_rn(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// Each thread keeps one query in VGPRs (bf16 pairs packed, unpacked at use); the
// block also sits in LDS (its input type) for the centroid update.
template <bool BF16, int D>
struct QueryRow {
  static constexpr int kWords = BF16 ? D / 2 : D;
  uint32_t w[kWords];
  __device__ __forceinline__ float get(int k) const {
    if constexpr (BF16) return (k & 1) ? __uint_as_float(w[k >> 1] & 0xFFFF0000u) : __uint_as_float(w[k >> 1] << 16);
    else return __uint_as_float(w[k]);
  }
};

// acc[u] += sl[u] (from lane J0 + j of the lane's 16-lane row) * xv[j], u < 4,
// j < 8, each a fused multiply-add with one rounding; the centroid operand is
// broadcast with DPP row_newbcast, so every lane of the wave must be active. The
// leading s_nop gives a DPP read of its source the wait states it needs after a
// VALU write.
template <int J0>
__device__ __forceinline__ void fma8_bcast(float (&acc)[4], const float (&sl)[4], const float (&xv)[8]);
template <>
__device__ __forceinline__ void fma8_bcast<0>(float (&acc)[4], const float (&sl)[4], const float (&xv)[8]) {
  asm volatile(
        "s_nop 1\n"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(sl[0]), "v"(sl[1]), "v"(sl[2]), "v"(sl[3]), "v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]),
          "v"(xv[4]), "v"(xv[5]), "v"(xv[6]), "v"(xv[7]));
}
template <>
__device__ __forceinline__ void fma8_bcast<8>(float (&acc)[4], const float (&sl)[4], const float (&xv)[8]) {
  asm volatile(
        "s_nop 1\n"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %8 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %9 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %10 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %12 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %13 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %14 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %4, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %5, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %6, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %7, %15 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(sl[0]), "v"(sl[1]), "v"(sl[2]), "v"(sl[3]), "v"(xv[0]), "v"(xv[1]), "v"(xv[2]), "v"(xv[3]),
          "v"(xv[4]), "v"(xv[5]), "v"(xv[6]), "v"(xv[7]));
}

// The same for bf16 queries: xw holds the eight dims as four packed pairs (low
// half the even dim), unpacked inside the block so that the unpacked values are
// never live outside it; the eight unpacking instructions also provide the DPP
// wait states.
template <int J0>
__device__ __forceinline__ void fma8_bcast_bf16(float (&acc)[4], const float (&sl)[4], const uint32_t* xw);
template <>
__device__ __forceinline__ void fma8_bcast_bf16<0>(float (&acc)[4], const float (&sl)[4], const uint32_t* xw) {
  float t[8];
  asm volatile(
        "v_lshlrev_b32 %4, 16, %16\n"
        "v_and_b32 %5, 0xffff0000, %16\n"
        "v_lshlrev_b32 %6, 16, %17\n"
        "v_and_b32 %7, 0xffff0000, %17\n"
        "v_lshlrev_b32 %8, 16, %18\n"
        "v_and_b32 %9, 0xffff0000, %18\n"
        "v_lshlrev_b32 %10, 16, %19\n"
        "v_and_b32 %11, 0xffff0000, %19\n"
        "v_fmac_f32_dpp %0, %12, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]),
          "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(sl[0]), "v"(sl[1]), "v"(sl[2]), "v"(sl[3]), "v"(xw[0]), "v"(xw[1]), "v"(xw[2]), "v"(xw[3]));
}
template <>
__device__ __forceinline__ void fma8_bcast_bf16<8>(float (&acc)[4], const float (&sl)[4], const uint32_t* xw) {
  float t[8];
  asm volatile(
        "v_lshlrev_b32 %4, 16, %16\n"
        "v_and_b32 %5, 0xffff0000, %16\n"
        "v_lshlrev_b32 %6, 16, %17\n"
        "v_and_b32 %7, 0xffff0000, %17\n"
        "v_lshlrev_b32 %8, 16, %18\n"
        "v_and_b32 %9, 0xffff0000, %18\n"
        "v_lshlrev_b32 %10, 16, %19\n"
        "v_and_b32 %11, 0xffff0000, %19\n"
        "v_fmac_f32_dpp %0, %12, %4 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %4 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %4 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %4 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %5 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %5 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %5 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %5 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %6 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %6 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %6 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %6 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %7 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %8 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %9 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %10 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %0, %12, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %1, %13, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %2, %14, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        "v_fmac_f32_dpp %3, %15, %11 row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]),
          "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]), "=&v"(t[6]), "=&v"(t[7])
        : "v"(sl[0]), "v"(sl[1]), "v"(sl[2]), "v"(sl[3]), "v"(xw[0]), "v"(xw[1]), "v"(xw[2]), "v"(xw[3]));
}

// Two threads per query row: thread t handles row t % Bq and the clusters
// c = c0 + 4*(t / Bq) + u (u < 4) of every group of 8.
template <bool BF16, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BF16 ? 4 : 2))) void kmeans_kernel(
    Dims P, const void* __restrict__ qv, float* __restrict__ cent, uint16_t* __restrict__ cent_bf16,
    int32_t* __restrict__ sizes_out, uint8_t* __restrict__ assign_out) {
  static_assert(D % 64 == 0, "a wave covers 64 dims of one cluster");
  constexpr int G = D / 64;  // 64-dim groups of the centroid norm
  extern __shared__ __align__(16) unsigned char smem[];
  const int Bq = P.Bq, C = P.C;
  const int CP = (C + 7) & ~7;  // padded cluster count of the transposed centroid table
  const int blk = blockIdx.x;   // (b*H + h)*nqb + i
  const int i = blk % P.nqb;
  const int bh = blk / P.nqb;
  const int row0 = i * Bq;
  const int n = min(Bq, P.N - row0);
  const int Ci = min(C, n);
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;  // 2 * Bq
  const int r_own = tid % Bq, chalf = tid / Bq;

  // LDS carve-up
  using elem_t = typename std::conditional<BF16, uint16_t, float>::type;
  elem_t* X = reinterpret_cast<elem_t*>(smem);                                       // [Bq][D]
  float* m2_t = reinterpret_cast<float*>(smem + size_t(Bq) * D * sizeof(elem_t));    // [D][CP]: -2 * mu
  float* npart = m2_t + size_t(D) * CP;                                              // [CP][G] norm partials
  int* asg = reinterpret_cast<int*>(npart + size_t(CP) * G);                         // [Bq]
  float* pbest = reinterpret_cast<float*>(asg + Bq);                                 // [Bq] best of the upper half
  int* pidx = reinterpret_cast<int*>(pbest + Bq);                                    // [Bq]
  int* ccount = pidx + Bq;                                                           // [C], padded to 16 bytes
  uint8_t* list = reinterpret_cast<uint8_t*>(ccount + ((C + 3) & ~3));               // [C][Bq] member rows

  // this thread's query, held in VGPRs for every iteration (16-byte global loads);
  // the two threads of a row each copy one half of it into the block's LDS copy
  const elem_t* qsrc = reinterpret_cast<const elem_t*>(qv) + (size_t(bh) * P.N + row0) * D;
  for (int p = tid; p < D * CP + CP * G; p += nthr) m2_t[p] = 0.0f;
  QueryRow<BF16, D> x;
  {
    constexpr int kChunks = QueryRow<BF16, D>::kWords / 4;  // 16-byte chunks of a row
    const uint4* src = reinterpret_cast<const uint4*>(qsrc + size_t(min(r_own, n - 1)) * D);
    uint4* dst = reinterpret_cast<uint4*>(X) + r_own * kChunks;
#pragma unroll
    for (int c4 = 0; c4 < kChunks; ++c4) {
      const uint4 u = src[c4];
      x.w[4 * c4 + 0] = u.x;
      x.w[4 * c4 + 1] = u.y;
      x.w[4 * c4 + 2] = u.z;
      x.w[4 * c4 + 3] = u.w;
      if (r_own < n && c4 / (kChunks / 2) == chalf) dst[c4] = u;
    }
  }
  __syncthreads();
  auto xlds = [&](int r, int k) -> float {
    if constexpr (BF16) return bf16_to_f32(X[r * D + k]); else return X[r * D + k];
  };
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // A wave owns whole clusters (c = wave, wave + waves, ...) when centroids are set;
  // lane l holds dims 64g + l (g < G). finish_cluster stores -2 mu and the norm
  // partials, the G halving-tree butterflies side by side.
  auto finish_cluster = [&](int c, const float (&mu)[G]) {
    float t[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m2_t[(64 * g + lane) * CP + c] = -2.0f * mu[g];  // exact
      t[g] = mul_rn(mu[g], mu[g]);
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1)
#pragma unroll
      for (int g = 0; g < G; ++g) t[g] = add_rn(t[g], __shfl_xor(t[g], sh, 64));
    if (lane == 0)
#pragma unroll
      for (int g = 0; g < G; ++g) npart[c * G + g] = t[g];
  };
  // bf16 rows of 128 dims in the update: lane l holds dims 2l and 2l+1 (one 32-bit
  // read per member). Its halving tree: dims k and k+32 are lanes l and l^16, k and
  // k+16 lanes l and l^8, ..., k and k+2 lanes l and l^1, then k and k+1 the two
  // halves of lane 0 (dims 0-63) and of lane 32 (dims 64-127).
  constexpr bool kPairs = BF16 && D == 128;
  auto finish_pair = [&](int c, float mu0, float mu1) {
    m2_t[(2 * lane) * CP + c] = -2.0f * mu0;  // exact
    m2_t[(2 * lane + 1) * CP + c] = -2.0f * mu1;
    float t0 = mul_rn(mu0, mu0), t1 = mul_rn(mu1, mu1);
#pragma unroll
    for (int sh = 16; sh >= 1; sh >>= 1) {
      t0 = add_rn(t0, __shfl_xor(t0, sh, 64));
      t1 = add_rn(t1, __shfl_xor(t1, sh, 64));
    }
    const float t = add_rn(t0, t1);
    if ((lane & 31) == 0) npart[c * G + (lane >> 5)] = t;
  };
  for (int c = wave; c < Ci; c += nthr >> 6) {
    float mu[G];
#pragma unroll
    for (int g = 0; g < G; ++g) mu[g] = xlds((c * n) / Ci, 64 * g + lane);
    finish_cluster(c, mu);
  }
  if (tid < C) ccount[tid] = 0;
  __syncthreads();

  for (int it = 0; it < P.T; ++it) {
    // ---- assignment: each half of the threads scans 4 of every 8 clusters ----
    // distance up to the row's own |x|^2: |mu|^2 + sum_k x_k * (-2 mu_k), one fused
    // multiply-add per term in ascending k. Every lane computes (rows past the block
    // end repeat its last row) so that the DPP broadcasts see a full wave; each wave
    // reads its four clusters' -2 mu for dims 16g + (lane % 16) into registers, one
    // 16-byte LDS read per 16 dims.
    float best = __builtin_inff();
    int bi = 0;
    for (int c0 = 0; c0 < Ci; c0 += 8) {
      const int cb = c0 + 4 * chalf;
      float acc[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        float a = npart[(cb + cc) * G];
#pragma unroll
        for (int g = 1; g < G; ++g) a = add_rn(a, npart[(cb + cc) * G + g]);
        acc[cc] = a;
      }
#pragma unroll
      for (int g = 0; g < D / 16; ++g) {
        const float4 v = *reinterpret_cast<const float4*>(&m2_t[(16 * g + (lane & 15)) * CP + cb]);
        const float sl[4] = {v.x, v.y, v.z, v.w};
        if constexpr (BF16) {
          fma8_bcast_bf16<0>(acc, sl, &x.w[8 * g]);
          fma8_bcast_bf16<8>(acc, sl, &x.w[8 * g + 4]);
        } else {
          float xa[8], xb[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            xa[e] = x.get(16 * g + e);
            xb[e] = x.get(16 * g + 8 + e);
          }
          fma8_bcast<0>(acc, sl, xa);
          fma8_bcast<8>(acc, sl, xb);
        }
      }
      const int lim = min(4, Ci - cb);
      for (int cc = 0; cc < lim; ++cc) {
        if (acc[cc] < best) {
          best = acc[cc];
          bi = cb + cc;
        }
      }
    }
    // merge the two halves: the lower cluster index wins ties. Within each half the
    // scan is in ascending cluster order, but the halves interleave (0-3 | 4-7, 8-11 |
    // 12-15, ...), so ties are broken by index explicitly.
    if (chalf == 1 && r_own < n) {
      pbest[r_own] = best;
      pidx[r_own] = bi;
    }
    __syncthreads();
    if (chalf == 0 && r_own < n) {
      const float ob = pbest[r_own];
      const int oi = pidx[r_own];
      if (ob < best || (ob == best && oi < bi)) bi = oi;
      asg[r_own] = bi;
    }
    __syncthreads();
    // ---- member lists (ascending rows per cluster); wave w builds clusters w, w + waves, ... ----
    {
      const int nwaves = nthr >> 6;
      int a_lo = -1, a_hi = -1;  // assignments of rows lane and 64 + lane
      if (lane < n) a_lo = asg[lane];
      if (64 + lane < n) a_hi = asg[64 + lane];
      for (int c = wave; c < Ci; c += nwaves) {
        uint8_t* lc = list + c * Bq;
        const uint64_t m_lo = __ballot(a_lo == c);
        const uint64_t m_hi = __ballot(a_hi == c);
        const uint64_t below = (uint64_t(1) << lane) - 1;
        if (a_lo == c) lc[__popcll(m_lo & below)] = uint8_t(lane);
        if (a_hi == c) lc[__popcll(m_lo) + __popcll(m_hi & below)] = uint8_t(64 + lane);
        if (lane == 0) ccount[c] = __popcll(m_lo) + __popcll(m_hi);
      }
    }
    __syncthreads();
    // ---- update: members summed in ascending row order, one correctly rounded division ----
    // Each wave sums the members of its clusters for dims 64g + lane, in ascending
    // row order, the G chains side by side. Member rows are fetched eight at a time
    // ahead of the in-order adds, and the next eight list entries while those rows
    // are read.
    if constexpr (kPairs) {
      const uint32_t* Xw = reinterpret_cast<const uint32_t*>(X);  // [Bq][64] bf16 pairs
      for (int c = wave; c < Ci; c += nthr >> 6) {
        const int cnt = ccount[c];
        float mu0, mu1;
        if (cnt > 0) {
          const uint8_t* lc = list + c * Bq;
          float s0 = 0.0f, s1 = 0.0f;
          int m = 0;
          uint2 rr = *reinterpret_cast<const uint2*>(lc);
          for (; m + 8 <= cnt; m += 8) {
            uint32_t v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = Xw[int(((u < 4 ? rr.x : rr.y) >> (8 * (u & 3))) & 0xFFu) * 64 + lane];
            rr = *reinterpret_cast<const uint2*>(lc + min(m + 8, Bq - 8));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              s0 = add_rn(s0, __uint_as_float(v[u] << 16));
              s1 = add_rn(s1, __uint_as_float(v[u] & 0xFFFF0000u));
            }
          }
          for (; m < cnt; ++m) {
            const uint32_t w = Xw[int(lc[m]) * 64 + lane];
            s0 = add_rn(s0, __uint_as_float(w << 16));
            s1 = add_rn(s1, __uint_as_float(w & 0xFFFF0000u));
          }
          mu0 = __fdiv_rn(s0, float(cnt));
          mu1 = __fdiv_rn(s1, float(cnt));
        } else {
          mu0 = -0.5f * m2_t[(2 * lane) * CP + c];  // kept centroid
          mu1 = -0.5f * m2_t[(2 * lane + 1) * CP + c];
        }
        finish_pair(c, mu0, mu1);
      }
    } else
    for (int c = wave; c < Ci; c += nthr >> 6) {
      const int cnt = ccount[c];
      float mu[G];
      if (cnt > 0) {
        const uint8_t* lc = list + c * Bq;
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) s[g] = 0.0f;
        int m = 0;
        uint2 rr = *reinterpret_cast<const uint2*>(lc);
        for (; m + 8 <= cnt; m += 8) {
          float v[G][8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int row = int(((u < 4 ? rr.x : rr.y) >> (8 * (u & 3))) & 0xFFu);
#pragma unroll
            for (int g = 0; g < G; ++g) v[g][u] = xlds(row, 64 * g + lane);
          }
          // next batch's member rows, in flight with this batch's reads (the list
          // region of a cluster holds Bq entries, so m + 8 stays inside it)
          rr = *reinterpret_cast<const uint2*>(lc + min(m + 8, Bq - 8));
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int g = 0; g < G; ++g) s[g] = add_rn(s[g], v[g][u]);
        }
        for (; m < cnt; ++m) {
          const int row = lc[m];
#pragma unroll
          for (int g = 0; g < G; ++g) s[g] = add_rn(s[g], xlds(row, 64 * g + lane));
        }
#pragma unroll
        for (int g = 0; g < G; ++g) mu[g] = __fdiv_rn(s[g], float(cnt));
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) mu[g] = -0.5f * m2_t[(64 * g + lane) * CP + c];  // kept centroid
      }
      finish_cluster(c, mu);
    }
    __syncthreads();
  }

  // ---- outputs ----
  // The bf16 copy is the matrix-core operand of the block estimate: the centroid
  // times c2 = scale * log2(e) (one fp32 product, then one rounding to bf16), so the
  // product with a key is the logit in base-2 units.
  const size_t cbase = size_t(blk) * C;
  const float c2 = P.scale * 1.4426950408889634f;
  for (int p = tid; p < C * D; p += nthr) {
    const int c = p / D, k = p % D;
    const float v = c < Ci ? -0.5f * m2_t[k * CP + c] : 0.0f;  // -0.5 * (-2 mu) is exact
    if (cent) cent[(cbase + c) * D + k] = v;
    if (cent_bf16) cent_bf16[(cbase + c) * D + k] = f32_to_bf16(v * c2);
  }
  if (sizes_out)
    for (int c = tid; c < C; c += nthr) sizes_out[cbase + c] = (c < Ci) ? ccount[c] : 0;
  if (assign_out)
    for (int r = tid; r < n; r += nthr) assign_out[size_t(bh) * P.N + row0 + r] = uint8_t(asg[r]);
}

template <bool BF16, int D>
hipError_t launch(const Dims& P, const void* q, float* cent, uint16_t* cb, int32_t* sz, uint8_t* as,
                  hipStream_t s) {
  const int CP = (P.C + 7) & ~7;
  const size_t lds = size_t(P.Bq) * D * (BF16 ? 2 : 4) + size_t(D + D / 64) * CP * 4 + size_t(P.Bq) * 12 +
                    size_t((P.C + 3) & ~3) * 4 + size_t(P.C) * P.Bq;
  auto kern = kmeans_kernel<BF16, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const int blocks = P.B * P.H * P.nqb;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(2 * P.Bq), lds, s, P, q, cent, cb, sz, as);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kmeans(const Dims& P, const void* q, float* cent, uint16_t* cb, int32_t* sz, uint8_t* as,
                         hipStream_t s) {
  if (P.bf16) return P.d == 64 ? launch<true, 64>(P, q, cent, cb, sz, as, s) : launch<true, 128>(P, q, cent, cb, sz, as, s);
  return P.d == 64 ? launch<false, 64>(P, q, cent, cb, sz, as, s) : launch<false, 128>(P, q, cent, cb, sz, as, s);
}

}  // namespace ab
