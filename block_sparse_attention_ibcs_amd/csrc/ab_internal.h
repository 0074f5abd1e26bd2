// Internal declarations shared by the HIP sources of libabattn (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ab_attn.h"

namespace ab {

// Element type tags.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even fp32 -> bf16 (inputs are finite in every use here).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }

// MI355X deals consecutive workgroup ids round-robin to its 8 XCDs, each with
// its own L2. This bijection on [0, n) gives every XCD one contiguous range of
// logical ids, so neighbouring work items (which read overlapping data) share
// an L2.
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_remap(int pid, int n) {
  const int xcd = pid % kXcds, local = pid / kXcds;
  const int per = (n + kXcds - 1) / kXcds;
  const int tall = n % kXcds;  // XCDs that receive `per` ids; the rest receive per - 1
  if (tall == 0 || xcd < tall) return xcd * per + local;
  return tall * per + (xcd - tall) * (per - 1) + local;
}

// Capacity of the Infinity Cache (MALL) that the XCDs share.
constexpr size_t kMallBytes = size_t(256) << 20;

// Head-major variant for ids (b*H + h)*nqb + i over nbh = B*H heads: all XCDs work
// on the same head at the same time, XCD x on its own contiguous slice of that
// head's query blocks, then all move on to the next head. The keys and values in
// use at any moment are then one or two heads' instead of about one head per XCD,
// which matters once eight heads' K and V no longer fit the Infinity Cache. Each
// head gives every XCD q = nqb / 8 blocks; its r = nqb % 8 extra blocks are dealt
// round-robin over the XCDs, continuing from head to head, so XCD x receives
// exactly as many ids as under xcd_remap (the first n % 8 XCDs one more) and the
// map is a bijection on [0, nbh * nqb).
__host__ __device__ inline int xcd_head_remap(int pid, int nbh, int nqb) {
  const int x = pid % kXcds, j = pid / kXcds;  // XCD and position in its sequence
  const int q = nqb / kXcds, r = nqb % kXcds;
  // first position of head h in XCD x's sequence: h*q plus the extra blocks dealt
  // to x by heads 0..h-1 (the integers below h*r congruent to x mod 8)
  auto start = [&](int h) {
    const long long e = (long long)h * r;
    return h * q + (e > x ? int((e - x + kXcds - 1) / kXcds) : 0);
  };
  int h = int(((long long)j * kXcds) / ((long long)q * kXcds + r));
  if (h > nbh - 1) h = nbh - 1;
  while (h > 0 && start(h) > j) --h;
  while (h + 1 < nbh && start(h + 1) <= j) ++h;
  // head h deals its extras to the XCDs a, a+1, ..., a+r-1 (mod 8), a = h*r mod 8;
  // XCD x's slice starts after x*q blocks and the extras of the XCDs below x
  const int a = int(((long long)h * r) % kXcds);
  int below;
  if (a + r <= kXcds) below = min(max(x - a, 0), r);
  else below = min(max(x - a, 0), kXcds - a) + min(x, a + r - kXcds);
  return h * nqb + x * q + below + (j - start(h));
}

// Derived sizes of one problem.
struct Dims {
  int B, H, N, d, Bq, Bk, C, T;
  int nqb, nkb, mrows;  // query blocks, key sub-blocks, centroid rows per head (nqb*C)
  float scale;
  bool bf16;
};

// Workspace carve-up of ab_score (byte offsets, 256-byte aligned).
struct ScoreWs {
  size_t centroids_f32;  // fp32 [B,H,nqb,C,d]
  size_t centroids_bf16; // bf16 [B,H,nqb,C,d]
  size_t sizes;          // int32 [B,H,nqb,C]
  size_t ell;            // fp32 [B,H,nqb,nkb,C]: base-2 log-sum-exp of each (block, sub-block, cluster)
  size_t lpart;          // fp32 [B,H,nqb*C,splits]: base-2 log-sum-exp of each row over one key split
  size_t total;
  int splits;            // key splits of the scorer GEMM
  int split_keys;        // keys per split (multiple of 128)
};

ScoreWs score_ws_layout(const Dims& D, int num_cus);
// the same carve-up with a given key split length (a multiple of 128)
ScoreWs score_ws_layout_split(const Dims& D, int split_keys);

// Launchers: return hipSuccess or the launch error.
hipError_t launch_kmeans(const Dims& D, const void* q, float* centroids, uint16_t* centroids_bf16,
                         int32_t* sizes, uint8_t* assign, hipStream_t s);
hipError_t launch_score_lse(const Dims& D, const ScoreWs& L, const void* k, const void* cent_any,
                            float* ell, float* lpart, hipStream_t s);
hipError_t launch_score_assemble(const Dims& D, const ScoreWs& L, const float* ell, const float* lpart,
                                 const int32_t* sizes, float* scores, hipStream_t s);
// systematic: fixed-size systematic draw instead of independent trials (rows of at
// most kTopkMaxNkb sub-blocks)
hipError_t launch_sample(const Dims& D, const float* scores, int K, uint64_t seed, int32_t* idx,
                         float* weights, int32_t* counts, uint32_t* mask, hipStream_t s, bool systematic);
constexpr int kTopkMaxNkb = 16384;  // longest row the top-K and systematic kernels take
hipError_t launch_topk(const Dims& D, const float* scores, int K, int32_t* idx, float* weights, int32_t* counts,
                       uint32_t* mask, hipStream_t s);
// order: NULL, or the rows in the order the workgroups take them (rows outside the grid skipped)
hipError_t launch_attn_fwd(const Dims& D, const void* q, const void* k, const void* v, const int32_t* idx,
                           const float* weights, const int32_t* counts, void* out, float* lse,
                           const int32_t* order, hipStream_t s);

// INTRA relay patterns: kept-sub-block lists of one layer (AB_INTRA_SCATTER or AB_INTRA_GATHER)
hipError_t launch_intra_lists(const Dims& D, int layer, int partition_tokens, int32_t* idx, float* weights,
                              int32_t* counts, int32_t* row_order, hipStream_t s);
int intra_default_partition(const Dims& D);  // q_block * ceil(sqrt(NQB))

// FP8 variant: operand preparation (workspace: fp8_ws_bytes)
size_t fp8_ws_bytes(const Dims& D);
hipError_t launch_fp8_prepare(const Dims& D, const void* q, const void* k, const void* v, uint8_t* qcode,
                              float* qscale, uint8_t* kcode, float* kscale, uint8_t* vcode, uint16_t* vmean,
                              float* vscale, uint32_t* vmean_scaled, void* ws, hipStream_t s);
// FP8 variant: attention (head dim 128, query block 128)
hipError_t launch_attn_fwd_fp8(const Dims& D, const uint8_t* qcode, const float* qscale, const uint8_t* kcode,
                               const float* kscale, const uint8_t* vcode, const float* vscale,
                               const uint32_t* vmean_scaled, const int32_t* idx, const float* weights,
                               const int32_t* counts, void* out, float* lse, hipStream_t s);

}  // namespace ab
