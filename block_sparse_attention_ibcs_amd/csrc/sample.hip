// SIP: sampling with inclusion-probability weighting (AB-Attention abstract,
// SIP sentence), integer-exact given the fp32 scores.
//
// Per row (b, h, i) of the score matrix:
//   w_j = max(1, floor(s_j * 2^24))          (NaN or s <= 0 -> 1, s >= 1 -> 2^24)
//   water-filling: grow a capped set while some uncapped j has (K - m) w_j >= S
//   (m = capped count, S = uncapped weight total); thresholds t_j = 2^24 when
//   capped, else max(1, floor((K - m) w_j 2^24 / S)); inclusion prob = t_j / 2^24
//   u_j = word (j mod 4) of Philox4x32-10(key = seed, counter = (j/4, i, h, b)) >> 8
//   keep iff u_j < t_j; weight = fp32(2^24) / fp32(t_j)
// Philox4x32-10 follows Salmon et al., SC'11.
//
// Rows with at most 4096 key sub-blocks (every workload in use): one wave per
// row, four rows per workgroup, no workgroup barriers. Lane l holds the
// quantized scores of sub-blocks [1024c + 16l, 1024c + 16l + 16) of every 1024-wide
// chunk c in VGPRs; each water-filling pass is a wave reduction; the lane draws
// its own four Philox blocks, computes thresholds with one reciprocal per row
// and an exact integer fix-up, and a wave prefix sum over the lanes' popcounts
// places the kept indices in ascending order.
// Rows of up to 16384 sub-blocks: the same scheme with one 256-thread workgroup per
// row and workgroup reductions. Longer rows: one workgroup per row, the capped set in
// an LDS bitset, scores re-read on every pass.
#include "ab_internal.h"

namespace ab {
namespace {

constexpr uint32_t kOne = 1u << 24;
constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t quantize(float s) {
  if (!(s > 0.0f)) return 1u;        // NaN, zero, negative
  if (s >= 1.0f) return kOne;
  const float v = s * 16777216.0f;   // exact
  const uint32_t q = uint32_t(v);    // truncation == floor for v >= 0
  return q > 0u ? q : 1u;
}

__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                             uint32_t k1) {
  const uint64_t p0 = uint64_t(0xD2511F53u) * c0;
  const uint64_t p1 = uint64_t(0xCD9E8D57u) * c2;
  const uint32_t hi0 = uint32_t(p0 >> 32), lo0 = uint32_t(p0);
  const uint32_t hi1 = uint32_t(p1 >> 32), lo1 = uint32_t(p1);
  const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
  c0 = n0;
  c1 = lo1;
  c2 = n2;
  c3 = lo0;
}

__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    philox_round(c0, c1, c2, c3, k0, k1);
  }
  return make_uint4(c0, c1, c2, c3);
}

template <typename T>
__device__ __forceinline__ T block_sum(T v, T* red) {
  // wave reduction then across the four waves
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  T t = red[0];
  for (int w = 1; w < kThreads / 64; ++w) t += red[w];
  return t;
}

// The water-filling test room * w >= S for every uncapped w of a row, as one bound per
// pass: for an integer w >= 0 it holds iff w >= ceil(S / room) (room > 0), and with
// room = 0 iff S = 0. The fp64 quotient is within one of the integer one; the
// fix-ups make it exact. Bounds past 2^32 - 1 are clamped (every w is below 2^25).
__device__ __forceinline__ uint32_t cap_bound(uint64_t S, uint64_t room) {
  if (room == 0) return S == 0 ? 0u : 0xFFFFFFFFu;
  uint64_t W = uint64_t(double(S) / double(room));
  while (W * room < S) ++W;
  while (W > 0 && (W - 1) * room >= S) --W;
  return W > 0xFFFFFFFFull ? 0xFFFFFFFFu : uint32_t(W);
}

// The threshold floor(room * w * 2^24 / S) of an uncapped w (room * w < S, so it is below
// 2^24). R = room * 2^24 / S in fp64 (both exact, one rounding), and w * R (one more
// rounding) lies within 2^-28 of the quotient, so its integer part is the floor unless
// the fraction lies within 2^-27 of an integer; there an exact integer comparison
// decides between the two candidates (room * w * 2^24 < S * 2^24 <= 65536 * 2^48: rows
// hold at most 65536 sub-blocks, so the product fits 64 bits).
__device__ __forceinline__ uint32_t threshold_floor(uint32_t w, uint64_t room, uint64_t S, double R) {
  const double y = double(w) * R;
  uint32_t t = uint32_t(y);
  const double fr = y - double(t);
  if (fr < 0x1p-27 || fr > 1.0 - 0x1p-27) {
    const uint64_t num = room * uint64_t(w) * uint64_t(kOne);
    if (uint64_t(t + 1) * S <= num) ++t;
    else if (uint64_t(t) * S > num) --t;
  }
  return t;
}

__global__ __launch_bounds__(kThreads) void sample_kernel(Dims P, int K, uint32_t seed_lo, uint32_t seed_hi,
                                                          const float* __restrict__ scores,
                                                          int32_t* __restrict__ idx, float* __restrict__ weights,
                                                          int32_t* __restrict__ counts,
                                                          uint32_t* __restrict__ mask) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int nkb = P.nkb;
  const int words = ceil_div(nkb, 32);
  uint32_t* capped = reinterpret_cast<uint32_t*>(smem);  // [words]
  __shared__ uint64_t red64[4];
  __shared__ int red32[4];
  __shared__ int scan_base;
  __shared__ int wave_tot[4];

  const int row = blockIdx.x;  // (b*H + h)*nqb + i
  const int i = row % P.nqb;
  const int bh = row / P.nqb;
  const int h = bh % P.H, b = bh / P.H;
  const float* s = scores + size_t(row) * nkb;
  const int tid = threadIdx.x;

  const bool all = (K >= nkb);
  for (int w = tid; w < words; w += kThreads) {
    uint32_t v = 0;
    if (all) {
      const int rem = nkb - w * 32;
      v = rem >= 32 ? 0xFFFFFFFFu : ((1u << rem) - 1u);
    }
    capped[w] = v;
  }
  __syncthreads();

  // ---- integer water-filling ----
  uint64_t room = 0, S = 1;
  if (!all) {
    int m = 0;
    for (;;) {
      uint64_t part = 0;
      for (int j = tid; j < nkb; j += kThreads)
        if (!((capped[j >> 5] >> (j & 31)) & 1u)) part += quantize(s[j]);
      S = block_sum<uint64_t>(part, red64);
      room = uint64_t(K - m);
      const uint32_t W = cap_bound(S, room);  // room * w >= S  <=>  w >= W
      __syncthreads();
      int nnew = 0;
      for (int j = tid; j < nkb; j += kThreads) {
        if (!((capped[j >> 5] >> (j & 31)) & 1u)) {
          if (quantize(s[j]) >= W) {
            atomicOr(&capped[j >> 5], 1u << (j & 31));
            ++nnew;
          }
        }
      }
      nnew = block_sum<int>(nnew, red32);
      __syncthreads();
      if (nnew == 0) break;
      m += nnew;
    }
  }

  // ---- draw, compaction, outputs ----
  const double R = double(room * uint64_t(kOne)) / double(S);
  if (tid == 0) scan_base = 0;
  __syncthreads();
  const size_t out0 = size_t(row) * nkb;
  for (int w0 = 0; w0 < words; w0 += kThreads) {
    const int w = w0 + tid;
    uint32_t keep = 0;
    uint32_t tw[32];
    if (w < words) {
      const uint32_t cw = capped[w];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int jg = w * 32 + g * 4;
        if (jg >= nkb) break;
        const uint4 r = philox4x32_10(uint32_t(jg >> 2), uint32_t(i), uint32_t(h), uint32_t(b), seed_lo, seed_hi);
        const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jg + e;
          const int bit = g * 4 + e;
          tw[bit] = kOne;
          if (j < nkb) {
            uint32_t t;
            if ((cw >> bit) & 1u) {
              t = kOne;
            } else {
              const uint32_t q = threshold_floor(quantize(s[j]), room, S, R);
              t = q > 0 ? q : 1u;
            }
            tw[bit] = t;
            if ((rr[e] >> 8) < t) keep |= 1u << bit;
          }
        }
      }
      if (mask) mask[size_t(row) * words + w] = keep;
    }
    // exclusive scan of popcounts across the workgroup (ascending word order)
    const int pc = __popc(keep);
    int incl = pc;
    const int lane = tid & 63, wave = tid >> 6;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int base = scan_base;
    for (int wv = 0; wv < wave; ++wv) base += wave_tot[wv];
    int pos = base + incl - pc;
    if (w < words) {
#pragma unroll
      for (int bit = 0; bit < 32; ++bit) {
        if ((keep >> bit) & 1u) {
          idx[out0 + pos] = w * 32 + bit;
          weights[out0 + pos] = __fdiv_rn(16777216.0f, float(tw[bit]));
          ++pos;
        }
      }
    }
    __syncthreads();
    if (tid == kThreads - 1) scan_base = base + incl;
    __syncthreads();
  }
  if (tid == 0) counts[row] = scan_base;
}



__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

constexpr int kLaneElems = 16;          // sub-blocks per lane per chunk
constexpr int kChunk = 64 * kLaneElems; // sub-blocks per chunk


// Inclusive prefix sum over the wave in lane order.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  const int lane = threadIdx.x & 63;
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  return v;
}

// Systematic draw of one lane's 16 blocks: the row's points U + m * 2^24 (m >= 0)
// against the half-open intervals [C_j, C_j + t_j) of the cumulative thresholds;
// c0 is C of the lane's first block.
__device__ __forceinline__ int64_t points_below(uint64_t x, uint32_t U) {
  return x > U ? int64_t((x - 1 - U) >> 24) + 1 : 0;
}
__device__ __forceinline__ uint32_t systematic_keep16(const uint32_t (&t)[kLaneElems], uint32_t valid, uint64_t c0,
                                                      uint32_t U) {
  uint32_t keep = 0u;
  uint64_t c = c0;
  int64_t below = points_below(c, U);
#pragma unroll
  for (int e = 0; e < kLaneElems; ++e) {
    if ((valid >> e) & 1u) {
      c += t[e];
      const int64_t nb = points_below(c, U);
      if (nb > below) keep |= 1u << e;
      below = nb;
    }
  }
  return keep;
}

template <int NCH, bool SYS>
__global__ __launch_bounds__(256) void sample_wave_kernel(Dims P, int K, int rows, uint32_t seed_lo,
                                                          uint32_t seed_hi, const float* __restrict__ scores,
                                                          int32_t* __restrict__ idx, float* __restrict__ weights,
                                                          int32_t* __restrict__ counts,
                                                          uint32_t* __restrict__ mask) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // the whole wave leaves; nothing below synchronises the workgroup
  const int nkb = P.nkb;
  const int i = row % P.nqb;
  const int bh = row / P.nqb;
  const int h = bh % P.H, b = bh / P.H;
  const float* s = scores + size_t(row) * nkb;
  const bool vec_ok = (nkb & 3) == 0;

  // ---- quantized scores in VGPRs; valid-element masks ----
  uint32_t w[NCH][kLaneElems];
  uint32_t valid[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int j0 = c * kChunk + lane * kLaneElems;
    const int nv = min(kLaneElems, max(0, nkb - j0));
    valid[c] = (1u << nv) - 1u;  // nv <= 16
    if (vec_ok && nv == kLaneElems) {
      const float4* s4 = reinterpret_cast<const float4*>(s + j0);
#pragma unroll
      for (int q = 0; q < kLaneElems / 4; ++q) {
        const float4 v = s4[q];
        w[c][4 * q + 0] = quantize(v.x);
        w[c][4 * q + 1] = quantize(v.y);
        w[c][4 * q + 2] = quantize(v.z);
        w[c][4 * q + 3] = quantize(v.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kLaneElems; ++e) w[c][e] = (e < nv) ? quantize(s[j0 + e]) : 0u;
    }
  }

  // ---- integer water-filling (capped bits per chunk) ----
  uint32_t cap[NCH];
  uint64_t room = 0, S = 1;
  if (K >= nkb) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) cap[c] = valid[c];
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) cap[c] = 0u;
    int m = 0;
    for (;;) {
      uint32_t part = 0;  // at most 64 values below 2^25
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) part += ((cap[c] >> e) & 1u) ? 0u : w[c][e];
      S = wave_sum_u64(uint64_t(part));
      room = uint64_t(K - m);
      const uint32_t W = cap_bound(S, room);  // room * w >= S  <=>  w >= W
      int nnew = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) {
          const bool un = ((valid[c] & ~cap[c]) >> e) & 1u;
          if (un && w[c][e] >= W) {
            cap[c] |= 1u << e;
            ++nnew;
          }
        }
      }
      nnew = wave_sum_i32(nnew);
      if (nnew == 0) break;
      m += nnew;
    }
  }

  // ---- draw: thresholds replace the weights in place ----
  const double R = double(room * uint64_t(kOne)) / double(S);
  uint32_t keep[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int e = 0; e < kLaneElems; ++e) {
      uint32_t t = kOne;
      if (!((cap[c] >> e) & 1u)) {
        const uint32_t q = threshold_floor(w[c][e], room, S, R);
        t = q > 0u ? q : 1u;
      }
      w[c][e] = ((valid[c] >> e) & 1u) ? t : 0u;
    }
  }
  if constexpr (SYS) {
    // one uniform per row; cumulative thresholds in index order (chunk, lane, element)
    const uint32_t U = philox4x32_10(0xFFFFFFFFu, uint32_t(i), uint32_t(h), uint32_t(b), seed_lo, seed_hi).x >> 8;
    uint64_t cbase = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint32_t lsum = 0;
#pragma unroll
      for (int e = 0; e < kLaneElems; ++e) lsum += w[c][e];
      const uint64_t incl = wave_incl_scan_u64(lsum);
      keep[c] = systematic_keep16(w[c], valid[c], cbase + incl - lsum, U);
      cbase += __shfl(incl, 63, 64);
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      keep[c] = 0u;
      const int g0 = (c * kChunk + lane * kLaneElems) >> 2;
#pragma unroll
      for (int g = 0; g < kLaneElems / 4; ++g) {
        if (!((valid[c] >> (4 * g)) & 0xFu)) continue;
        const uint4 r = philox4x32_10(uint32_t(g0 + g), uint32_t(i), uint32_t(h), uint32_t(b), seed_lo, seed_hi);
        const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int e = 4 * g + e4;
          if (((valid[c] >> e) & 1u) && (rr[e4] >> 8) < w[c][e]) keep[c] |= 1u << e;
        }
      }
    }
  }

  // ---- compaction in ascending sub-block order: chunk, then lane, then element ----
  const size_t out0 = size_t(row) * nkb;
  const int words = ceil_div(nkb, 32);
  int base = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int pc = __popc(keep[c]);
    int incl = pc;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    int pos = base + incl - pc;
    const int j0 = c * kChunk + lane * kLaneElems;
#pragma unroll
    for (int e = 0; e < kLaneElems; ++e) {
      if ((keep[c] >> e) & 1u) {
        idx[out0 + pos] = j0 + e;
        weights[out0 + pos] = __fdiv_rn(16777216.0f, float(w[c][e]));
        ++pos;
      }
    }
    base += __shfl(incl, 63, 64);
    if (mask) {
      const uint32_t hi = __shfl_down(keep[c], 1, 64);
      const int wd = (c * kChunk) / 32 + lane / 2;
      if (!(lane & 1) && wd < words) mask[size_t(row) * words + wd] = keep[c] | (hi << 16);
    }
  }
  if (lane == 0) counts[row] = base;
}

// Rows of 4097..16384 sub-blocks: one 256-thread workgroup per row, thread t holds
// the quantized scores of sub-blocks [4096c + 16t, 4096c + 16t + 16) of every
// 4096-wide chunk c in VGPRs; water-filling sums are workgroup reductions and the
// compaction is a workgroup prefix sum per chunk.
constexpr int kBlockChunk = kThreads * kLaneElems;

template <int NCH, bool SYS>
__global__ __launch_bounds__(kThreads) void sample_block_kernel(Dims P, int K, uint32_t seed_lo, uint32_t seed_hi,
                                                                const float* __restrict__ scores,
                                                                int32_t* __restrict__ idx,
                                                                float* __restrict__ weights,
                                                                int32_t* __restrict__ counts,
                                                                uint32_t* __restrict__ mask) {
  __shared__ uint64_t red64[4];
  __shared__ int red32[4];
  __shared__ int wtot[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;  // (b*H + h)*nqb + i
  const int nkb = P.nkb;
  const int i = row % P.nqb;
  const int bh = row / P.nqb;
  const int h = bh % P.H, b = bh / P.H;
  const float* s = scores + size_t(row) * nkb;
  const bool vec_ok = (nkb & 3) == 0;

  uint32_t w[NCH][kLaneElems];
  uint32_t valid[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int j0 = c * kBlockChunk + tid * kLaneElems;
    const int nv = min(kLaneElems, max(0, nkb - j0));
    valid[c] = (1u << nv) - 1u;  // nv <= 16
    if (vec_ok && nv == kLaneElems) {
      const float4* s4 = reinterpret_cast<const float4*>(s + j0);
#pragma unroll
      for (int q = 0; q < kLaneElems / 4; ++q) {
        const float4 v = s4[q];
        w[c][4 * q + 0] = quantize(v.x);
        w[c][4 * q + 1] = quantize(v.y);
        w[c][4 * q + 2] = quantize(v.z);
        w[c][4 * q + 3] = quantize(v.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kLaneElems; ++e) w[c][e] = (e < nv) ? quantize(s[j0 + e]) : 0u;
    }
  }

  // ---- integer water-filling ----
  uint32_t cap[NCH];
  uint64_t room = 0, S = 1;
  if (K >= nkb) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) cap[c] = valid[c];
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) cap[c] = 0u;
    int m = 0;
    for (;;) {
      uint32_t part = 0;  // at most 64 values below 2^25
#pragma unroll
      for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) part += ((cap[c] >> e) & 1u) ? 0u : w[c][e];
      S = block_sum<uint64_t>(uint64_t(part), red64);
      room = uint64_t(K - m);
      const uint32_t W = cap_bound(S, room);  // room * w >= S  <=>  w >= W
      int nnew = 0;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int e = 0; e < kLaneElems; ++e) {
          const bool un = ((valid[c] & ~cap[c]) >> e) & 1u;
          if (un && w[c][e] >= W) {
            cap[c] |= 1u << e;
            ++nnew;
          }
        }
      }
      nnew = block_sum<int>(nnew, red32);
      if (nnew == 0) break;
      m += nnew;
    }
  }

  // ---- draw: thresholds replace the weights in place ----
  const double R = double(room * uint64_t(kOne)) / double(S);
  uint32_t keep[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
#pragma unroll
    for (int e = 0; e < kLaneElems; ++e) {
      uint32_t t = kOne;
      if (!((cap[c] >> e) & 1u)) {
        const uint32_t q = threshold_floor(w[c][e], room, S, R);
        t = q > 0u ? q : 1u;
      }
      w[c][e] = ((valid[c] >> e) & 1u) ? t : 0u;
    }
  }
  if constexpr (SYS) {
    __shared__ uint64_t wtot64[4];
    const uint32_t U = philox4x32_10(0xFFFFFFFFu, uint32_t(i), uint32_t(h), uint32_t(b), seed_lo, seed_hi).x >> 8;
    uint64_t cbase = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint32_t lsum = 0;
#pragma unroll
      for (int e = 0; e < kLaneElems; ++e) lsum += w[c][e];
      const uint64_t incl = wave_incl_scan_u64(lsum);
      __syncthreads();  // wtot64 of the previous chunk is consumed
      if (lane == 63) wtot64[wave] = incl;
      __syncthreads();
      uint64_t woff = 0, tot = 0;
#pragma unroll
      for (int wv = 0; wv < kThreads / 64; ++wv) {
        woff += wv < wave ? wtot64[wv] : 0;
        tot += wtot64[wv];
      }
      keep[c] = systematic_keep16(w[c], valid[c], cbase + woff + incl - lsum, U);
      cbase += tot;
    }
  } else {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      keep[c] = 0u;
      const int g0 = (c * kBlockChunk + tid * kLaneElems) >> 2;
#pragma unroll
      for (int g = 0; g < kLaneElems / 4; ++g) {
        if (!((valid[c] >> (4 * g)) & 0xFu)) continue;
        const uint4 r = philox4x32_10(uint32_t(g0 + g), uint32_t(i), uint32_t(h), uint32_t(b), seed_lo, seed_hi);
        const uint32_t rr[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int e = 4 * g + e4;
          if (((valid[c] >> e) & 1u) && (rr[e4] >> 8) < w[c][e]) keep[c] |= 1u << e;
        }
      }
    }
  }

  // ---- compaction in ascending sub-block order: chunk, then thread, then element ----
  const size_t out0 = size_t(row) * nkb;
  const int words = ceil_div(nkb, 32);
  int base = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int pc = __popc(keep[c]);
    int incl = pc;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    __syncthreads();  // wtot of the previous chunk is consumed
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    int woff = 0, tot = 0;
#pragma unroll
    for (int wv = 0; wv < kThreads / 64; ++wv) {
      woff += wv < wave ? wtot[wv] : 0;
      tot += wtot[wv];
    }
    int pos = base + woff + incl - pc;
    const int j0 = c * kBlockChunk + tid * kLaneElems;
#pragma unroll
    for (int e = 0; e < kLaneElems; ++e) {
      if ((keep[c] >> e) & 1u) {
        idx[out0 + pos] = j0 + e;
        weights[out0 + pos] = __fdiv_rn(16777216.0f, float(w[c][e]));
        ++pos;
      }
    }
    base += tot;
    if (mask) {
      const uint32_t hi = __shfl_down(keep[c], 1, 64);
      const int wd = (c * kBlockChunk) / 32 + tid / 2;
      if (!(tid & 1) && wd < words) mask[size_t(row) * words + wd] = keep[c] | (hi << 16);
    }
  }
  if (tid == 0) counts[row] = base;
}

// Exclusive prefix sum of v over the workgroup in thread order; total receives the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* wtot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  __syncthreads();  // wtot of a previous scan is consumed
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int woff = 0;
  total = 0;
#pragma unroll
  for (int wv = 0; wv < kThreads / 64; ++wv) {
    woff += wv < wave ? wtot[wv] : 0;
    total += wtot[wv];
  }
  return woff + incl - v;
}

// Top-K truncation: one 256-thread workgroup per row, the quantized scores in VGPRs
// as in sample_block_kernel. The cut value theta is the largest w with at least K
// blocks at or above it (binary search over [1, 2^24], one workgroup count per
// step); blocks above theta are kept, and of those equal to theta the lowest
// K - #(w > theta) indices, found with a workgroup prefix count in index order.
template <int NCH>
__global__ __launch_bounds__(kThreads) void topk_block_kernel(Dims P, int K, const float* __restrict__ scores,
                                                              int32_t* __restrict__ idx,
                                                              float* __restrict__ weights,
                                                              int32_t* __restrict__ counts,
                                                              uint32_t* __restrict__ mask) {
  __shared__ int red32[4];
  __shared__ int wtot[4];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int nkb = P.nkb;
  const float* s = scores + size_t(row) * nkb;
  const bool vec_ok = (nkb & 3) == 0;

  uint32_t w[NCH][kLaneElems];
  uint32_t valid[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int j0 = c * kBlockChunk + tid * kLaneElems;
    const int nv = min(kLaneElems, max(0, nkb - j0));
    valid[c] = (1u << nv) - 1u;  // nv <= 16
    if (vec_ok && nv == kLaneElems) {
      const float4* s4 = reinterpret_cast<const float4*>(s + j0);
#pragma unroll
      for (int q = 0; q < kLaneElems / 4; ++q) {
        const float4 v = s4[q];
        w[c][4 * q + 0] = quantize(v.x);
        w[c][4 * q + 1] = quantize(v.y);
        w[c][4 * q + 2] = quantize(v.z);
        w[c][4 * q + 3] = quantize(v.w);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kLaneElems; ++e) w[c][e] = (e < nv) ? quantize(s[j0 + e]) : 0u;
    }
  }
  auto count_ge = [&](uint32_t th) {
    int n = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int e = 0; e < kLaneElems; ++e) n += (((valid[c] >> e) & 1u) && w[c][e] >= th) ? 1 : 0;
    return block_sum<int>(n, red32);
  };

  uint32_t keep[NCH];
  if (K >= nkb) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) keep[c] = valid[c];
  } else {
    uint32_t lo = 1u, hi = kOne + 1u;  // count_ge(lo) = nkb >= K, count_ge(hi) = 0 < K
    while (hi - lo > 1u) {
      const uint32_t mid = lo + (hi - lo) / 2u;
      if (count_ge(mid) >= K) lo = mid; else hi = mid;
    }
    const uint32_t theta = lo;
    const int need = K - count_ge(theta + 1u);  // blocks equal to theta to keep, lowest index first
    int tie_base = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint32_t above = 0u, tie = 0u;
#pragma unroll
      for (int e = 0; e < kLaneElems; ++e) {
        if ((valid[c] >> e) & 1u) {
          above |= (w[c][e] > theta ? 1u : 0u) << e;
          tie |= (w[c][e] == theta ? 1u : 0u) << e;
        }
      }
      int tot = 0;
      int rank = tie_base + block_excl_scan(__popc(tie), wtot, tot);
      uint32_t kt = 0u;
#pragma unroll
      for (int e = 0; e < kLaneElems; ++e) {
        if ((tie >> e) & 1u) {
          if (rank < need) kt |= 1u << e;
          ++rank;
        }
      }
      keep[c] = above | kt;
      tie_base += tot;
    }
  }

  // ---- compaction in ascending sub-block order, weight 1 ----
  const size_t out0 = size_t(row) * nkb;
  const int words = ceil_div(nkb, 32);
  int base = 0;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    int tot = 0;
    int pos = base + block_excl_scan(__popc(keep[c]), wtot, tot);
    const int j0 = c * kBlockChunk + tid * kLaneElems;
#pragma unroll
    for (int e = 0; e < kLaneElems; ++e) {
      if ((keep[c] >> e) & 1u) {
        idx[out0 + pos] = j0 + e;
        weights[out0 + pos] = 1.0f;
        ++pos;
      }
    }
    base += tot;
    if (mask) {
      const uint32_t hi16 = __shfl_down(keep[c], 1, 64);
      const int wd = (c * kBlockChunk) / 32 + tid / 2;
      if (!(tid & 1) && wd < words) mask[size_t(row) * words + wd] = keep[c] | (hi16 << 16);
    }
  }
  if (tid == 0) counts[row] = base;
}

}  // namespace

template <bool SYS>
hipError_t launch_sample_mode(const Dims& P, const float* scores, int K, uint64_t seed, int32_t* idx, float* weights,
                              int32_t* counts, uint32_t* mask, hipStream_t s) {
  const int rows = P.B * P.H * P.nqb;
  const uint32_t lo = uint32_t(seed), hi = uint32_t(seed >> 32);
  const dim3 grid(ceil_div(rows, 4)), block(256);
  switch (ceil_div(P.nkb, kChunk)) {
    case 1: hipLaunchKernelGGL((sample_wave_kernel<1, SYS>), grid, block, 0, s, P, K, rows, lo, hi, scores, idx, weights, counts, mask); break;
    case 2: hipLaunchKernelGGL((sample_wave_kernel<2, SYS>), grid, block, 0, s, P, K, rows, lo, hi, scores, idx, weights, counts, mask); break;
    case 3: hipLaunchKernelGGL((sample_wave_kernel<3, SYS>), grid, block, 0, s, P, K, rows, lo, hi, scores, idx, weights, counts, mask); break;
    case 4: hipLaunchKernelGGL((sample_wave_kernel<4, SYS>), grid, block, 0, s, P, K, rows, lo, hi, scores, idx, weights, counts, mask); break;
    default: {
      const dim3 g(rows), t(kThreads);
      switch (ceil_div(P.nkb, kBlockChunk)) {
        case 2: hipLaunchKernelGGL((sample_block_kernel<2, SYS>), g, t, 0, s, P, K, lo, hi, scores, idx, weights, counts, mask); break;
        case 3: hipLaunchKernelGGL((sample_block_kernel<3, SYS>), g, t, 0, s, P, K, lo, hi, scores, idx, weights, counts, mask); break;
        case 4: hipLaunchKernelGGL((sample_block_kernel<4, SYS>), g, t, 0, s, P, K, lo, hi, scores, idx, weights, counts, mask); break;
        default: {
          if (SYS) return hipErrorInvalidValue;  // rejected on the host before this point
          const size_t lds = size_t(ceil_div(P.nkb, 32)) * 4;
          hipLaunchKernelGGL(sample_kernel, g, t, lds, s, P, K, lo, hi, scores, idx, weights, counts, mask);
        }
      }
    }
  }
  return hipGetLastError();
}

hipError_t launch_sample(const Dims& P, const float* scores, int K, uint64_t seed, int32_t* idx, float* weights,
                         int32_t* counts, uint32_t* mask, hipStream_t s, bool systematic) {
  return systematic ? launch_sample_mode<true>(P, scores, K, seed, idx, weights, counts, mask, s)
                    : launch_sample_mode<false>(P, scores, K, seed, idx, weights, counts, mask, s);
}

hipError_t launch_topk(const Dims& P, const float* scores, int K, int32_t* idx, float* weights, int32_t* counts,
                       uint32_t* mask, hipStream_t s) {
  const dim3 g(P.B * P.H * P.nqb), t(kThreads);
  switch (ceil_div(P.nkb, kBlockChunk)) {
    case 1: hipLaunchKernelGGL(topk_block_kernel<1>, g, t, 0, s, P, K, scores, idx, weights, counts, mask); break;
    case 2: hipLaunchKernelGGL(topk_block_kernel<2>, g, t, 0, s, P, K, scores, idx, weights, counts, mask); break;
    case 3: hipLaunchKernelGGL(topk_block_kernel<3>, g, t, 0, s, P, K, scores, idx, weights, counts, mask); break;
    default: hipLaunchKernelGGL(topk_block_kernel<4>, g, t, 0, s, P, K, scores, idx, weights, counts, mask);
  }
  return hipGetLastError();
}

}  // namespace ab
