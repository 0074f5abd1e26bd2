// IBCS clustering: fixed-iteration k-means of the queries of every query block.
//
// AB-Attention abstract (paperdot search page, query "Xing Ma"), IBCS sentence:
// the queries of each query block are clustered on their own, tokens stay in
// place. The clustering is specified operation by operation in fp32 so that the
// result is reproducible bit for bit on any implementation:
//   * distance(r, c) = left-to-right fp32 sum over k of fl(fl(x_rk - mu_ck)^2),
//     starting at 0, with separate multiply and add (no fused multiply-add);
//   * assignment to the nearest centroid, ties to the lowest cluster index;
//   * centroid = fp32 sum of its members in ascending row order, divided by the
//     member count with one correctly rounded division; an empty cluster keeps
//     its centroid and gets size 0;
//   * initial centroids are the strided queries x[floor(c*n/C')], C' = min(C, n).
//
// One workgroup per (b, h, query block), two threads per query row: each keeps
// its query in VGPRs and scans four of every eight clusters with four
// independent distance chains; the two halves then merge their minima (lower
// index wins ties). Centroids sit in LDS transposed ([k][c]) so one 16-byte
// broadcast read feeds the four chains. The update uses per-cluster member
// lists built with wave ballots, so every (cluster, dim) thread only walks its
// own members, in ascending row order, reading them from the block's copy in LDS.
#include "ab_internal.h"

namespace ab {
namespace {

// Separately rounded fp32 operations. HIP's __fmul_rn and __fadd_rn are plain
// operators defined in its headers, where contraction is allowed, so once
// inlined they can still be fused into an FMA; these helpers carry the
// no-contraction setting of their own bodies instead.
__device__ __forceinline__ float sub_rn(float a, float b) {
#pragma clang fp contract(off)
  return a - b;
}
__device__ __forceinline__ float sqr_acc_rn(float acc, float t) {
#pragma clang fp contract(off)
  const float t2 = t * t;
  return acc + t2;
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

// Two threads per query row: thread t handles row t % Bq and the clusters
// c = c0 + 4*(t / Bq) + u (u < 4) of every group of 8.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void kmeans_kernel(Dims P, const void* __restrict__ qv,
                                                     float* __restrict__ cent,
                                                     uint16_t* __restrict__ cent_bf16,
                                                     int32_t* __restrict__ sizes_out,
                                                     uint8_t* __restrict__ assign_out) {
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
  float* mu_t = reinterpret_cast<float*>(smem + size_t(Bq) * D * sizeof(elem_t));    // [D][CP]
  int* asg = reinterpret_cast<int*>(mu_t + size_t(D) * CP);                          // [Bq]
  float* pbest = reinterpret_cast<float*>(asg + Bq);                                 // [Bq] best of the upper half
  int* pidx = reinterpret_cast<int*>(pbest + Bq);                                    // [Bq]
  int* ccount = pidx + Bq;                                                           // [C], padded to 16 bytes
  uint8_t* list = reinterpret_cast<uint8_t*>(ccount + ((C + 3) & ~3));               // [C][Bq] member rows

  const elem_t* qsrc = reinterpret_cast<const elem_t*>(qv) + (size_t(bh) * P.N + row0) * D;
  {
    constexpr int EPC = 16 / sizeof(elem_t);
    const int chunks = n * D / EPC;
    const uint4* src = reinterpret_cast<const uint4*>(qsrc);
    uint4* dst = reinterpret_cast<uint4*>(X);
    for (int p = tid; p < chunks; p += nthr) dst[p] = src[p];
  }
  for (int p = tid; p < D * CP; p += nthr) mu_t[p] = 0.0f;
  // this thread's query, held in VGPRs for every iteration (16-byte global loads)
  QueryRow<BF16, D> x;
  {
    const uint4* src = reinterpret_cast<const uint4*>(qsrc + size_t(min(r_own, n - 1)) * D);
#pragma unroll
    for (int c4 = 0; c4 < QueryRow<BF16, D>::kWords / 4; ++c4) {
      const uint4 u = src[c4];
      x.w[4 * c4 + 0] = u.x;
      x.w[4 * c4 + 1] = u.y;
      x.w[4 * c4 + 2] = u.z;
      x.w[4 * c4 + 3] = u.w;
    }
  }
  __syncthreads();
  auto xlds = [&](int r, int k) -> float {
    if constexpr (BF16) return bf16_to_f32(X[r * D + k]); else return X[r * D + k];
  };
  for (int p = tid; p < Ci * D; p += nthr) {
    const int c = p / D, k = p % D;
    mu_t[k * CP + c] = xlds((c * n) / Ci, k);
  }
  if (tid < C) ccount[tid] = 0;
  __syncthreads();

  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int it = 0; it < P.T; ++it) {
    // ---- assignment: each half of the threads scans 4 of every 8 clusters ----
    float best = __builtin_inff();
    int bi = 0;
    if (r_own < n) {
      for (int c0 = 0; c0 < Ci; c0 += 8) {
        const int cb = c0 + 4 * chalf;
        float acc[4];
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) acc[cc] = 0.0f;
#pragma unroll
        for (int k = 0; k < D; ++k) {
          const float xk = x.get(k);
          const float4 m4 = *reinterpret_cast<const float4*>(&mu_t[k * CP + cb]);
          const float m[4] = {m4.x, m4.y, m4.z, m4.w};
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            acc[cc] = sqr_acc_rn(acc[cc], sub_rn(xk, m[cc]));
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
    // (c, k) with k fastest: a wave shares c, so the member loop is uniform; member rows
    // are fetched eight at a time ahead of the in-order adds, and the next eight list
    // entries while those rows are read
    for (int p = tid; p < Ci * D; p += nthr) {
      const int c = p / D, k = p % D;
      const int cnt = ccount[c];
      if (cnt > 0) {
        const uint8_t* lc = list + c * Bq;
        float s = 0.0f;
        int m = 0;
        uint2 rr = *reinterpret_cast<const uint2*>(lc);
        for (; m + 8 <= cnt; m += 8) {
          float v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = xlds(int(((u < 4 ? rr.x : rr.y) >> (8 * (u & 3))) & 0xFFu), k);
          // next batch's member rows, in flight with this batch's reads (the list
          // region of a cluster holds Bq entries, so m + 8 stays inside it)
          rr = *reinterpret_cast<const uint2*>(lc + min(m + 8, Bq - 8));
#pragma unroll
          for (int u = 0; u < 8; ++u) s = add_rn(s, v[u]);
        }
        for (; m < cnt; ++m) s = add_rn(s, xlds(lc[m], k));
        mu_t[k * CP + c] = __fdiv_rn(s, float(cnt));
      }
    }
    __syncthreads();
  }

  // ---- outputs ----
  const size_t cbase = size_t(blk) * C;
  for (int p = tid; p < C * D; p += nthr) {
    const int c = p / D, k = p % D;
    const float v = mu_t[k * CP + c];  // zero for clusters c >= Ci
    if (cent) cent[(cbase + c) * D + k] = v;
    if (cent_bf16) cent_bf16[(cbase + c) * D + k] = f32_to_bf16(v);
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
  const size_t lds = size_t(P.Bq) * D * (BF16 ? 2 : 4) + size_t(D) * CP * 4 + size_t(P.Bq) * 12 +
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
