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
// One workgroup per (b, h, query block), one thread per query row. Each thread
// keeps its query in VGPRs and runs eight independent distance chains at once;
// centroids sit in LDS transposed ([k][c]) so one 16-byte broadcast read feeds
// four chains. The update uses per-cluster member lists built with wave
// ballots, so every (cluster, dim) thread only walks its own members, in
// ascending row order, with no divergence inside a wave.
#include "ab_internal.h"

namespace ab {
namespace {

#pragma clang fp contract(off)

template <bool BF16, int D>
__global__ __launch_bounds__(128) void kmeans_kernel(Dims P, const void* __restrict__ qv,
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
  const int nthr = blockDim.x;

  // LDS carve-up
  using elem_t = typename std::conditional<BF16, uint16_t, float>::type;
  elem_t* X = reinterpret_cast<elem_t*>(smem);                             // [Bq][D]
  float* mu_t = reinterpret_cast<float*>(smem + size_t(Bq) * D * sizeof(elem_t));  // [D][CP]
  int* asg = reinterpret_cast<int*>(mu_t + size_t(D) * CP);                 // [Bq]
  int* list = asg + Bq;                                                     // [Bq]
  int* cstart = list + Bq;                                                  // [C]
  int* ccount = cstart + C;                                                 // [C]

  const elem_t* qsrc = reinterpret_cast<const elem_t*>(qv) + (size_t(bh) * P.N + row0) * D;
  // stage the query block (16-byte chunks)
  {
    constexpr int EPC = 16 / sizeof(elem_t);
    const int chunks = n * D / EPC;
    const uint4* src = reinterpret_cast<const uint4*>(qsrc);
    uint4* dst = reinterpret_cast<uint4*>(X);
    for (int p = tid; p < chunks; p += nthr) dst[p] = src[p];
  }
  for (int p = tid; p < D * CP; p += nthr) mu_t[p] = 0.0f;
  __syncthreads();
  for (int p = tid; p < Ci * D; p += nthr) {
    const int c = p / D, k = p % D;
    const int r = (c * n) / Ci;
    float x;
    if constexpr (BF16) x = bf16_to_f32(X[r * D + k]); else x = X[r * D + k];
    mu_t[k * CP + c] = x;
  }
  if (tid < C) ccount[tid] = 0;
  __syncthreads();

  const int lane = tid & 63;
  const int wave = tid >> 6;
  // this thread's query, held in VGPRs for every iteration (16-byte global loads)
  float x[D];
  {
    constexpr int EPC = 16 / sizeof(elem_t);
    const uint4* src = reinterpret_cast<const uint4*>(qsrc + size_t(min(tid, n - 1)) * D);
#pragma unroll
    for (int c = 0; c < D / EPC; ++c) {
      const uint4 u = src[c];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (BF16) x[c * EPC + e] = bf16_to_f32(uint16_t(w[e >> 1] >> ((e & 1) * 16)));
        else x[c * EPC + e] = __uint_as_float(w[e]);
      }
    }
  }
  for (int it = 0; it < P.T; ++it) {
    // ---- assignment ----
    if (tid < n) {
      float best = __builtin_inff();
      int bi = 0;
      for (int c0 = 0; c0 < Ci; c0 += 8) {
        float acc[8];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) acc[cc] = 0.0f;
#pragma unroll
        for (int k = 0; k < D; ++k) {
          const float4 m0 = *reinterpret_cast<const float4*>(&mu_t[k * CP + c0]);
          const float4 m1 = *reinterpret_cast<const float4*>(&mu_t[k * CP + c0 + 4]);
          const float m[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
          for (int cc = 0; cc < 8; ++cc) {
            const float df = __fsub_rn(x[k], m[cc]);
            acc[cc] = __fadd_rn(acc[cc], __fmul_rn(df, df));
          }
        }
        const int lim = min(8, Ci - c0);
        for (int cc = 0; cc < lim; ++cc) {
          if (acc[cc] < best) {
            best = acc[cc];
            bi = c0 + cc;
          }
        }
      }
      asg[tid] = bi;
    }
    __syncthreads();
    // ---- member lists (ascending rows per cluster), one wave ----
    if (wave == 0) {
      int base = 0;
      for (int c = 0; c < Ci; ++c) {
        const int st = base;
        for (int r0 = 0; r0 < n; r0 += 64) {
          const int r = r0 + lane;
          const bool pred = (r < n) && (asg[r] == c);
          const uint64_t m = __ballot(pred);
          if (pred) list[base + __popcll(m & ((uint64_t(1) << lane) - 1))] = r;
          base += __popcll(m);
        }
        if (lane == 0) {
          cstart[c] = st;
          ccount[c] = base - st;
        }
      }
    }
    __syncthreads();
    // ---- update ----
    for (int p = tid; p < Ci * D; p += nthr) {
      const int c = p / D, k = p % D;
      const int cnt = ccount[c];
      if (cnt > 0) {
        const int st = cstart[c];
        float s = 0.0f;
        for (int m = 0; m < cnt; ++m) {
          const int r = list[st + m];
          float x;
          if constexpr (BF16) x = bf16_to_f32(X[r * D + k]); else x = X[r * D + k];
          s = __fadd_rn(s, x);
        }
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
  const size_t lds = size_t(P.Bq) * D * (BF16 ? 2 : 4) + size_t(D) * CP * 4 + size_t(P.Bq) * 8 + size_t(P.C) * 8;
  auto kern = kmeans_kernel<BF16, D>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const int blocks = P.B * P.H * P.nqb;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(P.Bq), lds, s, P, q, cent, cb, sz, as);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kmeans(const Dims& P, const void* q, float* cent, uint16_t* cb, int32_t* sz, uint8_t* as,
                         hipStream_t s) {
  if (P.bf16) return P.d == 64 ? launch<true, 64>(P, q, cent, cb, sz, as, s) : launch<true, 128>(P, q, cent, cb, sz, as, s);
  return P.d == 64 ? launch<false, 64>(P, q, cent, cb, sz, as, s) : launch<false, 128>(P, q, cent, cb, sz, as, s);
}

}  // namespace ab
