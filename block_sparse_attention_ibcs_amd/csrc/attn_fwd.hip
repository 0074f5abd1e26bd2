// Weighted block-sparse attention forward with sub-tile key gathering.
//
// AB-Attention abstract (paperdot search page, query "Xing Ma"): exact attention
// on the kept key/value blocks only (problem sentence); each kept block j is
// weighted by the inverse of its inclusion probability w_j in both the softmax
// numerator and denominator, so one pass estimates dense attention (SIP
// sentence); key/value sub-blocks much smaller than a matrix-core tile are
// gathered into full tiles (kernel sentence). The INTRA abstract (paperdot
// search page, query "Wenbo Lu") describes the same idea for static patterns:
// a FlashAttention-style kernel that loads non-contiguous tokens and packs them
// densely.
//
// bf16 design (gfx950, wave64): one workgroup per (b, h, query block); each
// wave owns 32 query rows. A tile is 64 key slots: the compacted list of kept
// sub-blocks is laid end to end, so a 64-slot tile holds 64/Bk sub-blocks for
// Bk <= 64 and half of one for Bk = 128; the gather is one coalesced run per
// sub-block row into LDS. The logits are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so every lane owns one query row
// and 16 keys: the row max and row sum need one exchange between the two wave
// halves, and the probabilities are already in the B-operand layout of
// O^T += V^T P^T. The weight enters as log2(w_j) added to the logits of block
// j's keys, which multiplies numerator and denominator alike while keeping
// every probability in [0, 1]. V is stored transposed in LDS so each lane's A
// operand is two 8-byte reads.
#include "ab_internal.h"
#include "mfma.h"

namespace ab {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSlots = 64;

template <int D>
struct AttnCfg {
  static constexpr int kKPitch = D * 2 + 16;      // bytes per key row of the K tile
  static constexpr int kVPitch = kSlots * 2 + 8;  // bytes per dim row of the transposed V tile
  static constexpr int kKBytes = kSlots * kKPitch;
  static constexpr int kVBytes = D * kVPitch;
  static constexpr int kChunks = D / 8;           // 16-byte chunks per key row
};

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2) void attn_fwd_bf16(Dims P, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ weights,
                                                         const int32_t* __restrict__ counts,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse) {
  using Cfg = AttnCfg<D>;
  constexpr int NT = BQ * 2;
  __shared__ __align__(16) unsigned char Ks[Cfg::kKBytes];
  __shared__ __align__(16) unsigned char Vt[Cfg::kVBytes];
  __shared__ int slot_key[kSlots];
  __shared__ float slot_lw[kSlots];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int blk = blockIdx.x;  // (b*H + h)*nqb + i
  const int i = blk % P.nqb, bh = blk / P.nqb;
  const int N = P.N, Bk = P.Bk;
  const int row0 = i * BQ;
  const int n = min(BQ, N - row0);
  const int cnt = counts[blk];
  const int32_t* list = idx + size_t(blk) * P.nkb;
  const float* wl = weights + size_t(blk) * P.nkb;
  const uint16_t* kh = k + size_t(bh) * N * D;
  const uint16_t* vh = v + size_t(bh) * N * D;

  // Q^T as the B operand: lane -> query row (wave*32 + col), 8 dims per k step
  const int qr = wave * 32 + col;
  bf16x8_t qf[D / 16];
  {
    const uint16_t* src = q + (size_t(bh) * N + row0 + qr) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (qr < n) u = *reinterpret_cast<const uint4*>(src + kk * 16);
      qf[kk] = as_bf16x8(u);
    }
  }
  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  float m = -__builtin_inff(), l = 0.0f;
  const float c2 = P.scale * kLog2e;

  const int ntiles = ceil_div(cnt * Bk, kSlots);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // previous tile fully consumed
    if (tid < kSlots) {
      const int gs = t * kSlots + tid;
      const int ord = gs / Bk, e = gs - ord * Bk;
      int key = -1;
      float lw = -__builtin_inff();
      if (ord < cnt) {
        const int kk = list[ord] * Bk + e;
        if (kk < N) {
          key = kk;
          lw = __builtin_amdgcn_logf(wl[ord]);
        }
      }
      slot_key[tid] = key;
      slot_lw[tid] = lw;
    }
    __syncthreads();
    // gather K rows (coalesced 16-byte chunks of each key row)
    for (int p = tid; p < kSlots * Cfg::kChunks; p += NT) {
      const int s = p / Cfg::kChunks, ch = p - s * Cfg::kChunks;
      const int key = slot_key[s];
      uint4 u = make_uint4(0, 0, 0, 0);
      if (key >= 0) u = *reinterpret_cast<const uint4*>(kh + size_t(key) * D + ch * 8);
      *reinterpret_cast<uint4*>(Ks + s * Cfg::kKPitch + ch * 16) = u;
    }
    // gather V rows in slot pairs and store them transposed: Vt[dim][slot]
    for (int p = tid; p < (kSlots / 2) * Cfg::kChunks; p += NT) {
      const int pr = p / Cfg::kChunks, ch = p - pr * Cfg::kChunks;
      const int k0 = slot_key[2 * pr], k1 = slot_key[2 * pr + 1];
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (k0 >= 0) a = *reinterpret_cast<const uint4*>(vh + size_t(k0) * D + ch * 8);
      if (k1 >= 0) b = *reinterpret_cast<const uint4*>(vh + size_t(k1) * D + ch * 8);
      const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = (aw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
        const uint32_t hi = (bw[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
        *reinterpret_cast<uint32_t*>(Vt + (ch * 8 + e) * Cfg::kVPitch + pr * 4) = lo | (hi << 16);
      }
    }
    __syncthreads();

#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      if (t * kSlots + hb * 32 >= cnt * Bk) break;
      f32x16_t acc = {};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 a = *reinterpret_cast<const uint4*>(Ks + (hb * 32 + col) * Cfg::kKPitch + (kk * 16 + half * 8) * 2);
        acc = mfma32x32x16(as_bf16x8(a), qf[kk], acc);
      }
      float x[16];
      float mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int s = hb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
        x[e] = __builtin_fmaf(acc[e], c2, slot_lw[s]);
        mx = fmaxf(mx, x[e]);
      }
      mx = fmaxf(mx, swap_halves(mx));
      // a window of only padding slots after real keys leaves mn = m (finite)
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      float ps = 0.0f;
      float p[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = fast_exp2(x[e] - mn);
        ps += p[e];
      }
      ps += swap_halves(ps);
      l = l * alpha + ps;
      m = mn;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = __bf16(p[8 * g + e]);
        const int s0 = hb * 32 + 16 * g + half * 4;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const unsigned char* vr = Vt + (db * 32 + col) * Cfg::kVPitch;
          const uint2 lo = *reinterpret_cast<const uint2*>(vr + s0 * 2);
          const uint2 hi = *reinterpret_cast<const uint2*>(vr + (s0 + 8) * 2);
          const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
          o[db] = mfma32x32x16(as_bf16x8(av), pb, o[db]);
        }
      }
    }
  }

  // epilogue: O^T lane layout -> row qr, dims db*32 + (e/4)*8 + half*4 + e%4
  if (qr < n) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* dst = out + (size_t(bh) * N + row0 + qr) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + half * 4;
        uint2 w;
        w.x = uint32_t(f32_to_bf16(o[db][4 * g + 0] * inv)) | (uint32_t(f32_to_bf16(o[db][4 * g + 1] * inv)) << 16);
        w.y = uint32_t(f32_to_bf16(o[db][4 * g + 2] * inv)) | (uint32_t(f32_to_bf16(o[db][4 * g + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(dst + d0) = w;
      }
    }
    if (lse && half == 0) lse[size_t(bh) * N + row0 + qr] = l > 0.0f ? (m + fast_log2(l)) * kLn2 : -__builtin_inff();
  }
}

// fp32 inputs: one thread per query row, VALU dot products against LDS tiles.
template <int D>
__global__ __launch_bounds__(128) void attn_fwd_f32(Dims P, const float* __restrict__ q, const float* __restrict__ k,
                                                    const float* __restrict__ v, const int32_t* __restrict__ idx,
                                                    const float* __restrict__ weights,
                                                    const int32_t* __restrict__ counts, float* __restrict__ out,
                                                    float* __restrict__ lse) {
  constexpr int TS = 32;
  __shared__ float Kt[TS][D];
  __shared__ float Vv[TS][D];
  __shared__ int skey[TS];
  __shared__ float slw[TS];
  const int blk = blockIdx.x;
  const int i = blk % P.nqb, bh = blk / P.nqb;
  const int N = P.N, Bk = P.Bk, Bq = P.Bq;
  const int row0 = i * Bq;
  const int n = min(Bq, N - row0);
  const int cnt = counts[blk];
  const int32_t* list = idx + size_t(blk) * P.nkb;
  const float* wl = weights + size_t(blk) * P.nkb;
  const int r = threadIdx.x;
  float qv[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = (r < n) ? q[(size_t(bh) * N + row0 + r) * D + d] : 0.0f;
    o[d] = 0.0f;
  }
  float m = -__builtin_inff(), l = 0.0f;
  const float c2 = P.scale * kLog2e;
  const int total = cnt * Bk;
  for (int t0 = 0; t0 < total; t0 += TS) {
    __syncthreads();
    if (threadIdx.x < TS) {
      const int gs = t0 + threadIdx.x;
      const int ord = gs / Bk, e = gs - ord * Bk;
      int key = -1;
      float lw = -__builtin_inff();
      if (ord < cnt) {
        const int kk = list[ord] * Bk + e;
        if (kk < N) {
          key = kk;
          lw = __builtin_amdgcn_logf(wl[ord]);
        }
      }
      skey[threadIdx.x] = key;
      slw[threadIdx.x] = lw;
    }
    __syncthreads();
    for (int p = threadIdx.x; p < TS * D; p += blockDim.x) {
      const int s = p / D, d = p % D;
      const int key = skey[s];
      Kt[s][d] = key >= 0 ? k[(size_t(bh) * N + key) * D + d] : 0.0f;
      Vv[s][d] = key >= 0 ? v[(size_t(bh) * N + key) * D + d] : 0.0f;
    }
    __syncthreads();
    for (int s = 0; s < TS; ++s) {
      if (skey[s] < 0) continue;
      float dot = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) dot = __builtin_fmaf(qv[d], Kt[s][d], dot);
      const float x = __builtin_fmaf(dot, c2, slw[s]);
      const float mn = fmaxf(m, x);
      const float alpha = fast_exp2(m - mn);
      const float pp = fast_exp2(x - mn);
      l = l * alpha + pp;
      m = mn;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(pp, Vv[s][d], o[d] * alpha);
    }
  }
  if (r < n) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int d = 0; d < D; ++d) out[(size_t(bh) * N + row0 + r) * D + d] = o[d] * inv;
    if (lse) lse[size_t(bh) * N + row0 + r] = l > 0.0f ? (m + fast_log2(l)) * kLn2 : -__builtin_inff();
  }
}

}  // namespace

hipError_t launch_attn_fwd(const Dims& P, const void* q, const void* k, const void* v, const int32_t* idx,
                           const float* weights, const int32_t* counts, void* out, float* lse, hipStream_t s) {
  const dim3 grid(P.B * P.H * P.nqb);
  if (P.bf16) {
    auto Q = static_cast<const uint16_t*>(q);
    auto Kp = static_cast<const uint16_t*>(k);
    auto Vp = static_cast<const uint16_t*>(v);
    auto O = static_cast<uint16_t*>(out);
    if (P.d == 128 && P.Bq == 128)
      hipLaunchKernelGGL((attn_fwd_bf16<128, 128>), grid, dim3(256), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse);
    else if (P.d == 128)
      hipLaunchKernelGGL((attn_fwd_bf16<128, 64>), grid, dim3(128), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse);
    else if (P.Bq == 128)
      hipLaunchKernelGGL((attn_fwd_bf16<64, 128>), grid, dim3(256), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse);
    else
      hipLaunchKernelGGL((attn_fwd_bf16<64, 64>), grid, dim3(128), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse);
  } else {
    auto Q = static_cast<const float*>(q);
    auto Kp = static_cast<const float*>(k);
    auto Vp = static_cast<const float*>(v);
    auto O = static_cast<float*>(out);
    if (P.d == 128)
      hipLaunchKernelGGL(attn_fwd_f32<128>, grid, dim3(P.Bq), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse);
    else
      hipLaunchKernelGGL(attn_fwd_f32<64>, grid, dim3(P.Bq), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse);
  }
  return hipGetLastError();
}

}  // namespace ab
