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

template <int D, int BQ>
struct AttnCfg {
  static constexpr int kThreads = BQ * 2;          // one wave per 32 query rows
  static constexpr int kPitch = D * 2 + 16;        // bytes per slot row of a K or V tile (padded)
  static constexpr int kTileBytes = kSlots * kPitch;
  static constexpr int kChunks = D / 8;            // 16-byte chunks per key row
  static constexpr int kPerThread = kSlots * kChunks / kThreads;  // chunks of one matrix per thread
  static constexpr int kWindow = 512;              // kept-list entries staged in LDS at a time
};

// LDS: two K tiles, two V tiles (natural [slot][d] layout), per-slot log-weights
// of both tiles, and a window of the kept-block list (first key, log2 weight).
template <int D, int BQ>
struct AttnSmem {
  using Cfg = AttnCfg<D, BQ>;
  unsigned char k[2][Cfg::kTileBytes];
  unsigned char v[2][Cfg::kTileBytes];
  float lw[2][kSlots];
  int ent_key[Cfg::kWindow];
  float ent_lw[Cfg::kWindow];
};

template <int D, int BQ>
__global__ __launch_bounds__(BQ * 2) __attribute__((amdgpu_waves_per_eu(BQ == 128 ? 2 : 1, 2))) void attn_fwd_bf16(Dims P, const uint16_t* __restrict__ q,
                                                         const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ weights,
                                                         const int32_t* __restrict__ counts,
                                                         uint16_t* __restrict__ out, float* __restrict__ lse) {
  using Cfg = AttnCfg<D, BQ>;
  constexpr int NT = Cfg::kThreads;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  AttnSmem<D, BQ>& sm = *reinterpret_cast<AttnSmem<D, BQ>*>(smem_raw);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int blk = blockIdx.x;  // (b*H + h)*nqb + i
  const int i = blk % P.nqb, bh = blk / P.nqb;
  const int N = P.N, Bk = P.Bk;
  const int bk_shift = __builtin_ctz(Bk);
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
    const uint16_t* src = q + (size_t(bh) * N + row0 + min(qr, n - 1)) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 u = *reinterpret_cast<const uint4*>(src + kk * 16);
      if (qr >= n) u = make_uint4(0, 0, 0, 0);
      qf[kk] = as_bf16x8(u);
    }
  }
  f32x16_t o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16_t{};
  float m = -__builtin_inff(), l = 0.0f;
  const float c2 = P.scale * kLog2e;

  const int total = cnt << bk_shift;  // key slots, padding of the ragged tail block included
  const int ntiles = ceil_div(total, kSlots);
  int ebase = 0;  // first list entry held in the LDS window

  auto stage_window = [&](int first) {
    for (int e = tid; e < Cfg::kWindow; e += NT) {
      const int ord = first + e;
      int key0 = 0x7FFFFFFF;
      float lw = -__builtin_inff();
      if (ord < cnt) {
        key0 = list[ord] << bk_shift;
        lw = __builtin_amdgcn_logf(wl[ord]);
      }
      sm.ent_key[e] = key0;
      sm.ent_lw[e] = lw;
    }
  };

  // register staging of one tile: kPerThread K chunks and as many V chunks
  uint4 sk[Cfg::kPerThread], sv[Cfg::kPerThread];
  float slw = -__builtin_inff();
  auto load_tile = [&](int t) {
#pragma unroll
    for (int r = 0; r < Cfg::kPerThread; ++r) {
      const int p = tid + r * NT;
      const int s = p / Cfg::kChunks, ch = p - s * Cfg::kChunks;
      const int gs = t * kSlots + s;
      const int ord = gs >> bk_shift;
      const int key = (ord < cnt) ? sm.ent_key[ord - ebase] + (gs & (Bk - 1)) : N;
      sk[r] = make_uint4(0, 0, 0, 0);
      sv[r] = make_uint4(0, 0, 0, 0);
      if (key < N) {
        sk[r] = *reinterpret_cast<const uint4*>(kh + size_t(key) * D + ch * 8);
        sv[r] = *reinterpret_cast<const uint4*>(vh + size_t(key) * D + ch * 8);
      }
    }
    if (tid < kSlots) {
      const int gs = t * kSlots + tid;
      const int ord = gs >> bk_shift;
      slw = -__builtin_inff();
      if (ord < cnt && sm.ent_key[ord - ebase] + (gs & (Bk - 1)) < N) slw = sm.ent_lw[ord - ebase];
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < Cfg::kPerThread; ++r) {
      const int p = tid + r * NT;
      const int s = p / Cfg::kChunks, ch = p - s * Cfg::kChunks;
      *reinterpret_cast<uint4*>(sm.k[buf] + s * Cfg::kPitch + ch * 16) = sk[r];
      *reinterpret_cast<uint4*>(sm.v[buf] + s * Cfg::kPitch + ch * 16) = sv[r];
    }
    if (tid < kSlots) sm.lw[buf][tid] = slw;
  };
  // the kept-list window must cover every entry tile t touches
  auto ensure_window = [&](int t) {
    const int last_ord = min(cnt - 1, ((t + 1) * kSlots - 1) >> bk_shift);
    if (last_ord >= ebase + Cfg::kWindow) {
      ebase = (t * kSlots) >> bk_shift;
      __syncthreads();  // nobody reads the old window any more
      stage_window(ebase);
      __syncthreads();
    }
  };

  // per-lane constants of the transposed V read: lane J of 16-lane group G points at
  // slot (J%16)/4 of its group's 4-slot run and dims 4*((J%16)%4) of its 16-dim half
  const int tgrp = lane >> 4, tj = lane & 15;
  const int tr_slot = ((tgrp >> 1) << 2) + (tj >> 2);
  const int tr_dim = ((tgrp & 1) << 4) + ((tj & 3) << 2);

  if (ntiles > 0) {
    stage_window(0);
    __syncthreads();
    load_tile(0);
    store_tile(0);
    __syncthreads();
  }
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) {
      ensure_window(t + 1);
      load_tile(t + 1);  // global loads in flight during this tile's math
    }
    const unsigned char* kt = sm.k[buf];
    const unsigned char* vt = sm.v[buf];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      if (t * kSlots + hb * 32 >= total) break;
      f32x16_t acc = {};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 a = *reinterpret_cast<const uint4*>(kt + (hb * 32 + col) * Cfg::kPitch + (kk * 16 + half * 8) * 2);
        acc = mfma32x32x16(as_bf16x8(a), qf[kk], acc);
      }
      // per-slot log2 weights of this lane's 16 keys (4 runs of 4 consecutive slots)
      float lw[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const float4 w4 = *reinterpret_cast<const float4*>(&sm.lw[buf][hb * 32 + g4 * 8 + half * 4]);
        lw[4 * g4 + 0] = w4.x;
        lw[4 * g4 + 1] = w4.y;
        lw[4 * g4 + 2] = w4.z;
        lw[4 * g4 + 3] = w4.w;
      }
      // probabilities against the running row max; the max is only moved (and O
      // rescaled) when some probability of this block would exceed 2^8
      float p[16];
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(acc[e], c2, lw[e] - m));
        ps += p[e];
      }
      ps = pair_sum(ps);
      if (__builtin_amdgcn_ballot_w64(!(ps <= 256.0f)) != 0) {
        float mx = -__builtin_inff();
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, __builtin_fmaf(acc[e], c2, lw[e]));
        mx = pair_max(mx);
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mn);  // 0 on the first block (m = -inf)
        l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
        m = mn;
        ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          p[e] = fast_exp2(__builtin_fmaf(acc[e], c2, lw[e] - m));
          ps += p[e];
        }
        ps = pair_sum(ps);
      }
      l += ps;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        bf16x8_t pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = __bf16(p[8 * g + e]);
        const int s0 = hb * 32 + 16 * g + tr_slot;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const unsigned char* base = vt + s0 * Cfg::kPitch + (db * 32 + tr_dim) * 2;
          const uint2 lo = lds_read_tr16(base);
          const uint2 hi = lds_read_tr16(base + 8 * Cfg::kPitch);
          o[db] = mfma32x32x16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pb, o[db]);
        }
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
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

template <int D, int BQ>
hipError_t launch_bf16(const Dims& P, const void* q, const void* k, const void* v, const int32_t* idx,
                       const float* weights, const int32_t* counts, void* out, float* lse, hipStream_t s) {
  auto kern = attn_fwd_bf16<D, BQ>;
  const size_t lds = sizeof(AttnSmem<D, BQ>);
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(P.B * P.H * P.nqb), dim3(AttnCfg<D, BQ>::kThreads), lds, s, P,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     idx, weights, counts, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const Dims& P, const void* q, const void* k, const void* v, const int32_t* idx,
                           const float* weights, const int32_t* counts, void* out, float* lse, hipStream_t s) {
  if (P.bf16) {
    if (P.d == 128 && P.Bq == 128) return launch_bf16<128, 128>(P, q, k, v, idx, weights, counts, out, lse, s);
    if (P.d == 128) return launch_bf16<128, 64>(P, q, k, v, idx, weights, counts, out, lse, s);
    if (P.Bq == 128) return launch_bf16<64, 128>(P, q, k, v, idx, weights, counts, out, lse, s);
    return launch_bf16<64, 64>(P, q, k, v, idx, weights, counts, out, lse, s);
  }
  const dim3 grid(P.B * P.H * P.nqb);
  auto Q = static_cast<const float*>(q);
  auto Kp = static_cast<const float*>(k);
  auto Vp = static_cast<const float*>(v);
  auto O = static_cast<float*>(out);
  if (P.d == 128)
    hipLaunchKernelGGL(attn_fwd_f32<128>, grid, dim3(P.Bq), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse);
  else
    hipLaunchKernelGGL(attn_fwd_f32<64>, grid, dim3(P.Bq), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse);
  return hipGetLastError();
}

}  // namespace ab
