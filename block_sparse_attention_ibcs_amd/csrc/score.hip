// IBCS block-importance estimate (AB-Attention abstract, IBCS sentence).
//
// Every query block is stood in for by its C centroids mu_c with weights
// n_c / n_i. For centroid row c of block i and key sub-block j:
//   l_cj = log sum_{k in j} exp(scale * mu_c . k_k),   L_c = log sum_j exp(l_cj),
//   s_ij = sum_c (n_c / n_i) exp(l_cj - L_c).
//
// Stage 1 (score_lse): per (b, h) the centroids form an [NQB*C, d] matrix that
// is multiplied by the keys on the matrix cores. The product is computed
// transposed (keys x centroids), so each lane owns one centroid and 16 keys of
// a 32-key block: sub-block log-sum-exps are in-register reductions plus one
// exchange with the other half of the wave. Exponentials use a per-centroid
// reference that is only moved when the next block would overflow, so most
// blocks need no max pass. Results are base-2 log-sum-exps, stored as
// ell[b, h, i, j, c] (the C centroids of a block are contiguous), plus one
// partial log-sum-exp per (row, key split).
// Stage 2 (score_assemble): per (b, h, i), combine the split partials into
// L_c and write s_ij for every j.
#include "ab_internal.h"
#include "mfma.h"

namespace ab {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kTileKeys = 64;  // keys per LDS tile (two 32-key MFMA blocks)

template <int D>
struct LseCfg {
  static constexpr int kRowPitch = D * 2 + 16;                 // bytes per key row in LDS (padded)
  static constexpr int kTileBytes = kTileKeys * kRowPitch;      // one buffer
  static constexpr int kChunksPerRow = D / 8;                   // 16-byte chunks per key row
  static constexpr int kChunksPerThread = kTileKeys * kChunksPerRow / 256;
};

// Running base-2 log-sum-exp state of one centroid row held by a lane pair.
struct LseState {
  float mref;  // reference (log2 units)
  float tot;   // sum of 2^(x - mref) over every key seen in this split
  float sub;   // same, over the keys of the open sub-block (k_block >= 64)
};

template <int D>
__global__ __launch_bounds__(256) void score_lse_bf16(Dims P, int split_keys, int splits,
                                                      const uint16_t* __restrict__ keys,
                                                      const uint16_t* __restrict__ cent,
                                                      float* __restrict__ ell,
                                                      float* __restrict__ lpart) {
  using Cfg = LseCfg<D>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int bh = blockIdx.z;
  const int split = blockIdx.y;
  const int cr = blockIdx.x * 128 + wave * 32 + col;  // centroid row of this lane
  const bool row_ok = cr < P.mrows;
  const int N = P.N;
  const int key_begin = split * split_keys;
  const int key_end = min(N, key_begin + split_keys);

  // B operand: this lane's centroid, 8 dims per 16-wide k step.
  bf16x8_t bfrag[D / 16];
  {
    const uint16_t* src = cent + (size_t(bh) * P.mrows + cr) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 u = make_uint4(0, 0, 0, 0);
      if (row_ok) u = *reinterpret_cast<const uint4*>(src + kk * 16);
      bfrag[kk] = as_bf16x8(u);
    }
  }
  const size_t ell_row = row_ok ? (size_t(bh) * P.nqb + cr / P.C) * size_t(P.nkb) * P.C + (cr % P.C) : 0;
  const float c2 = P.scale * kLog2e;
  const int Bk = P.Bk;

  const uint16_t* kbase = keys + size_t(bh) * N * D;
  const int ntiles = ceil_div(key_end - key_begin, kTileKeys);

  // cooperative tile load: thread -> (row, chunk)
  uint4 stage[Cfg::kChunksPerThread];
  auto load_tile = [&](int t) {
    const int k0 = key_begin + t * kTileKeys;
#pragma unroll
    for (int r = 0; r < Cfg::kChunksPerThread; ++r) {
      const int p = tid + r * 256;
      const int row = p / Cfg::kChunksPerRow, ch = p % Cfg::kChunksPerRow;
      const int key = k0 + row;
      stage[r] = make_uint4(0, 0, 0, 0);
      if (key < key_end) stage[r] = *reinterpret_cast<const uint4*>(kbase + size_t(key) * D + ch * 8);
    }
  };
  auto store_tile = [&](int buf) {
    unsigned char* base = smem + buf * Cfg::kTileBytes;
#pragma unroll
    for (int r = 0; r < Cfg::kChunksPerThread; ++r) {
      const int p = tid + r * 256;
      const int row = p / Cfg::kChunksPerRow, ch = p % Cfg::kChunksPerRow;
      *reinterpret_cast<uint4*>(base + row * Cfg::kRowPitch + ch * 16) = stage[r];
    }
  };

  LseState st{-__builtin_inff(), 0.0f, 0.0f};
  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);
    const unsigned char* kt = smem + buf * Cfg::kTileBytes;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int kb = key_begin + t * kTileKeys + blk * 32;  // first key of this 32-key block
      if (kb >= key_end) break;
      f32x16_t acc = {};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 a = *reinterpret_cast<const uint4*>(kt + (blk * 32 + col) * Cfg::kRowPitch + (kk * 16 + half * 8) * 2);
        acc = mfma32x32x16(as_bf16x8(a), bfrag[kk], acc);
      }
      float x[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) x[e] = acc[e];
      if (kb + 32 > key_end) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kb + (e >> 2) * 8 + half * 4 + (e & 3);
          if (key >= key_end) x[e] = -__builtin_inff();
        }
      }
      // exponentials against the running reference; rebase when it is unset or would overflow
      float ev[16];
      float s_own = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ev[e] = fast_exp2(__builtin_fmaf(x[e], c2, -st.mref));
        s_own += ev[e];
      }
      float s_pair = s_own + swap_halves(s_own);
      if (!(s_pair < 1.8446744e19f)) {  // 2^64; also catches the unset reference (inf/NaN)
        float bm = x[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) bm = fmaxf(bm, x[e]);
        bm = fmaxf(bm, swap_halves(bm));
        const float nref = bm * c2;
        const float f = fast_exp2(st.mref - nref);  // 0 when the old reference was unset
        st.tot *= f;
        st.sub *= f;
        st.mref = nref;
        s_own = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          ev[e] = fast_exp2(__builtin_fmaf(x[e], c2, -st.mref));
          s_own += ev[e];
        }
        s_pair = s_own + swap_halves(s_own);
      }
      st.tot += s_pair;
      if (Bk == 16) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s0 += ev[e];
#pragma unroll
        for (int e = 8; e < 16; ++e) s1 += ev[e];
        s0 += swap_halves(s0);
        s1 += swap_halves(s1);
        const int j = kb / 16 + half;
        const float v = st.mref + fast_log2(half ? s1 : s0);
        if (row_ok && j < P.nkb) ell[ell_row + size_t(j) * P.C] = v;
      } else if (Bk == 32) {
        const int j = kb / 32;
        if (row_ok && half == 0) ell[ell_row + size_t(j) * P.C] = st.mref + fast_log2(s_pair);
      } else {
        st.sub += s_pair;
        const bool last = ((kb + 32) % Bk == 0) || (kb + 32 >= key_end);
        if (last) {
          const int j = kb / Bk;
          if (row_ok && half == 0) ell[ell_row + size_t(j) * P.C] = st.mref + fast_log2(st.sub);
          st.sub = 0.0f;
        }
      }
    }
  }
  if (row_ok && half == 0) lpart[(size_t(bh) * P.mrows + cr) * splits + split] = st.mref + fast_log2(st.tot);
}

// fp32 inputs: plain VALU dot products, one thread per (centroid, sub-block).
template <int D>
__global__ __launch_bounds__(256) void score_lse_f32(Dims P, const float* __restrict__ keys,
                                                     const float* __restrict__ cent, float* __restrict__ ell,
                                                     float* __restrict__ lpart) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x;
  const int C = P.C, N = P.N, Bk = P.Bk;
  __shared__ float Lm[128], Ls[128];
  const float c2 = P.scale * kLog2e;
  const float* kb = keys + size_t(bh) * N * D;
  const float* cb = cent + (size_t(bh) * P.nqb + i) * C * D;
  float* eb = ell + (size_t(bh) * P.nqb + i) * size_t(P.nkb) * C;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    Lm[c] = -__builtin_inff();
    Ls[c] = 0.0f;
  }
  __syncthreads();
  // pass 1: every (c, j) log-sum-exp
  for (int p = threadIdx.x; p < C * P.nkb; p += blockDim.x) {
    const int j = p / C, c = p % C;
    float m = -__builtin_inff(), s = 0.0f;
    const int k1 = min(N, (j + 1) * Bk);
    for (int key = j * Bk; key < k1; ++key) {
      float dot = 0.0f;
      for (int k = 0; k < D; ++k) dot = __builtin_fmaf(cb[c * D + k], kb[size_t(key) * D + k], dot);
      const float x = dot * c2;
      const float nm = fmaxf(m, x);
      s = s * fast_exp2(m - nm) + fast_exp2(x - nm);
      m = nm;
    }
    eb[size_t(j) * C + c] = m + fast_log2(s);
  }
  __syncthreads();
  // pass 2: each row's log-sum-exp over its sub-blocks (single split)
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float m = -__builtin_inff(), s = 0.0f;
    for (int j = 0; j < P.nkb; ++j) {
      const float x = eb[size_t(j) * C + c];
      const float nm = fmaxf(m, x);
      s = s * fast_exp2(m - nm) + fast_exp2(x - nm);
      m = nm;
    }
    lpart[(size_t(bh) * P.mrows + i * C + c)] = m + fast_log2(s);
  }
}

__global__ __launch_bounds__(256) void score_assemble(Dims P, int splits, const float* __restrict__ ell,
                                                      const float* __restrict__ lpart,
                                                      const int32_t* __restrict__ sizes,
                                                      float* __restrict__ scores) {
  __shared__ float Lc[128], wc[128];
  const int blk = blockIdx.x;  // (b*H + h)*nqb + i
  const int i = blk % P.nqb, bh = blk / P.nqb;
  const int C = P.C;
  const int n = min(P.Bq, P.N - i * P.Bq);
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    const float* lp = lpart + (size_t(bh) * P.mrows + i * C + c) * splits;
    float m = -__builtin_inff();
    for (int s = 0; s < splits; ++s) m = fmaxf(m, lp[s]);
    float acc = 0.0f;
    for (int s = 0; s < splits; ++s) acc += fast_exp2(lp[s] - m);
    Lc[c] = m + fast_log2(acc);
    wc[c] = float(sizes[size_t(blk) * C + c]) / float(n);
  }
  __syncthreads();
  const float* eb = ell + size_t(blk) * P.nkb * C;
  float* out = scores + size_t(blk) * P.nkb;
  for (int j = threadIdx.x; j < P.nkb; j += blockDim.x) {
    float s = 0.0f;
    for (int c = 0; c < C; ++c) {
      const float w = wc[c];
      if (w > 0.0f) s += w * fast_exp2(eb[size_t(j) * C + c] - Lc[c]);
    }
    out[j] = s;
  }
}

}  // namespace

ScoreWs score_ws_layout(const Dims& D, int num_cus) {
  ScoreWs L{};
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t heads = size_t(D.B) * D.H;
  // key splits: enough (row tile, split, head) workgroups for two waves of the chip
  int splits = 1;
  if (D.bf16) {
    const long tiles = long(ceil_div(D.mrows, 128)) * long(heads);
    const long want = 2L * num_cus;
    while (tiles * splits < want && splits < 64) splits *= 2;
    // at least two 64-key tiles per split
    const int max_splits = max(1, ceil_div(D.N, 256));
    splits = min(splits, max_splits);
  }
  int split_keys = ceil_div(ceil_div(D.N, splits), 128) * 128;
  splits = ceil_div(D.N, split_keys);
  L.splits = splits;
  L.split_keys = split_keys;
  size_t off = 0;
  L.centroids_f32 = off;
  off = al(off + heads * D.nqb * D.C * D.d * 4);
  L.centroids_bf16 = off;
  off = al(off + heads * D.nqb * D.C * D.d * 2);
  L.sizes = off;
  off = al(off + heads * D.nqb * D.C * 4);
  L.ell = off;
  off = al(off + heads * D.nqb * size_t(D.nkb) * D.C * 4);
  L.lpart = off;
  off = al(off + heads * D.mrows * size_t(splits) * 4);
  L.total = off;
  return L;
}

hipError_t launch_score_lse(const Dims& P, const ScoreWs& L, const void* k, const void* cent, float* ell,
                            float* lpart, hipStream_t s) {
  if (P.bf16) {
    const dim3 grid(ceil_div(P.mrows, 128), L.splits, P.B * P.H);
    if (P.d == 128) {
      const size_t lds = 2 * LseCfg<128>::kTileBytes;
      hipLaunchKernelGGL(score_lse_bf16<128>, grid, dim3(256), lds, s, P, L.split_keys, L.splits,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(cent), ell, lpart);
    } else {
      const size_t lds = 2 * LseCfg<64>::kTileBytes;
      hipLaunchKernelGGL(score_lse_bf16<64>, grid, dim3(256), lds, s, P, L.split_keys, L.splits,
                         static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(cent), ell, lpart);
    }
  } else {
    const dim3 grid(P.nqb, P.B * P.H);
    if (P.d == 128)
      hipLaunchKernelGGL(score_lse_f32<128>, grid, dim3(256), 0, s, P, static_cast<const float*>(k),
                         static_cast<const float*>(cent), ell, lpart);
    else
      hipLaunchKernelGGL(score_lse_f32<64>, grid, dim3(256), 0, s, P, static_cast<const float*>(k),
                         static_cast<const float*>(cent), ell, lpart);
  }
  return hipGetLastError();
}

hipError_t launch_score_assemble(const Dims& P, const ScoreWs& L, const float* ell, const float* lpart,
                                 const int32_t* sizes, float* scores, hipStream_t s) {
  hipLaunchKernelGGL(score_assemble, dim3(P.B * P.H * P.nqb), dim3(256), 0, s, P, L.splits, ell, lpart, sizes,
                     scores);
  return hipGetLastError();
}

}  // namespace ab
