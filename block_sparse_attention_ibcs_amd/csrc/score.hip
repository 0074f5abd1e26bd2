// IBCS block-importance estimate (AB-Attention abstract, IBCS sentence).
//
// Every query block is stood in for by its C centroids mu_c with weights
// n_c / n_i. For centroid row c of block i and key sub-block j:
//   l_cj = log sum_{k in j} exp(scale * mu_c . k_k),   L_c = log sum_j exp(l_cj),
//   s_ij = sum_c (n_c / n_i) exp(l_cj - L_c).
//
// Stage 1 (score_lse): per (b, h) the centroids form an [NQB*C, d] matrix that
// is multiplied by the keys on the matrix cores (the bf16 centroids carry
// scale * log2 e, so the products are base-2 logits). The product is computed
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
  static constexpr int kWaves = 4;
  static constexpr int kRows = kWaves * 64;                 // centroid rows per workgroup (64 per wave)
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = D / 8;                     // 16-byte chunks per key row
  static constexpr int kTileBytes = kTileKeys * kRowBytes;
  static constexpr int kLoadsPerWave = kTileBytes / 1024 / kWaves;
  static constexpr int kKeysPerLoad = 1024 / kRowBytes;
};

// Running base-2 log-sum-exp state of one centroid row (identical in the lane pair
// l, l ^ 32 that holds it).
struct LseState {
  float mref;  // reference (log2 units); only raised, and only when a block would overflow
  float tot;   // sum of 2^(x - mref) over every key seen in this split
  float sub;   // same, over the keys of the open sub-block (k_block >= 64)
};

// One centroid row group's epilogue for one 32-key block: base-2 logits x (this
// lane's 16 keys of the block; the centroid operand already carries scale * log2 e),
// running state st, first key of the block kb.
//
// The first block sets the reference: its maximum, or 0 when that maximum lies in
// [-40, 40] (then 2^x itself neither overflows nor loses the block's largest terms).
// While every row of the wave keeps reference 0 the exponentials take the logits
// as they are, one instruction per key instead of two. A block whose sum would
// pass 2^64 raises the reference of those rows to the running maximum (the sums
// so far are rescaled), and the block is redone against it.
template <int BK>
__device__ __forceinline__ void lse_block(const f32x16_t& acc, LseState& st, int kb, int key_end, int half,
                                          bool row_ok, float* ell_row, int C, int nkb) {
  // This lane's 16 keys: e < 8 lie in the block's first 16 keys, e >= 8 in the last 16.
  float ev[16];
  float s0, s1;  // this lane's sums over its keys of the first and of the last 16
  auto sums = [&]() {
    s0 = ev[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) s0 += ev[e];
    s1 = ev[8];
#pragma unroll
    for (int e = 9; e < 16; ++e) s1 += ev[e];
  };
  auto exps_ref = [&]() {
#pragma unroll
    for (int e = 0; e < 16; ++e) ev[e] = fast_exp2(acc[e] - st.mref);
    sums();
  };
  if (__builtin_amdgcn_ballot_w64(st.mref != 0.0f) == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) ev[e] = fast_exp2(acc[e]);  // reference 0 in every row
    sums();
  } else {
    exps_ref();
  }
  float s_pair = pair_sum(s0 + s1);
  // rebase the rows whose reference is unset (first block: x + inf) or whose sum
  // would pass 2^64
  const bool rebase = !(s_pair < 1.8446744e19f);
  if (__builtin_amdgcn_ballot_w64(rebase) != 0) {
    float bm = acc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) bm = fmaxf(bm, acc[e]);
    bm = pair_max(bm);
    float nref = st.mref;
    if (rebase) {
      nref = fmaxf(st.mref, bm);
      if (st.mref == -__builtin_inff() && nref >= -40.0f && nref <= 40.0f) nref = 0.0f;
    }
    const float f = fast_exp2(st.mref - nref);  // 0 when the old reference was unset, 1 when kept
    st.tot *= f;
    st.sub *= f;
    st.mref = nref;
    exps_ref();
    s_pair = pair_sum(s0 + s1);
  }
  st.tot += s_pair;
  if constexpr (BK == 16) {
    // half 0 stores the first sub-block and needs the other half's s0; half 1 the
    // second and needs s1: one exchange carries both
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(half ? s0 : s1), __float_as_uint(half ? s0 : s1),
                                                    false, false);
    const float other = __uint_as_float(half ? r[0] : r[1]);
    const float sub = (half ? s1 : s0) + other;
    const int j = kb / 16 + half;
    if (row_ok && j < nkb) ell_row[size_t(j) * C] = st.mref + fast_log2(sub);
  } else if constexpr (BK == 32) {
    if (row_ok && half == 0) ell_row[size_t(kb / 32) * C] = st.mref + fast_log2(s_pair);
  } else {
    st.sub += s_pair;
    if (((kb + 32) % BK == 0) || (kb + 32 >= key_end)) {
      if (row_ok && half == 0) ell_row[size_t(kb / BK) * C] = st.mref + fast_log2(st.sub);
      st.sub = 0.0f;
    }
  }
}

// Work item = (b*H + h, key split, row tile of 256 centroid rows), row tile fastest,
// remapped so an XCD holds consecutive row tiles of one head and split (same keys).
template <int D, int BK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 4)))
void score_lse_bf16(Dims P, int split_keys, int splits, int row_tiles, const uint16_t* __restrict__ keys,
                    const uint16_t* __restrict__ cent, float* __restrict__ ell, float* __restrict__ lpart) {
  using Cfg = LseCfg<D>;
  __shared__ __align__(16) unsigned char kb0[Cfg::kTileBytes];
  __shared__ __align__(16) unsigned char kb1[Cfg::kTileBytes];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int wid = xcd_remap(blockIdx.x, gridDim.x);
  const int rt = wid % row_tiles;
  const int split = (wid / row_tiles) % splits;
  const int bh = wid / (row_tiles * splits);
  const int N = P.N;
  const int key_begin = split * split_keys;
  const int key_end = min(N, key_begin + split_keys);
  const int ntiles = ceil_div(key_end - key_begin, kTileKeys);

  // B operands: this lane's two centroid rows (row groups), 8 dims per 16-wide k step
  int cr[2];
  bool row_ok[2];
  float* ell_row[2];
  bf16x8_t bfrag[2][D / 16];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    cr[rg] = rt * Cfg::kRows + wave * 64 + rg * 32 + col;
    row_ok[rg] = cr[rg] < P.mrows;
    const int r = min(cr[rg], P.mrows - 1);
    const uint16_t* src = cent + (size_t(bh) * P.mrows + r) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 u = *reinterpret_cast<const uint4*>(src + kk * 16);
      if (!row_ok[rg]) u = make_uint4(0, 0, 0, 0);
      bfrag[rg][kk] = as_bf16x8(u);
    }
    ell_row[rg] = ell + (size_t(bh) * P.nqb + r / P.C) * size_t(P.nkb) * P.C + (r % P.C);
  }
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(keys + size_t(bh) * N * D), (short)0, N * Cfg::kRowBytes, 0x00020000);
  // Per-lane constant part of each gather load's byte offset (key row in the tile,
  // permuted chunk). Keys past the split end but below N are gathered too and masked
  // in the math; rows at or past N read zeros through the buffer range check.
  uint32_t gofs[Cfg::kLoadsPerWave];
#pragma unroll
  for (int j = 0; j < Cfg::kLoadsPerWave; ++j) {
    const int krow = (wave * Cfg::kLoadsPerWave + j) * Cfg::kKeysPerLoad + lane / Cfg::kChunks;
    const int pos = lane % Cfg::kChunks;
    gofs[j] = uint32_t(krow * Cfg::kRowBytes + ((pos ^ kfrag_swz<D>(krow)) << 4));
  }
  auto issue_tile = [&](int t, unsigned char* dst) {
    const uint32_t base = uint32_t(key_begin + t * kTileKeys) * Cfg::kRowBytes;
#pragma unroll
    for (int j = 0; j < Cfg::kLoadsPerWave; ++j)
      buffer_load_lds16(rk, dst + (wave * Cfg::kLoadsPerWave + j) * 1024, base + gofs[j]);
  };
  int koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = col * Cfg::kRowBytes + (((2 * kk + half) ^ kfrag_swz<D>(col)) << 4);

  LseState st[2] = {{-__builtin_inff(), 0.0f, 0.0f}, {-__builtin_inff(), 0.0f, 0.0f}};
  if (ntiles > 0) issue_tile(0, kb0);
  __builtin_amdgcn_s_waitcnt(0);
  auto step = [&](int t, const unsigned char* kc, unsigned char* kn) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of tile t is in LDS
    __syncthreads();                // all of it; tile t-1 is consumed
    if (t + 1 < ntiles) issue_tile(t + 1, kn);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int kb = key_begin + t * kTileKeys + hb * 32;  // first key of this 32-key block (uniform)
      if (kb >= key_end) break;
      f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
      // the key fragment of step kk + 1 is read before the two products of step kk
      // are issued (the scheduling-group barriers keep that order)
      {
        uint4 kf[2];
        kf[0] = *reinterpret_cast<const uint4*>(kc + hb * 32 * Cfg::kRowBytes + koff[0]);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          if (kk + 1 < D / 16) {
            kf[(kk + 1) & 1] = *reinterpret_cast<const uint4*>(kc + hb * 32 * Cfg::kRowBytes + koff[kk + 1]);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
          }
          acc[0] = mfma32x32x16(as_bf16x8(kf[kk & 1]), bfrag[0][kk], acc[0]);
          acc[1] = mfma32x32x16(as_bf16x8(kf[kk & 1]), bfrag[1][kk], acc[1]);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
        }
      }
      if (kb + 32 > key_end) {  // ragged end of the keys
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool dead = kb + (e >> 2) * 8 + half * 4 + (e & 3) >= key_end;
          if (dead) {
            acc[0][e] = -__builtin_inff();
            acc[1][e] = -__builtin_inff();
          }
        }
      }
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) lse_block<BK>(acc[rg], st[rg], kb, key_end, half, row_ok[rg], ell_row[rg], P.C, P.nkb);
    }
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, kb0, kb1);
    if (t + 1 < ntiles) step(t + 1, kb1, kb0);
  }
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
    if (row_ok[rg] && half == 0) lpart[(size_t(bh) * P.mrows + cr[rg]) * splits + split] = st[rg].mref + fast_log2(st[rg].tot);
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
  // pass 2: each row's log-sum-exp over its sub-blocks (single split); the running
  // sum is kept in fp64 so that the many small terms of a long row are not rounded
  // away against it (in fp32, NKB additions can lose up to NKB * 2^-24 of the sum)
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float m = -__builtin_inff();
    double s = 0.0;
    for (int j = 0; j < P.nkb; ++j) {
      const float x = eb[size_t(j) * C + c];
      const float nm = fmaxf(m, x);
      s = __builtin_fma(s, double(fast_exp2(m - nm)), double(fast_exp2(x - nm)));
      m = nm;
    }
    lpart[(size_t(bh) * P.mrows + i * C + c)] = m + fast_log2(float(s));
  }
}

// s_j = sum_c (|cluster c| / n) 2^(ell_jc - L_c), L_c the row's base-2
// log-sum-exp over all keys, ascending c, empty clusters skipped. CT is the
// cluster count when it is fixed at compile time (float4 loads of the C values
// of a sub-block, four sub-blocks in flight per thread), 0 for any count.
template <int CT>
__global__ __launch_bounds__(256) void score_assemble(Dims P, int splits, const float* __restrict__ ell,
                                                      const float* __restrict__ lpart,
                                                      const int32_t* __restrict__ sizes,
                                                      float* __restrict__ scores) {
  __shared__ float Lc[128], wc[128];
  const int blk = blockIdx.x;  // (b*H + h)*nqb + i
  const int i = blk % P.nqb, bh = blk / P.nqb;
  const int C = CT > 0 ? CT : P.C;
  const int n = min(P.Bq, P.N - i * P.Bq);
  const int nkb = P.nkb;
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
  const float* eb = ell + size_t(blk) * nkb * C;
  float* out = scores + size_t(blk) * nkb;
  if constexpr (CT > 0) {
    constexpr int C4 = CT / 4;
    constexpr int U = 4;
    const float4* eb4 = reinterpret_cast<const float4*>(eb);
    for (int j0 = 0; j0 < nkb; j0 += U * 256) {
      float4 e[U][C4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = min(j0 + u * 256 + int(threadIdx.x), nkb - 1);
#pragma unroll
        for (int q = 0; q < C4; ++q) e[u][q] = eb4[size_t(j) * C4 + q];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < C4; ++q) {
          const float x[4] = {e[u][q].x, e[u][q].y, e[u][q].z, e[u][q].w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float w = wc[4 * q + t];
            const float v = w * fast_exp2(x[t] - Lc[4 * q + t]);
            s += (w > 0.0f) ? v : 0.0f;
          }
        }
        const int j = j0 + u * 256 + int(threadIdx.x);
        if (j < nkb) out[j] = s;
      }
    }
  } else {
    for (int j = threadIdx.x; j < nkb; j += blockDim.x) {
      float s = 0.0f;
      for (int c = 0; c < C; ++c) {
        const float w = wc[c];
        if (w > 0.0f) s += w * fast_exp2(eb[size_t(j) * C + c] - Lc[c]);
      }
      out[j] = s;
    }
  }
}

}  // namespace

ScoreWs score_ws_layout(const Dims& D, int num_cus) {
  ScoreWs L{};
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t heads = size_t(D.B) * D.H;
  // Key splits: all (row tile, split, head) workgroups do the same work, and a CU holds
  // three of them at once (occupancy 3), so the time goes as (rounds of resident
  // workgroups) x (keys per workgroup), plus about one tile of set-up per workgroup;
  // take the split count that minimises it (at least two 64-key tiles per split).
  int splits = 1;
  if (D.bf16) {
    const long tiles = long(ceil_div(D.mrows, 256)) * long(heads);
    const long slots = 3L * max(1, num_cus);
    const int max_splits = min(64, max(1, ceil_div(D.N, 256)));
    long best = -1;
    for (int s = 1; s <= max_splits; ++s) {
      const long sk = long(ceil_div(ceil_div(D.N, s), 128)) * 128;
      const long s_eff = (D.N + sk - 1) / sk;
      const long rounds = (tiles * s_eff + slots - 1) / slots;
      const long cost = rounds * (sk + 64);
      if (best < 0 || cost < best) {
        best = cost;
        splits = s;
      }
    }
  }
  const int split_keys = ceil_div(ceil_div(D.N, splits), 128) * 128;
  return score_ws_layout_split(D, split_keys);
}

ScoreWs score_ws_layout_split(const Dims& D, int split_keys) {
  ScoreWs L{};
  auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t heads = size_t(D.B) * D.H;
  const int splits = ceil_div(D.N, split_keys);
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

namespace {

template <int D, int BK>
void launch_lse_bf16(const Dims& P, const ScoreWs& L, const void* k, const void* cent, float* ell, float* lpart,
                     hipStream_t s) {
  const int row_tiles = ceil_div(P.mrows, LseCfg<D>::kRows);
  const int grid = row_tiles * L.splits * P.B * P.H;
  hipLaunchKernelGGL((score_lse_bf16<D, BK>), dim3(grid), dim3(256), 0, s, P, L.split_keys, L.splits, row_tiles,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(cent), ell, lpart);
}

template <int D>
void launch_lse_bf16_d(const Dims& P, const ScoreWs& L, const void* k, const void* cent, float* ell, float* lpart,
                       hipStream_t s) {
  switch (P.Bk) {
    case 16: launch_lse_bf16<D, 16>(P, L, k, cent, ell, lpart, s); break;
    case 32: launch_lse_bf16<D, 32>(P, L, k, cent, ell, lpart, s); break;
    case 64: launch_lse_bf16<D, 64>(P, L, k, cent, ell, lpart, s); break;
    default: launch_lse_bf16<D, 128>(P, L, k, cent, ell, lpart, s); break;
  }
}

}  // namespace

hipError_t launch_score_lse(const Dims& P, const ScoreWs& L, const void* k, const void* cent, float* ell, float* lpart,
                            hipStream_t s) {
  if (P.bf16) {
    if (P.d == 128) launch_lse_bf16_d<128>(P, L, k, cent, ell, lpart, s);
    else launch_lse_bf16_d<64>(P, L, k, cent, ell, lpart, s);
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
  const dim3 grid(P.B * P.H * P.nqb), block(256);
  switch (P.C) {
    case 4: hipLaunchKernelGGL(score_assemble<4>, grid, block, 0, s, P, L.splits, ell, lpart, sizes, scores); break;
    case 8: hipLaunchKernelGGL(score_assemble<8>, grid, block, 0, s, P, L.splits, ell, lpart, sizes, scores); break;
    case 16: hipLaunchKernelGGL(score_assemble<16>, grid, block, 0, s, P, L.splits, ell, lpart, sizes, scores); break;
    default: hipLaunchKernelGGL(score_assemble<0>, grid, block, 0, s, P, L.splits, ell, lpart, sizes, scores);
  }
  return hipGetLastError();
}

}  // namespace ab
