// Weighted block-sparse attention forward with sub-tile key gathering.
//
// AB-Attention abstract (paperdot search page, query "Xing Ma"): exact attention
// on the kept key/value blocks only (problem sentence); each kept block j is
// weighted by the inverse of its inclusion probability w_j in both the softmax
// numerator and denominator, which makes a single pass an unbiased
// Horvitz-Thompson estimate of the dense numerator and denominator (SIP
// sentence); kept sub-blocks, each holding far fewer keys than one matrix-core
// tile, are packed side by side to fill whole tiles (kernel sentence). The INTRA abstract (paperdot
// search page, query "Wenbo Lu") describes the same idea for static patterns:
// a FlashAttention-style kernel that loads non-contiguous tokens and packs them
// densely.
//
// bf16 design (gfx950, wave64): one workgroup per (b, h, query block); each
// wave owns 32 query rows (at q_block 64 and d 128, two waves per 32 rows, each
// with one 32-slot half of every tile, merged at the end). A tile is 64 key slots: the compacted list of kept
// sub-blocks is laid end to end, so a 64-slot tile holds 64/Bk sub-blocks for
// Bk <= 64 and half of one for Bk = 128; the gather is one coalesced run per
// sub-block row into LDS. The logits are computed transposed,
// S^T = K Q^T, with v_mfma_f32_32x32x16_bf16, so every lane owns one query row
// and 16 keys: the row max and row sum need one exchange between the two wave
// halves, and the probabilities are already in the B-operand layout of
// O^T += V^T P^T. The weight enters as log2(w_j) added to the logits of block
// j's keys, which multiplies numerator and denominator alike. The softmax
// reference is moved only when a row's sum of exponentials overflows its bound,
// so most tiles need no max pass. V is read from its natural [slot][d] layout
// with transposing LDS reads, two 8-byte reads per A operand.
#include "ab_internal.h"
#include "mfma.h"

namespace ab {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSlots = 64;

template <int D, int BQ, int BK>
struct AttnCfg {
  // Bq = 64 at d = 128: four waves, two per 32 query rows, each taking one 32-slot half
  // of every tile, so a CU still holds two workgroups of four waves (64 KB of LDS each;
  // with two waves per workgroup it would hold one wave per SIMD); the two softmax
  // states of a row are merged at the end.
  static constexpr bool kSplit = BQ == 64 && D == 128;
  static constexpr int kWaves = kSplit ? 4 : BQ / 32;  // each wave owns 32 query rows
  static constexpr int kHalves = kSplit ? 1 : 2;       // 32-slot halves of a tile per wave
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRowBytes = D * 2;          // one key row of K or V
  static constexpr int kChunks = D / 8;            // 16-byte chunks per row
  static constexpr int kTileBytes = kSlots * kRowBytes;
  static constexpr int kLoadsPerTile = kTileBytes / 1024;     // 64 lanes x 16 bytes per load
  static constexpr int kLoadsPerWave = kLoadsPerTile / kWaves;
  static constexpr int kSlotsPerLoad = 1024 / kRowBytes;      // 4 or 8: within one sub-block
  static constexpr int kWaveSlots = kSlots / kWaves;          // consecutive slots gathered by one wave
  static constexpr int kWaveEntries = BK >= kWaveSlots ? 1 : kWaveSlots / BK;  // sub-blocks per wave
  static constexpr int kTileEntries = BK >= kSlots ? 1 : kSlots / BK;         // sub-blocks per tile
  static constexpr int kEntryShift = __builtin_ctz(BK * kRowBytes);            // sub-block -> byte offset
  static_assert(kSlotsPerLoad <= BK, "one gather load must stay inside one sub-block");
};

// Tiles are unpadded [slot][d] rows whose 16-byte chunks are permuted by an XOR
// of the slot index, which makes both LDS read patterns conflict-free on
// gfx950 (measured): the K fragment read (32 rows, same chunk) and the
// transposed V read (4 rows x 64 bytes per half wave).
template <int D>
__device__ __forceinline__ int k_swz(int slot) {
  return kfrag_swz<D>(slot);
}
template <int D>
__device__ __forceinline__ int v_swz(int slot) {
  return D == 128 ? ((slot & 3) << 2) : (((slot >> 1) & 1) << 2);
}

// Sub-block of tile-relative slot s (s < 64): its index among the tile's entries.
template <int BK>
__device__ __forceinline__ constexpr int slot_entry(int s) {
  return BK >= kSlots ? 0 : s / BK;
}

template <int D, int BQ, int BK>
__global__ __launch_bounds__((AttnCfg<D, BQ, BK>::kThreads)) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(Dims P, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
                   const float* __restrict__ weights, const int32_t* __restrict__ counts,
                   uint16_t* __restrict__ out, float* __restrict__ lse, const int32_t* __restrict__ order,
                   int head_major) {
  using Cfg = AttnCfg<D, BQ, BK>;
  // Four separate LDS objects (K and V, two stages each): the compiler can then tell
  // that the gather landing in one stage does not alias the reads of the other, and
  // keeps its vector-memory waits out of the math.
  __shared__ __align__(16) unsigned char k0s[Cfg::kTileBytes];
  __shared__ __align__(16) unsigned char k1s[Cfg::kTileBytes];
  __shared__ __align__(16) unsigned char v0s[Cfg::kTileBytes];
  __shared__ __align__(16) unsigned char v1s[Cfg::kTileBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  constexpr int HB = Cfg::kHalves;
  const int qsel = Cfg::kSplit ? (wave & 1) : wave;  // this wave's 32 query rows
  const int sh = Cfg::kSplit ? (wave >> 1) : 0;      // its 32-slot half of each tile (split)
  int blk;  // (b*H + h)*nqb + i
  if (order) {  // the caller's processing order; rows outside the grid are skipped
    blk = order[xcd_remap(blockIdx.x, gridDim.x)];
    if (blk < 0 || blk >= int(gridDim.x)) return;
  } else {
    blk = head_major ? xcd_head_remap(blockIdx.x, P.B * P.H, P.nqb) : xcd_remap(blockIdx.x, gridDim.x);
  }
  const int i = blk % P.nqb, bh = blk / P.nqb;
  const int N = P.N;
  const int row0 = i * BQ;
  const int n = min(BQ, N - row0);
  // a count outside [0, NKB] is clamped, so no list or weight read leaves the row
  const int cnt = min(max(counts[blk], 0), P.nkb);
  const int32_t* list = idx + size_t(blk) * P.nkb;
  const float* wl = weights + size_t(blk) * P.nkb;
  // one head of K or V; rows at or beyond N read as zeros (buffer range check)
  const int head_bytes = N * Cfg::kRowBytes;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(k + size_t(bh) * N * D), (short)0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc((void*)(v + size_t(bh) * N * D), (short)0, head_bytes, 0x00020000);

  // Q^T as the B operand: lane -> query row (qsel*32 + col), 8 dims per k step
  const int qr = qsel * 32 + col;
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

  // key slots: the kept sub-blocks laid end to end; the ragged tail block (always the
  // last entry when kept) leaves its padding at the very end, so slot gs holds a real
  // key iff gs < vend
  const int total = cnt * BK;
  const int ntiles = ceil_div(total, kSlots);
  const int tail_pad = (cnt > 0 && list[cnt - 1] == P.nkb - 1) ? P.nkb * BK - N : 0;
  const int vend = total - tail_pad;

  // Kept-list entries and weights are fetched ahead with unconditional loads clamped
  // to the list, whose results are only consumed in a later iteration, so no wait on
  // them ever sits between a tile's gather and its math. Slots past the list end thus
  // gather a real sub-block again; the last tile masks them. Both go through buffer
  // (vector-memory) loads: a scalar load would share its wait counter with the LDS
  // reads of the math and stall them.
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)list, (short)0, P.nkb * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)wl, (short)0, P.nkb * 4, 0x00020000);
  // entries(t): the sub-blocks this wave gathers for tile t
  auto entries = [&](int t, int (&kv)[Cfg::kWaveEntries]) {
    const int ord0 = (t * kSlots + wave * Cfg::kWaveSlots) / BK;
#pragma unroll
    for (int e = 0; e < Cfg::kWaveEntries; ++e)
      kv[e] = __builtin_amdgcn_raw_buffer_load_b32(rl, uint32_t(min(ord0 + e, cnt - 1)) * 4, 0, 0);
  };
  // weights of the sub-blocks of tile t
  auto tile_weights = [&](int t, float (&wv)[Cfg::kTileEntries]) {
    const int ord0 = (t * kSlots) / BK;
#pragma unroll
    for (int e = 0; e < Cfg::kTileEntries; ++e)
      wv[e] = __builtin_bit_cast(float,
                                 __builtin_amdgcn_raw_buffer_load_b32(rw, uint32_t(min(ord0 + e, cnt - 1)) * 4, 0, 0));
  };
  // Per-lane constant part of each gather load's byte offset: the key row inside its
  // sub-block and the permuted 16-byte chunk. The sub-block part is added per tile.
  uint32_t kofs[Cfg::kLoadsPerWave], vofs[Cfg::kLoadsPerWave];
#pragma unroll
  for (int j = 0; j < Cfg::kLoadsPerWave; ++j) {
    const int slot = wave * Cfg::kWaveSlots + j * Cfg::kSlotsPerLoad + lane / Cfg::kChunks;  // row in the tile
    const int within = slot % BK;  // row inside its sub-block (tiles start on sub-block bounds for BK <= 64)
    const int pos = lane % Cfg::kChunks;
    kofs[j] = uint32_t(within * Cfg::kRowBytes + ((pos ^ k_swz<D>(slot)) << 4));
    vofs[j] = uint32_t(within * Cfg::kRowBytes + ((pos ^ v_swz<D>(slot)) << 4));
  }
  // asynchronous gather of tile t straight into LDS (no VGPR staging)
  auto issue_tile = [&](int t, unsigned char* kdst, unsigned char* vdst, const int (&kv)[Cfg::kWaveEntries]) {
    // a 128-key sub-block spans two tiles: odd tiles take its second half
    const uint32_t hoff = BK > kSlots ? uint32_t((t * kSlots) % BK) * Cfg::kRowBytes : 0u;
#pragma unroll
    for (int j = 0; j < Cfg::kLoadsPerWave; ++j) {
      const int e = Cfg::kWaveEntries == 1 ? 0 : (j * Cfg::kSlotsPerLoad) / BK;
      const uint32_t sb = (uint32_t(kv[e]) << Cfg::kEntryShift) + hoff;
      const int ld = wave * Cfg::kLoadsPerWave + j;
      buffer_load_lds16(rk, kdst + ld * 1024, sb + kofs[j]);
      buffer_load_lds16(rv, vdst + ld * 1024, sb + vofs[j]);
    }
  };
  // log2 weight of each of this lane's eight 4-slot groups (tile slots
  // (g/4)*32 + (g%4)*8 + half*4 + [0, 4))
  auto tile_lw = [&](const float (&wv)[Cfg::kTileEntries], float (&lwg)[8]) {
    float le[Cfg::kTileEntries];
#pragma unroll
    for (int e = 0; e < Cfg::kTileEntries; ++e) le[e] = __builtin_amdgcn_logf(wv[e]);
#pragma unroll
    for (int g = 0; g < 4 * HB; ++g) {
      if constexpr (Cfg::kSplit)
        lwg[g] = sh ? le[slot_entry<BK>(32 + (g & 3) * 8)] : le[slot_entry<BK>((g & 3) * 8)];
      else
        lwg[g] = le[slot_entry<BK>((g >> 2) * 32 + (g & 3) * 8)];
    }
  };

  // LDS byte offsets of this lane's fragment reads (independent of the tile)
  int koff[D / 16];  // K rows col (+32 for the second half), chunk 2*kk + half
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    koff[kk] = (sh * 32 + col) * Cfg::kRowBytes + (((2 * kk + half) ^ k_swz<D>(col)) << 4);
  // transposed V read: lane J of 16-lane group G points at slot (J%16)/4 of its group's
  // 4-slot run and dims 4*((J%16)%4) of its 16-dim half of each 32-dim block
  const int tgrp = lane >> 4, tj = lane & 15;
  const int tr_slot = ((tgrp >> 1) << 2) + (tj >> 2);
  int voff[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int byte = db * 64 + (tgrp & 1) * 32 + (tj & 3) * 8;  // logical byte within the row
    voff[db] = (sh * 32 + tr_slot) * Cfg::kRowBytes + ((((byte >> 4) ^ v_swz<D>(tr_slot)) << 4) | (byte & 15));
  }

  int kv[Cfg::kWaveEntries];
  float wv[Cfg::kTileEntries];
  if (ntiles > 0) {
    entries(0, kv);
    __builtin_amdgcn_s_waitcnt(0);
    issue_tile(0, k0s, v0s, kv);
    if (ntiles > 1) entries(1, kv);
    tile_weights(0, wv);
  }
  // Drain every load issued so far (the Q fragments included) so the compiler's
  // wait-count analysis does not keep waits on them inside the loop.
  __builtin_amdgcn_s_waitcnt(0);
  // One tile: wait for its gather, prefetch the next tile into the other stage, then
  // S^T = K Q^T, softmax with the inverse-probability weights, O^T += V^T P^T.
  auto step = [&](int t, const unsigned char* kc, const unsigned char* vc, unsigned char* kn, unsigned char* vn) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's gather of tile t has landed in LDS
    __syncthreads();                // ... and every other wave's; tile t-1 is fully consumed
    float lwg[8];
    tile_lw(wv, lwg);
    if (t + 1 < ntiles) issue_tile(t + 1, kn, vn, kv);  // lands while tile t is computed
    if (t + 2 < ntiles) entries(t + 2, kv);
    if (t + 1 < ntiles) tile_weights(t + 1, wv);
    // (split) a wave whose half of the tile holds only padding has nothing to add
    if (Cfg::kSplit && t * kSlots + sh * 32 >= vend) return;
    // S^T for this wave's 32-slot halves, as independent accumulation chains
    f32x16_t acc[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x16_t{};
    // The K fragments of step kk + 1 are read before the products of step kk are
    // issued, so each read has two products' time to land (the scheduling-group
    // barriers keep the compiler from sinking the reads next to their use).
    {
      uint4 kf[2][HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) kf[0][hb] = *reinterpret_cast<const uint4*>(kc + hb * 32 * Cfg::kRowBytes + koff[0]);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, HB, 0);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        if (kk + 1 < D / 16) {
#pragma unroll
          for (int hb = 0; hb < HB; ++hb)
            kf[(kk + 1) & 1][hb] = *reinterpret_cast<const uint4*>(kc + hb * 32 * Cfg::kRowBytes + koff[kk + 1]);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, HB, 0);
        }
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma32x32x16(as_bf16x8(kf[kk & 1][hb]), qf[kk], acc[hb]);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, HB, 0);
      }
    }
    // The V operands of the first D/32 products of O^T += V^T P^T are read now, so
    // they land while the softmax runs; the rest follow one 32-dim block behind the
    // products (a ring of D/32 operands).
    constexpr int kVdb = D / 32;
    uint4 vf[kVdb];
    auto vread = [&](int i) {  // operand of product i: 16-slot group i / kVdb, dim block i % kVdb
      const unsigned char* vrow = vc + 16 * (i / kVdb) * Cfg::kRowBytes;
      const uint2 lo = lds_read_tr16(vrow + voff[i % kVdb]);
      const uint2 hi = lds_read_tr16(vrow + 8 * Cfg::kRowBytes + voff[i % kVdb]);
      vf[i % kVdb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    };
#pragma unroll
    for (int i = 0; i < kVdb; ++i) vread(i);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kVdb, 0);
    // padding slots of the last tile get probability 0
    const bool ragged = (t + 1) * kSlots > vend;
    if (ragged) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int gs = t * kSlots + (sh + hb) * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (gs >= vend) acc[hb][e] = -__builtin_inff();
        }
    }
    // Probabilities 2^(x - m) against the running reference m, packed to bf16, and
    // the row sum. The reference is only moved (O and l rescaled, the tile redone)
    // when a row sum is not finite or passes 2^64: on a row's first tile (m = -inf)
    // and when the logits grow by more than about 64 - 6 in log2 units. Values up to
    // 2^64 are exact enough (relative rounding does not depend on magnitude) and keep
    // O and l far from overflow.
    // The row sum adds the bf16-rounded probabilities, two per dot2 instruction:
    // the same values the P V product uses.
    bf16x8_t pb[2 * HB];
    float ps;
    auto probs = [&]() {
#pragma unroll
      for (int g = 0; g < 4 * HB; ++g) {
        const float bias = lwg[g] - m;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          pb[g >> 1][(g & 1) * 4 + e] = __bf16(fast_exp2(__builtin_fmaf(acc[g >> 2][(g & 3) * 4 + e], c2, bias)));
      }
      const bf16x2_t ones = {__bf16(1.0f), __bf16(1.0f)};
      float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
      for (int j = 0; j < 2 * HB; ++j) {
        s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pb[j][0], pb[j][1]}, ones, s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pb[j][2], pb[j][3]}, ones, s1, false);
        s0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pb[j][4], pb[j][5]}, ones, s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2_t{pb[j][6], pb[j][7]}, ones, s1, false);
      }
      ps = pair_sum(s0 + s1);
    };
    probs();
    if (__builtin_amdgcn_ballot_w64(!(ps <= 1.8446744e19f)) != 0) {
      float amax = acc[0][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) amax = fmaxf(amax, acc[0][e]);
#pragma unroll
      for (int hb = 1; hb < HB; ++hb)
#pragma unroll
        for (int e = 0; e < 16; ++e) amax = fmaxf(amax, acc[hb][e]);
      float lwmax = lwg[0];
#pragma unroll
      for (int g = 1; g < 4 * HB; ++g) lwmax = fmaxf(lwmax, lwg[g]);
      // every row has a real key in the first slot of this wave's part of the tile (a
      // part holding only padding is skipped above), so the bound is finite
      const float mn = fmaxf(m, pair_max(__builtin_fmaf(amax, c2, lwmax)));
      const float alpha = fast_exp2(m - mn);  // 0 on the first tile (m = -inf)
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
      m = mn;
      probs();
    }
    l += ps;
    // O^T += V^T P^T over this wave's 16-slot groups; D/32 independent accumulators. The
    // wave raises its issue priority for these products, so on a SIMD shared with a
    // wave that is in its softmax the matrix core is fed first and the other wave's
    // VALU work fills the gaps.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 2 * HB * kVdb; ++i) {
      o[i % kVdb] = mfma32x32x16(as_bf16x8(vf[i % kVdb]), pb[i / kVdb], o[i % kVdb]);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
      if (i + kVdb < 2 * HB * kVdb) {
        vread(i + kVdb);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, k0s, v0s, k1s, v1s);
    if (t + 1 < ntiles) step(t + 1, k1s, v1s, k0s, v0s);
  }

  if constexpr (Cfg::kSplit) {
    // merge the two slot halves of each row: the second-half wave of a row pair hands
    // its reference, sum and O^T to the first through LDS (the K stages, now free)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    float4* xo = reinterpret_cast<float4*>(qsel ? k1s : k0s);  // 16 KB per row pair
    float* xm = reinterpret_cast<float*>(qsel ? v1s : v0s);
    if (sh == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          xo[(db * 4 + q4) * 64 + lane] = make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
      xm[lane] = m;
      xm[64 + lane] = l;
    }
    __syncthreads();
    if (sh == 1) return;
    const float m1 = xm[lane], l1 = xm[64 + lane];
    const float mt = fmaxf(m, m1);
    // a half that never saw a real key keeps m = -inf and contributes nothing
    const float f0 = mt == -__builtin_inff() ? 0.0f : fast_exp2(m - mt);
    const float f1 = mt == -__builtin_inff() ? 0.0f : fast_exp2(m1 - mt);
    l = l * f0 + l1 * f1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = xo[(db * 4 + q4) * 64 + lane];
        o[db][4 * q4 + 0] = o[db][4 * q4 + 0] * f0 + x.x * f1;
        o[db][4 * q4 + 1] = o[db][4 * q4 + 1] * f0 + x.y * f1;
        o[db][4 * q4 + 2] = o[db][4 * q4 + 2] * f0 + x.z * f1;
        o[db][4 * q4 + 3] = o[db][4 * q4 + 3] * f0 + x.w * f1;
      }
    m = mt;
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

// fp32 inputs: two threads per query row (lanes 2r and 2r + 1), each holding one half
// of the row's dims of q and of the output; the pair adds its two half dot products
// (a DPP swap of neighbouring lanes, the same sum in both). VALU products against LDS
// tiles of TS keys. The online softmax advances CH keys at a time (the chunk's
// probabilities summed among themselves first) and keeps the row sum and the output
// in fp64, which runs at the fp32 vector rate here: fp32 running sums rounded a long
// row's many small terms away (up to 2e-5 of the output on rows of a few thousand
// keys, more on longer ones).
template <int D>
__global__ __launch_bounds__(256) void attn_fwd_f32(Dims P, const float* __restrict__ q, const float* __restrict__ k,
                                                    const float* __restrict__ v, const int32_t* __restrict__ idx,
                                                    const float* __restrict__ weights,
                                                    const int32_t* __restrict__ counts, float* __restrict__ out,
                                                    float* __restrict__ lse, const int32_t* __restrict__ order) {
  constexpr int TS = 32, CH = 8, HD = D / 2;
  constexpr int RS = D + 2;  // LDS row: the second half starts one word late (another bank)
  __shared__ float Kt[TS][RS];
  __shared__ float Vv[TS][RS];
  __shared__ int skey[TS];
  __shared__ float slw[TS];
  int blk = blockIdx.x;
  if (order) {  // the caller's processing order; rows outside the grid are skipped
    blk = order[blk];
    if (blk < 0 || blk >= int(gridDim.x)) return;
  }
  const int i = blk % P.nqb, bh = blk / P.nqb;
  const int N = P.N, Bk = P.Bk, Bq = P.Bq;
  const int row0 = i * Bq;
  const int n = min(Bq, N - row0);
  const int cnt = min(max(counts[blk], 0), P.nkb);  // clamped to the row
  const int32_t* list = idx + size_t(blk) * P.nkb;
  const float* wl = weights + size_t(blk) * P.nkb;
  const int r = threadIdx.x >> 1, hv = threadIdx.x & 1;
  const int hoff = hv * (HD + 1);  // this thread's half of an LDS row
  float qv[HD];
  double o[HD];
#pragma unroll
  for (int d = 0; d < HD; ++d) {
    qv[d] = (r < n) ? q[(size_t(bh) * N + row0 + r) * D + hv * HD + d] : 0.0f;
    o[d] = 0.0;
  }
  float m = -__builtin_inff();
  double l = 0.0;
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
        if (kk >= 0 && kk < N) {  // entries outside the sequence contribute nothing
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
      const int c = d < HD ? d : d + 1;
      Kt[s][c] = key >= 0 ? k[(size_t(bh) * N + key) * D + d] : 0.0f;
      Vv[s][c] = key >= 0 ? v[(size_t(bh) * N + key) * D + d] : 0.0f;
    }
    __syncthreads();
    for (int s0 = 0; s0 < TS; s0 += CH) {
      float p[CH];
      float tm = -__builtin_inff();
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        float x = -__builtin_inff();  // keys outside the sequence weigh nothing
        if (skey[s0 + s] >= 0) {      // the same for every thread: skey is shared
          float dot = 0.0f;
#pragma unroll
          for (int d = 0; d < HD; ++d) dot = __builtin_fmaf(qv[d], Kt[s0 + s][hoff + d], dot);
          // quad_perm [1, 0, 3, 2]: the neighbouring lane's half (every lane is active)
          const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dot), 0xB1, 0xF, 0xF, false));
          x = __builtin_fmaf(dot + other, c2, slw[s0 + s]);
        }
        p[s] = x;
        tm = fmaxf(tm, x);
      }
      if (tm == -__builtin_inff()) continue;  // no key of the sequence in this chunk (uniform)
      const float mn = fmaxf(m, tm);
      const double alpha = fast_exp2(m - mn);  // 0 before the first key
      float ps = 0.0f;
#pragma unroll
      for (int s = 0; s < CH; ++s) {
        p[s] = fast_exp2(p[s] - mn);
        ps += p[s];
      }
      l = __builtin_fma(l, alpha, double(ps));
      m = mn;
#pragma unroll
      for (int d = 0; d < HD; ++d) {
        float t = 0.0f;
#pragma unroll
        for (int s = 0; s < CH; ++s) t = __builtin_fmaf(p[s], Vv[s0 + s][hoff + d], t);
        o[d] = __builtin_fma(o[d], alpha, double(t));
      }
    }
  }
  if (r < n) {
    const double inv = l > 0.0 ? 1.0 / l : 0.0;
#pragma unroll
    for (int d = 0; d < HD; ++d) out[(size_t(bh) * N + row0 + r) * D + hv * HD + d] = float(o[d] * inv);
    if (lse && hv == 0)
      lse[size_t(bh) * N + row0 + r] = l > 0.0 ? (m + fast_log2(float(l))) * kLn2 : -__builtin_inff();
  }
}

// When eight heads' K and V (what eight XCDs on eight different heads read at once)
// exceed the Infinity Cache, the query blocks are taken head-major (xcd_head_remap);
// otherwise each XCD keeps one contiguous range of query blocks (xcd_remap), the
// better order for its own L2. Measured on one box, same inputs: 75600 tokens x 40
// heads 9.65 -> 9.12 ms, 118800 x 24 heads 14.83 -> 13.63 ms; 32760 x 12 heads (all
// of K and V fit) 634 -> 644 us, so it keeps the contiguous ranges.

template <int D, int BQ, int BK>
hipError_t launch_bf16(const Dims& P, const void* q, const void* k, const void* v, const int32_t* idx,
                       const float* weights, const int32_t* counts, void* out, float* lse, const int32_t* order,
                       hipStream_t s) {
  const size_t head_kv = size_t(P.N) * D * 2 * sizeof(uint16_t);
  const int head_major = !order && size_t(kXcds) * head_kv > kMallBytes;
  hipLaunchKernelGGL((attn_fwd_bf16<D, BQ, BK>), dim3(P.B * P.H * P.nqb), dim3(AttnCfg<D, BQ, BK>::kThreads), 0, s,
                     P, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), idx, weights, counts, static_cast<uint16_t*>(out), lse, order,
                     head_major);
  return hipGetLastError();
}

template <int D, int BQ>
hipError_t launch_bf16_bk(const Dims& P, const void* q, const void* k, const void* v, const int32_t* idx,
                          const float* weights, const int32_t* counts, void* out, float* lse, const int32_t* order,
                          hipStream_t s) {
  switch (P.Bk) {
    case 16: return launch_bf16<D, BQ, 16>(P, q, k, v, idx, weights, counts, out, lse, order, s);
    case 32: return launch_bf16<D, BQ, 32>(P, q, k, v, idx, weights, counts, out, lse, order, s);
    case 64: return launch_bf16<D, BQ, 64>(P, q, k, v, idx, weights, counts, out, lse, order, s);
    default: return launch_bf16<D, BQ, 128>(P, q, k, v, idx, weights, counts, out, lse, order, s);
  }
}

}  // namespace

hipError_t launch_attn_fwd(const Dims& P, const void* q, const void* k, const void* v, const int32_t* idx,
                           const float* weights, const int32_t* counts, void* out, float* lse, const int32_t* order,
                           hipStream_t s) {
  if (P.bf16) {
    if (P.d == 128 && P.Bq == 128) return launch_bf16_bk<128, 128>(P, q, k, v, idx, weights, counts, out, lse, order, s);
    if (P.d == 128) return launch_bf16_bk<128, 64>(P, q, k, v, idx, weights, counts, out, lse, order, s);
    if (P.Bq == 128) return launch_bf16_bk<64, 128>(P, q, k, v, idx, weights, counts, out, lse, order, s);
    return launch_bf16_bk<64, 64>(P, q, k, v, idx, weights, counts, out, lse, order, s);
  }
  const dim3 grid(P.B * P.H * P.nqb);
  auto Q = static_cast<const float*>(q);
  auto Kp = static_cast<const float*>(k);
  auto Vp = static_cast<const float*>(v);
  auto O = static_cast<float*>(out);
  // two threads per query row
  if (P.d == 128)
    hipLaunchKernelGGL(attn_fwd_f32<128>, grid, dim3(2 * P.Bq), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse, order);
  else
    hipLaunchKernelGGL(attn_fwd_f32<64>, grid, dim3(2 * P.Bq), 0, s, P, Q, Kp, Vp, idx, weights, counts, O, lse, order);
  return hipGetLastError();
}

}  // namespace ab
