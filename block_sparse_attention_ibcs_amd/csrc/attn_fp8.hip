// FP8 weighted block-sparse attention (VC-Attention page, iitak.ru news on
// MiniMax-H3: 8-bit products, V-Smooth, ExpCast-FP8; applied to the kept
// sub-blocks of AB-Attention's SIP sampler as in the bf16 kernel).
//
// Operands come from ab_fp8_prepare: E4M3 codes of Q (one scale per query
// block), K (one scale per key sub-block), the V residual after V-Smooth (one
// scale per head, operand order) and the sub-block means divided by that scale.
// Per 64-slot tile of the kept list and per query row r (one lane pair):
//   S^T = Kc Qc^T on v_mfma_f32_32x32x64_f8f6f4 (exact products, fp32 sums);
//   x = S * (qscale * kscale_j * scale * log2 e) + log2 w_j, the row reference m
//   raised to the tile maximum (O and l rescaled by 2^(m_old - m) when it moves);
//   ExpCast-FP8: the probability's E4M3 code is round(8 (x - m) + 126), clamped
//   to [0, 126] by v_cvt_pk_u8_f32, written straight into the packed B operand;
//   O^T += Vc^T P^T (FP8), and one more FP8 product against indicator rows gives
//   each row's sum of P over every sub-block t of the tile (S_t); l += sum S_t;
//   V-Smooth add-back O^T += mean'^T S^T on v_mfma_f32_32x32x16_bf16 with mean'
//   and S split into bf16 hi + lo pairs.
// out = vscale * O / l, lse = (m + log2 l - 8.75) ln 2.
//
// Layouts (one workgroup = 128 query rows, four waves of 32; head dim 128):
//   K tile in LDS: [64 slots][128 bytes], 16-byte chunks XOR-permuted by slot & 7.
//   V tile: [half][sub-block][dim][k_block/2] (k_block <= 64) or [half][dim][32]
//   (k_block 128: half of a sub-block per tile): a lane's 32-byte A operand (its
//   dim, its half of the 64 slots) is one to four contiguous runs, in the order in
//   which the lane holds the matching probabilities (slot (e/16)*32 + ((e%16)/4)*8
//   + half*4 + e%4 at byte e).
//   Means: [sub-block][dim] bf16 pairs.
#include "ab_internal.h"
#include "mfma.h"

namespace ab {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kSlots = 64;
constexpr int kD = 128;
constexpr float kTopCode = 126.0f;    // E4M3 code of the row reference (448)
constexpr float kLog2Top = 8.75f;     // a code c stands for 2^((c - 56) / 8)

typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int BK>
struct Fp8Cfg {
  static constexpr int kT = BK >= kSlots ? 1 : kSlots / BK;   // sub-blocks per tile
  static constexpr int kRun = BK >= kSlots ? 32 : BK / 2;     // bytes of one sub-block per (half, dim)
  static constexpr int kTileBytes = kSlots * kD;              // K or V tile: 8 KB
  static constexpr int kMeanBytes = 4 * kD * 4;               // up to 4 sub-blocks x 128 dims x 4 bytes
};

template <int BK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void attn_fwd_fp8(Dims P, const uint8_t* __restrict__ qcode, const float* __restrict__ qscale,
                  const uint8_t* __restrict__ kcode, const float* __restrict__ kscale,
                  const uint8_t* __restrict__ vcode, const float* __restrict__ vscale,
                  const uint32_t* __restrict__ vms, const int32_t* __restrict__ idx,
                  const float* __restrict__ weights, const int32_t* __restrict__ counts,
                  uint16_t* __restrict__ out, float* __restrict__ lse, int head_major) {
  using Cfg = Fp8Cfg<BK>;
  constexpr int kT = Cfg::kT;
  // separate LDS objects per stage: the gather landing in one stage never aliases
  // the reads of the other, so no vector-memory wait sits in the math
  __shared__ __align__(16) unsigned char k0s[Cfg::kTileBytes];
  __shared__ __align__(16) unsigned char k1s[Cfg::kTileBytes];
  __shared__ __align__(16) unsigned char v0s[Cfg::kTileBytes];
  __shared__ __align__(16) unsigned char v1s[Cfg::kTileBytes];
  __shared__ __align__(16) unsigned char m0s[Cfg::kMeanBytes];
  __shared__ __align__(16) unsigned char m1s[Cfg::kMeanBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  // (b*H + h)*nqb + i, head-major when the gathered operands of eight heads exceed the
  // Infinity Cache (as in the bf16 kernel)
  const int blk = head_major ? xcd_head_remap(blockIdx.x, P.B * P.H, P.nqb) : xcd_remap(blockIdx.x, gridDim.x);
  const int i = blk % P.nqb, bh = blk / P.nqb;
  const int N = P.N;
  const int row0 = i * 128;
  const int n = min(128, N - row0);
  const int cnt = min(max(counts[blk], 0), P.nkb);  // clamped to the row: no read leaves it
  const int32_t* list = idx + size_t(blk) * P.nkb;
  const float* wl = weights + size_t(blk) * P.nkb;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kcode + size_t(bh) * N * kD), (short)0, N * kD, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vcode + size_t(bh) * P.nkb * kD * BK), (short)0, P.nkb * kD * BK, 0x00020000);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(vms + size_t(bh) * P.nkb * kD), (short)0, P.nkb * kD * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)list, (short)0, P.nkb * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)wl, (short)0, P.nkb * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t rks = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kscale + size_t(bh) * P.nkb), (short)0, P.nkb * 4, 0x00020000);

  // Q^T as the B operand: lane -> query row wave*32 + col, dims kk*64 + half*32 + [0, 32)
  const int qr = wave * 32 + col;
  i32x8_t qf[2];
  {
    const uint8_t* src = qcode + (size_t(bh) * N + row0 + min(qr, n - 1)) * kD + half * 32;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 u0 = *reinterpret_cast<const uint4*>(src + kk * 64);
      uint4 u1 = *reinterpret_cast<const uint4*>(src + kk * 64 + 16);
      if (qr >= n) u0 = u1 = make_uint4(0, 0, 0, 0);
      qf[kk] = i32x8_t{int(u0.x), int(u0.y), int(u0.z), int(u0.w), int(u1.x), int(u1.y), int(u1.z), int(u1.w)};
    }
  }
  const float qsc = qscale[blk] * (P.scale * kLog2e);
  const float vsc = vscale[bh] > 0.0f ? vscale[bh] : 1.0f;
  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16_t{};
  float m = -__builtin_inff(), l = 0.0f;

  const int total = cnt * BK;
  const int ntiles = ceil_div(total, kSlots);
  const int tail_pad = (cnt > 0 && list[cnt - 1] == P.nkb - 1) ? P.nkb * BK - N : 0;
  const int vend = total - tail_pad;

  // indicator rows of the sub-block sums: rows 0-3 and 4-7 both mark sub-block
  // row % 4, so either half of a lane pair receives every sum
  i32x8_t ind;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const int e = w * 4 + e4;
      const int s = BK >= kSlots ? 0 : e / (BK / 2);
      if (col < 8 && (col & 3) < kT && s == (col & 3)) word |= 0x38u << (8 * e4);
    }
    ind[w] = int(word);
  }

  // Gather offsets. K: wave w loads slots w*16 + j*8 + lane/8 (j = 0, 1), 16-byte
  // chunk lane%8 of the LDS row holding global chunk (lane%8) ^ (slot & 7).
  uint32_t kofs[2], vofs[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = (wave * 2 + j) * 8 + lane / 8;
    const int p = lane % 8;
    kofs[j] = uint32_t((BK >= kSlots ? r : r % BK) * kD + ((p ^ (r & 7)) << 4));
    const int ld = wave * 2 + j;  // 1 KB of the V tile
    if constexpr (BK <= kSlots) {
      const int wo = (ld % 4) * 1024 + lane * 16;    // offset within the half
      vofs[j] = uint32_t((ld / 4) * (64 * BK) + wo % (64 * BK));
    } else {
      const int d = (ld % 4) * 32 + lane / 2;
      vofs[j] = uint32_t((ld / 4) * (64 * BK) + d * 64 + (lane % 2) * 16);
    }
  }
  // sub-block (within the tile) of wave w's K slots and of V load j
  const int ks_idx = BK >= kSlots ? 0 : (wave * 16) / BK;
  auto v_sidx = [&](int j) -> int {
    if constexpr (BK >= kSlots) return 0;
    else return (((wave * 2 + j) % 4) * 1024) / (64 * BK);
  };

  // kept-list entries of tile t (clamped loads: slots past the list gather a real
  // sub-block again and the last tile masks them)
  auto entries = [&](int t, int (&tv)[kT]) {
    const int ord0 = (t * kSlots) / BK;
#pragma unroll
    for (int s = 0; s < kT; ++s) tv[s] = __builtin_amdgcn_raw_buffer_load_b32(rl, uint32_t(min(ord0 + s, cnt - 1)) * 4, 0, 0);
  };
  // log2 weights and K scales of tile t's sub-blocks
  auto tile_consts = [&](int t, const int (&tv)[kT], float (&tw)[kT], float (&tk)[kT]) {
    const int ord0 = (t * kSlots) / BK;
#pragma unroll
    for (int s = 0; s < kT; ++s) {
      tw[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rw, uint32_t(min(ord0 + s, cnt - 1)) * 4, 0, 0));
      tk[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rks, uint32_t(tv[s]) * 4, 0, 0));
    }
  };
  auto issue_tile = [&](int t, unsigned char* kd, unsigned char* vd, unsigned char* md, const int (&tv)[kT]) {
    const int th = BK > kSlots ? (t & 1) : 0;  // which half of a 128-key sub-block
    const uint32_t kb = uint32_t(tv[ks_idx]) * BK * kD + uint32_t(th * kSlots * kD);
#pragma unroll
    for (int j = 0; j < 2; ++j) buffer_load_lds16(rk, kd + (wave * 2 + j) * 1024, kb + kofs[j]);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t vb = uint32_t(tv[v_sidx(j)]) * BK * kD + uint32_t(th * 32);
      buffer_load_lds16(rv, vd + (wave * 2 + j) * 1024, vb + vofs[j]);
    }
    // means: kT * 512 bytes, 1 KB per load, waves 3 and 2
    constexpr int kMeanLoads = (kT * 512 + 1023) / 1024;
    const int ml = 3 - wave;
    if (ml < kMeanLoads) {
      const int c = ml * 64 + lane;  // 16-byte chunk
      const int s = c / 32;
      if (s < kT) buffer_load_lds16(rm, md + ml * 1024, uint32_t(tv[min(s, kT - 1)]) * (kD * 4) + (c % 32) * 16);
    }
  };

  // LDS read offsets of this lane's operands
  int koff[2][2];  // [hb][kk], two 16-byte reads at +0 and at the next chunk
  int koff2[2][2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r = hb * 32 + col;
      const int c = kk * 4 + half * 2;
      koff[hb][kk] = r * kD + ((c ^ (r & 7)) << 4);
      koff2[hb][kk] = r * kD + (((c + 1) ^ (r & 7)) << 4);
    }
  int vrd[4];  // start of this lane's first run for dim block db
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 32 + col;
    vrd[db] = half * 4096 + d * Cfg::kRun;  // each half of the tile's slots takes 4 KB
  }

  int tv[kT];
  float tw[kT], tk[kT];
  if (ntiles > 0) {
    entries(0, tv);
    __builtin_amdgcn_s_waitcnt(0);
    issue_tile(0, k0s, v0s, m0s, tv);
    tile_consts(0, tv, tw, tk);
    if (ntiles > 1) entries(1, tv);
  }
  __builtin_amdgcn_s_waitcnt(0);

  auto step = [&](int t, const unsigned char* kc, const unsigned char* vc, const unsigned char* mc, unsigned char* kn,
                  unsigned char* vn, unsigned char* mn) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of tile t, and the loads below, have landed
    __syncthreads();                // ... every wave's; tile t-1 is consumed
    // per-group constants of tile t (group g = hb*4 + i/4 covers slots hb*32 + (i/4)*8 + half*4 + [0, 4))
    float ag[8], bg[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int s = BK >= kSlots ? 0 : ((g >> 2) * 32 + (g & 3) * 8) / BK;
      // (a zero scale means zero codes and zero products; the tiny floor keeps masked
      // keys at -inf instead of -inf * 0)
      ag[g] = fmaxf(qsc * tk[s], 1e-30f);
      bg[g] = __builtin_amdgcn_logf(tw[s]);
    }
    if (t + 1 < ntiles) {
      issue_tile(t + 1, kn, vn, mn, tv);
      tile_consts(t + 1, tv, tw, tk);
    }
    if (t + 2 < ntiles) entries(t + 2, tv);

    // S^T for the two 32-slot halves
    f32x16_t acc[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      acc[hb] = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint4 a0 = *reinterpret_cast<const uint4*>(kc + koff[hb][kk]);
        const uint4 a1 = *reinterpret_cast<const uint4*>(kc + koff2[hb][kk]);
        const i32x8_t a = {int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
        acc[hb] = mfma_fp8(a, qf[kk], acc[hb]);
      }
    }
    const bool ragged = (t + 1) * kSlots > vend;
    if (ragged) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int gs = t * kSlots + hb * 32 + (e >> 2) * 8 + half * 4 + (e & 3);
          if (gs >= vend) acc[hb][e] = -__builtin_inff();
        }
    }
    // tile maximum of x = acc * a_g + b_g (a_g >= 0)
    float mx = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const f32x16_t& a = acc[g >> 2];
      const int e0 = (g & 3) * 4;
      const float mg = fmaxf(fmaxf(a[e0], a[e0 + 1]), fmaxf(a[e0 + 2], a[e0 + 3]));
      mx = fmaxf(mx, __builtin_fmaf(mg, ag[g], bg[g]));
    }
    const float mnew = fmaxf(m, pair_max(mx));
    if (__builtin_amdgcn_ballot_w64(mnew > m) != 0) {
      const float alpha = fast_exp2(m - mnew);  // 0 on the first tile (m = -inf)
      l *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m = mnew;
    }
    // ExpCast-FP8 codes, packed four to a register in the B operand order
    i32x8_t pk;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const f32x16_t& a = acc[g >> 2];
      const int e0 = (g & 3) * 4;
      const float a8 = 8.0f * ag[g];
      const float c8 = __builtin_fmaf(8.0f, bg[g] - m, kTopCode);
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e)  // masked keys: -inf -> code 0
        word = __builtin_amdgcn_cvt_pk_u8_f32(__builtin_fmaf(a[e0 + e], a8, c8), e, word);
      pk[g] = int(word);
    }
    // O^T += Vc^T P^T, the sums of P and the V-Smooth add-back: the wave raises its
    // issue priority for these products (the other wave of the SIMD is then
    // usually in its softmax, whose VALU work fills the gaps)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x8_t a;
      if constexpr (BK == 16) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint2 u = *reinterpret_cast<const uint2*>(vc + vrd[db] + s * (64 * BK));
          a[2 * s] = int(u.x);
          a[2 * s + 1] = int(u.y);
        }
      } else if constexpr (BK == 32) {
        const uint4 u0 = *reinterpret_cast<const uint4*>(vc + vrd[db]);
        const uint4 u1 = *reinterpret_cast<const uint4*>(vc + vrd[db] + 64 * BK);
        a = i32x8_t{int(u0.x), int(u0.y), int(u0.z), int(u0.w), int(u1.x), int(u1.y), int(u1.z), int(u1.w)};
      } else {
        const uint4 u0 = *reinterpret_cast<const uint4*>(vc + vrd[db]);
        const uint4 u1 = *reinterpret_cast<const uint4*>(vc + vrd[db] + 16);
        a = i32x8_t{int(u0.x), int(u0.y), int(u0.z), int(u0.w), int(u1.x), int(u1.y), int(u1.z), int(u1.w)};
      }
      o[db] = mfma_fp8(a, pk, o[db]);
    }
    // sums of P over the tile's sub-blocks (both halves of the lane pair hold them)
    const f32x16_t sacc = mfma_fp8(ind, pk, f32x16_t{});
    float st[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) st[s] = s < kT ? sacc[s] : 0.0f;
    float ps = st[0];
#pragma unroll
    for (int s = 1; s < kT; ++s) ps += st[s];
    l += ps;
    // V-Smooth add-back, K = 16: k 0-3 mean_hi * S_hi, 4-7 mean_lo * S_hi (lanes of
    // half 0), 8-11 mean_hi * S_lo (half 1), 12-15 zero
    bf16x8_t bs;
    {
      __bf16 hb[4], lb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        hb[s] = __bf16(st[s]);
        lb[s] = __bf16(st[s] - float(hb[s]));
      }
      const __bf16 z = __bf16(0.0f);
      bs = half == 0 ? bf16x8_t{hb[0], hb[1], hb[2], hb[3], hb[0], hb[1], hb[2], hb[3]}
                     : bf16x8_t{lb[0], lb[1], lb[2], lb[3], z, z, z, z};
    }
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = db * 32 + col;
      uint32_t u[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int s = 0; s < kT && s < 4; ++s) u[s] = *reinterpret_cast<const uint32_t*>(mc + s * (kD * 4) + d * 4);
      const uint32_t h01 = (u[0] & 0xFFFFu) | (u[1] << 16);
      const uint32_t h23 = (u[2] & 0xFFFFu) | (u[3] << 16);
      const uint32_t l01 = half == 0 ? ((u[0] >> 16) | (u[1] & 0xFFFF0000u)) : 0u;
      const uint32_t l23 = half == 0 ? ((u[2] >> 16) | (u[3] & 0xFFFF0000u)) : 0u;
      o[db] = mfma32x32x16(as_bf16x8(make_uint4(h01, h23, l01, l23)), bs, o[db]);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, k0s, v0s, m0s, k1s, v1s, m1s);
    if (t + 1 < ntiles) step(t + 1, k1s, v1s, m1s, k0s, v0s, m0s);
  }

  // epilogue: O^T lane layout -> row qr, dims db*32 + (e/4)*8 + half*4 + e%4
  if (qr < n) {
    const float inv = l > 0.0f ? vsc / l : 0.0f;
    uint16_t* dst = out + (size_t(bh) * N + row0 + qr) * kD;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + g * 8 + half * 4;
        uint2 w;
        w.x = uint32_t(f32_to_bf16(o[db][4 * g + 0] * inv)) | (uint32_t(f32_to_bf16(o[db][4 * g + 1] * inv)) << 16);
        w.y = uint32_t(f32_to_bf16(o[db][4 * g + 2] * inv)) | (uint32_t(f32_to_bf16(o[db][4 * g + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(dst + d0) = w;
      }
    }
    if (lse && half == 0)
      lse[size_t(bh) * N + row0 + qr] = l > 0.0f ? (m + fast_log2(l) - kLog2Top) * kLn2 : -__builtin_inff();
  }
}

template <int BK>
hipError_t launch(const Dims& P, const uint8_t* qc, const float* qs, const uint8_t* kc, const float* ks,
                  const uint8_t* vc, const float* vs, const uint32_t* vm, const int32_t* idx, const float* w,
                  const int32_t* cnt, void* out, float* lse, hipStream_t s) {
  // gathered operands of one head: K codes, V codes (padded to whole sub-blocks) and
  // the scaled V-Smooth means
  const size_t head_bytes = size_t(P.N) * kD + size_t(P.nkb) * BK * kD + size_t(P.nkb) * kD * 4;
  const int head_major = size_t(kXcds) * head_bytes > kMallBytes;
  hipLaunchKernelGGL((attn_fwd_fp8<BK>), dim3(P.B * P.H * P.nqb), dim3(256), 0, s, P, qc, qs, kc, ks, vc, vs, vm, idx,
                     w, cnt, static_cast<uint16_t*>(out), lse, head_major);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_fp8(const Dims& P, const uint8_t* qc, const float* qs, const uint8_t* kc, const float* ks,
                               const uint8_t* vc, const float* vs, const uint32_t* vm, const int32_t* idx,
                               const float* w, const int32_t* cnt, void* out, float* lse, hipStream_t s) {
  switch (P.Bk) {
    case 16: return launch<16>(P, qc, qs, kc, ks, vc, vs, vm, idx, w, cnt, out, lse, s);
    case 32: return launch<32>(P, qc, qs, kc, ks, vc, vs, vm, idx, w, cnt, out, lse, s);
    case 64: return launch<64>(P, qc, qs, kc, ks, vc, vs, vm, idx, w, cnt, out, lse, s);
    default: return launch<128>(P, qc, qs, kc, ks, vc, vs, vm, idx, w, cnt, out, lse, s);
  }
}

}  // namespace ab
