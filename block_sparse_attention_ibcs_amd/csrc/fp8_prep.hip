// FP8 operands of the FP8 attention variant (VC-Attention page, iitak.ru news on
// MiniMax-H3: 8-bit attention products; V-Smooth subtracts a per-block mean from
// the values and quantises only the residual).
//
// OCP E4M3 codes with one fp32 scale per block, the block's largest magnitude
// mapping to 448: inv = 448 / amax (correctly rounded), code = E4M3(x * inv) with
// round-to-nearest-even (v_cvt_pk_fp8_f32, no saturation needed: |x * inv| stays
// below 464), scale = amax / 448. Q: one scale per query block; K: one per key
// sub-block; V-Smooth: the mean of each key sub-block (fp32 sum in ascending key
// order, one division, rounded to bf16) is subtracted and the residual quantised
// with one scale per head. The residual codes of a sub-block are stored for the
// attention kernel's matrix-core operand: [half h][dim][k_block/2], key t at half
// (t >> 2) & 1, position (t >> 3) * 4 + (t & 3).
#include "ab_internal.h"

namespace ab {
namespace {

constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ uint32_t fp8_code(float x) {
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false)) & 0xFFu;
}

// max over the workgroup (non-negative values; block of 256 threads)
__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < int(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// One block of rows (a query block or a key sub-block) of one head -> codes + scale.
// blk = (b*H + h) * nblk + i; rows [i*rows_per, min(N, (i+1)*rows_per)).
template <int D>
__global__ __launch_bounds__(256) void quant_rows(int N, int rows_per, int nblk, const uint16_t* __restrict__ x,
                                                  uint8_t* __restrict__ codes, float* __restrict__ scales) {
  __shared__ float red[4];
  constexpr int kMaxChunks = 128 * D / 8 / 256;  // 16-byte chunks per thread for up to 128 rows
  const int blk = blockIdx.x;
  const int i = blk % nblk, bh = blk / nblk;
  const int r0 = i * rows_per, r1 = min(N, r0 + rows_per);
  const size_t base = (size_t(bh) * N + r0) * D;
  const int n8 = (r1 - r0) * D / 8;  // 8-element (16-byte) chunks
  const uint4* src = reinterpret_cast<const uint4*>(x + base);
  uint4 u[kMaxChunks];  // the block is read once and kept in registers
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < kMaxChunks; ++k) {
    const int c = threadIdx.x + k * 256;
    u[k] = c < n8 ? src[c] : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      m = fmaxf(m, fabsf(__uint_as_float(w[e] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(w[e] & 0xFFFF0000u)));
    }
  }
  const float amax = block_max(m, red);
  const float inv = amax > 0.0f ? __fdiv_rn(kE4M3Max, amax) : 0.0f;
  uint2* dst = reinterpret_cast<uint2*>(codes + base);
#pragma unroll
  for (int k = 0; k < kMaxChunks; ++k) {
    const int c = threadIdx.x + k * 256;
    if (c < n8) {
      const uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
      uint32_t out[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = fp8_code(__fmul_rn(__uint_as_float(w[e] << 16), inv));
        const uint32_t hi = fp8_code(__fmul_rn(__uint_as_float(w[e] & 0xFFFF0000u), inv));
        out[e >> 1] |= (lo | (hi << 8)) << (16 * (e & 1));
      }
      dst[c] = make_uint2(out[0], out[1]);
    }
  }
  if (threadIdx.x == 0) scales[blk] = __fdiv_rn(amax, kE4M3Max);
}

// V-Smooth statistics of one key sub-block: per dimension the mean (fp32 sum in
// ascending key order, one division, bf16) and the largest residual magnitude.
// The sub-block is staged in LDS with 16-byte loads; one thread per dimension sums
// its column in key order.
template <int D, int Bk>
__global__ __launch_bounds__(256) void v_stats(int N, int nkb, const uint16_t* __restrict__ v,
                                               uint16_t* __restrict__ vmean, float* __restrict__ ramax) {
  __shared__ __align__(16) uint16_t tile[Bk * D];
  __shared__ float mu[D];
  __shared__ float red[4];
  const int blk = blockIdx.x;
  const int j = blk % nkb, bh = blk / nkb;
  const int r0 = j * Bk, rows = min(N, r0 + Bk) - r0;
  const uint4* src = reinterpret_cast<const uint4*>(v + (size_t(bh) * N + r0) * D);
  uint4* dst = reinterpret_cast<uint4*>(tile);
  for (int c = threadIdx.x; c < rows * D / 8; c += blockDim.x) dst[c] = src[c];
  __syncthreads();
  if (threadIdx.x < D) {
    const int c = threadIdx.x;
    float s = 0.0f;
    for (int r = 0; r < rows; ++r) s = __fadd_rn(s, bf16_to_f32(tile[r * D + c]));
    const uint16_t mb = f32_to_bf16(__fdiv_rn(s, float(rows)));
    vmean[size_t(blk) * D + c] = mb;
    mu[c] = bf16_to_f32(mb);
  }
  __syncthreads();
  float m = 0.0f;
  for (int e = threadIdx.x; e < rows * D; e += blockDim.x)
    m = fmaxf(m, fabsf(__fsub_rn(bf16_to_f32(tile[e]), mu[e % D])));
  const float bm = block_max(m, red);
  if (threadIdx.x == 0) ramax[blk] = bm;
}

// Per head: the residual scale from the sub-blocks' largest residuals.
__global__ __launch_bounds__(256) void v_scale(int nkb, const float* __restrict__ ramax, float* __restrict__ vscale,
                                               float* __restrict__ hamax) {
  __shared__ float red[4];
  const int bh = blockIdx.x;
  float m = 0.0f;
  for (int j = threadIdx.x; j < nkb; j += blockDim.x) m = fmaxf(m, ramax[size_t(bh) * nkb + j]);
  const float a = block_max(m, red);
  if (threadIdx.x == 0) {
    vscale[bh] = __fdiv_rn(a, kE4M3Max);
    hamax[bh] = a;
  }
}

// Residual codes of one sub-block in the operand layout, and the sub-block mean
// divided by the head's residual scale (1 when the scale is 0) as a bf16 pair
// (hi | lo << 16, hi + lo the fp32 quotient to about 2^-16). The sub-block is
// staged in LDS; thread -> (group g of 4 keys, half h2, dimension d), dimension fastest.
template <int D, int Bk>
__global__ __launch_bounds__(256) void v_codes(int N, int nkb, const uint16_t* __restrict__ v,
                                               const uint16_t* __restrict__ vmean, const float* __restrict__ vscale,
                                               const float* __restrict__ hamax, uint8_t* __restrict__ vcode,
                                               uint32_t* __restrict__ vms) {
  __shared__ __align__(16) uint16_t tile[Bk * D];
  const int blk = blockIdx.x;
  const int j = blk % nkb, bh = blk / nkb;
  const int r0 = j * Bk, rows = min(N, r0 + Bk) - r0;
  const uint4* src = reinterpret_cast<const uint4*>(v + (size_t(bh) * N + r0) * D);
  uint4* dst = reinterpret_cast<uint4*>(tile);
  for (int c = threadIdx.x; c < rows * D / 8; c += blockDim.x) dst[c] = src[c];
  const float amax = hamax[bh];
  const float inv = amax > 0.0f ? __fdiv_rn(kE4M3Max, amax) : 0.0f;
  const float vs = vscale[bh] > 0.0f ? vscale[bh] : 1.0f;
  const uint16_t* vm = vmean + size_t(blk) * D;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const float q = __fdiv_rn(bf16_to_f32(vm[d]), vs);
    const uint16_t hi = f32_to_bf16(q);
    const uint16_t lo = f32_to_bf16(__fsub_rn(q, bf16_to_f32(hi)));
    vms[size_t(blk) * D + d] = uint32_t(hi) | (uint32_t(lo) << 16);
  }
  __syncthreads();
  constexpr int groups = Bk / 8;  // 4-key groups per half
  constexpr int total = groups * 2 * D;
  uint8_t* out = vcode + size_t(blk) * D * Bk;
  for (int p = threadIdx.x; p < total; p += blockDim.x) {
    const int d = p % D, h2 = (p / D) % 2, g = p / (2 * D);
    const float mu = bf16_to_f32(vm[d]);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = g * 8 + h2 * 4 + e;  // key of the sub-block
      uint32_t code = 0;
      if (t < rows) code = fp8_code(__fmul_rn(__fsub_rn(bf16_to_f32(tile[t * D + d]), mu), inv));
      word |= code << (8 * e);
    }
    *reinterpret_cast<uint32_t*>(out + (size_t(h2) * D + d) * (Bk / 2) + g * 4) = word;
  }
}

}  // namespace

size_t fp8_ws_bytes(const Dims& P) { return size_t(P.B) * P.H * (size_t(P.nkb) + 1) * sizeof(float); }

namespace {

template <int D, int Bk>
void launch_v(const Dims& P, const uint16_t* V, uint16_t* vmean, float* vscale, uint8_t* vcode, uint32_t* vms,
              float* ramax, float* hamax, hipStream_t s) {
  const int heads = P.B * P.H;
  hipLaunchKernelGGL((v_stats<D, Bk>), dim3(heads * P.nkb), dim3(256), 0, s, P.N, P.nkb, V, vmean, ramax);
  hipLaunchKernelGGL(v_scale, dim3(heads), dim3(256), 0, s, P.nkb, ramax, vscale, hamax);
  hipLaunchKernelGGL((v_codes<D, Bk>), dim3(heads * P.nkb), dim3(256), 0, s, P.N, P.nkb, V, vmean, vscale, hamax,
                     vcode, vms);
}

template <int D>
void launch_v_d(const Dims& P, const uint16_t* V, uint16_t* vmean, float* vscale, uint8_t* vcode, uint32_t* vms,
                float* ramax, float* hamax, hipStream_t s) {
  switch (P.Bk) {
    case 16: launch_v<D, 16>(P, V, vmean, vscale, vcode, vms, ramax, hamax, s); break;
    case 32: launch_v<D, 32>(P, V, vmean, vscale, vcode, vms, ramax, hamax, s); break;
    case 64: launch_v<D, 64>(P, V, vmean, vscale, vcode, vms, ramax, hamax, s); break;
    default: launch_v<D, 128>(P, V, vmean, vscale, vcode, vms, ramax, hamax, s); break;
  }
}

}  // namespace

hipError_t launch_fp8_prepare(const Dims& P, const void* q, const void* k, const void* v, uint8_t* qcode,
                              float* qscale, uint8_t* kcode, float* kscale, uint8_t* vcode, uint16_t* vmean,
                              float* vscale, uint32_t* vms, void* ws, hipStream_t s) {
  const int heads = P.B * P.H;
  auto Q = static_cast<const uint16_t*>(q);
  auto K = static_cast<const uint16_t*>(k);
  auto V = static_cast<const uint16_t*>(v);
  float* ramax = static_cast<float*>(ws);
  float* hamax = ramax + size_t(heads) * P.nkb;
  if (P.d == 128) {
    hipLaunchKernelGGL(quant_rows<128>, dim3(heads * P.nqb), dim3(256), 0, s, P.N, P.Bq, P.nqb, Q, qcode, qscale);
    hipLaunchKernelGGL(quant_rows<128>, dim3(heads * P.nkb), dim3(256), 0, s, P.N, P.Bk, P.nkb, K, kcode, kscale);
    launch_v_d<128>(P, V, vmean, vscale, vcode, vms, ramax, hamax, s);
  } else {
    hipLaunchKernelGGL(quant_rows<64>, dim3(heads * P.nqb), dim3(256), 0, s, P.N, P.Bq, P.nqb, Q, qcode, qscale);
    hipLaunchKernelGGL(quant_rows<64>, dim3(heads * P.nkb), dim3(256), 0, s, P.N, P.Bk, P.nkb, K, kcode, kscale);
    launch_v_d<64>(P, V, vmean, vscale, vcode, vms, ramax, hamax, s);
  }
  return hipGetLastError();
}

}  // namespace ab
