// C ABI of libabattn: argument validation, workspace carve-up and launches.
// Every check runs on the host before anything is enqueued; failures return a
// negative AB_ERR_* code and leave a thread-local message (nothing aborts).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "ab_internal.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(AB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxN = 1 << 24;
constexpr int kMaxNkb = 65536;
constexpr int kMaxHeads = 65535;

// Immutable per-device fact: is it gfx950? 0 = unknown, 1 = yes, 2 = no.
std::atomic<int> g_arch_ok[64];

int32_t check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(AB_ERR_DEVICE, "device index %d out of range", dev);
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
    if (st == 2) return fail(AB_ERR_DEVICE, "device %d is %s, the library is built for gfx950", dev, prop.gcnArchName);
  }
  if (st == 2) return fail(AB_ERR_DEVICE, "device %d is not gfx950", dev);
  return AB_OK;
}

int32_t make_dims(const ab_desc* d, ab::Dims* P) {
  if (!d) return fail(AB_ERR_NULL, "desc is NULL");
  if (d->B < 1 || d->H < 1 || d->N < 1) return fail(AB_ERR_SHAPE, "B, H and N must be >= 1 (got %d, %d, %d)", d->B, d->H, d->N);
  if (d->d != 64 && d->d != 128) return fail(AB_ERR_SHAPE, "head dim must be 64 or 128 (got %d)", d->d);
  if (d->N > kMaxN) return fail(AB_ERR_SHAPE, "N = %d exceeds the supported maximum %d", d->N, kMaxN);
  if (int64_t(d->B) * d->H > kMaxHeads) return fail(AB_ERR_SHAPE, "B*H = %lld exceeds %d", (long long)d->B * d->H, kMaxHeads);
  if (d->dtype != AB_BF16 && d->dtype != AB_F32) return fail(AB_ERR_DTYPE, "dtype must be AB_BF16 or AB_F32 (got %d)", d->dtype);
  if (d->q_block != 64 && d->q_block != 128) return fail(AB_ERR_PARAM, "q_block must be 64 or 128 (got %d)", d->q_block);
  if (d->k_block != 16 && d->k_block != 32 && d->k_block != 64 && d->k_block != 128)
    return fail(AB_ERR_PARAM, "k_block must be 16, 32, 64 or 128 (got %d)", d->k_block);
  if (d->n_clusters < 1 || d->n_clusters > d->q_block)
    return fail(AB_ERR_PARAM, "n_clusters must be in [1, q_block] (got %d)", d->n_clusters);
  if (d->kmeans_iters < 1 || d->kmeans_iters > 64) return fail(AB_ERR_PARAM, "kmeans_iters must be in [1, 64] (got %d)", d->kmeans_iters);
  ab::Dims& D = *P;
  D.B = d->B;
  D.H = d->H;
  D.N = d->N;
  D.d = d->d;
  D.Bq = d->q_block;
  D.Bk = d->k_block;
  D.C = d->n_clusters;
  D.T = d->kmeans_iters;
  D.nqb = ab::ceil_div(D.N, D.Bq);
  D.nkb = ab::ceil_div(D.N, D.Bk);
  D.mrows = D.nqb * D.C;
  D.bf16 = d->dtype == AB_BF16;
  D.scale = (d->scale > 0.0f && std::isfinite(d->scale)) ? d->scale : float(1.0 / std::sqrt(double(D.d)));
  if (D.nkb > kMaxNkb) return fail(AB_ERR_SHAPE, "N/k_block = %d sub-blocks exceeds %d", D.nkb, kMaxNkb);
  // Kernels address one head's K or V with 32-bit buffer offsets and use 2^31 as
  // an always-out-of-range offset, so one head must stay below 2 GiB.
  const int64_t head_bytes = int64_t(D.N) * D.d * (D.bf16 ? 2 : 4);
  if (head_bytes >= (int64_t(1) << 31))
    return fail(AB_ERR_SHAPE, "one head of K/V takes %lld bytes, the limit is 2^31 - 1", (long long)head_bytes);
  return AB_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// K = clamp(floor(density * NKB + 0.5), 1, NKB), two separately rounded fp64 operations
int budget_blocks(double density, int nkb) {
  volatile double prod = density * double(nkb);
  const double t = prod + 0.5;
  long long K = static_cast<long long>(std::floor(t));
  if (K < 1) K = 1;
  if (K > nkb) K = nkb;
  return int(K);
}

// Scratch of the allocation-free scorer: a fixed device array in the library's code
// object (each GPU the library runs on holds its own copy until the process ends).
// Host code never passes this name to a kernel or a copy: it is a host-side stand-in;
// the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = AB_SCORE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once resolved

// Device address of this device's scratch array, resolved on the first call on the
// device with that device current.
int32_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(AB_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(AB_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AB_OK;
}

}  // namespace

extern "C" {

int32_t ab_abi_version(void) { return AB_ABI_VERSION; }

const char* ab_status_str(int32_t code) {
  switch (code) {
    case AB_OK: return "ok";
    case AB_ERR_NULL: return "null pointer";
    case AB_ERR_SHAPE: return "bad shape";
    case AB_ERR_PARAM: return "bad block, cluster or iteration parameter";
    case AB_ERR_DENSITY: return "density not in (0, 1]";
    case AB_ERR_DTYPE: return "bad dtype";
    case AB_ERR_WORKSPACE: return "workspace too small or misaligned";
    case AB_ERR_HIP: return "HIP error";
    case AB_ERR_DEVICE: return "unsupported device";
    default: return "unknown status";
  }
}

const char* ab_last_error(void) { return g_err; }

size_t ab_score_workspace_size(const ab_desc* desc) {
  ab::Dims P;
  if (make_dims(desc, &P) != AB_OK) return 0;
  return ab::score_ws_layout(P, 256).total;
}

int32_t ab_score(const ab_desc* desc, const void* q, const void* k, float* scores, void* ws, size_t ws_bytes,
                 void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!q || !k || !scores || !ws) return fail(AB_ERR_NULL, "q, k, scores and ws must be non-NULL");
  const ab::ScoreWs L = ab::score_ws_layout(P, 256);
  if (ws_bytes < L.total) return fail(AB_ERR_WORKSPACE, "workspace of %zu bytes < required %zu", ws_bytes, L.total);
  if (!aligned(ws, 256)) return fail(AB_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scores, 4)) return fail(AB_ERR_SHAPE, "q and k must be 16-byte aligned");
  if ((rc = check_device())) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* w = static_cast<unsigned char*>(ws);
  float* cf = reinterpret_cast<float*>(w + L.centroids_f32);
  uint16_t* cb = reinterpret_cast<uint16_t*>(w + L.centroids_bf16);
  int32_t* sz = reinterpret_cast<int32_t*>(w + L.sizes);
  float* ell = reinterpret_cast<float*>(w + L.ell);
  float* lpart = reinterpret_cast<float*>(w + L.lpart);
  hipError_t e = ab::launch_kmeans(P, q, cf, P.bf16 ? cb : nullptr, sz, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "k-means launch");
  e = ab::launch_score_lse(P, L, k, P.bf16 ? static_cast<const void*>(cb) : static_cast<const void*>(cf), ell, lpart, s);
  if (e != hipSuccess) return hip_fail(e, "score log-sum-exp launch");
  e = ab::launch_score_assemble(P, L, ell, lpart, sz, scores, s);
  if (e != hipSuccess) return hip_fail(e, "score assembly launch");
  return AB_OK;
}

int32_t ab_score_noalloc(const ab_desc* desc, const void* q, const void* k, float* scores, void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!q || !k || !scores) return fail(AB_ERR_NULL, "q, k and scores must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(scores, 4)) return fail(AB_ERR_SHAPE, "q and k must be 16-byte aligned");
  // Heads are independent through the scorer, so the problem runs in chunks of heads
  // that each fit the scratch array. Every chunk uses the key splits the whole problem
  // would use, so each head's arithmetic, and its result, is the same as in ab_score.
  const ab::ScoreWs full = ab::score_ws_layout(P, 256);
  const int heads = P.B * P.H;
  int per_chunk = 0;
  for (int hc = heads; hc >= 1; hc = hc > 1 ? (hc + 1) / 2 : 0) {
    ab::Dims Pc = P;
    Pc.B = 1;
    Pc.H = hc;
    if (ab::score_ws_layout_split(Pc, full.split_keys).total <= kScratchBytes) {
      per_chunk = hc;
      break;
    }
  }
  if (per_chunk == 0) {
    ab::Dims P1 = P;
    P1.B = 1;
    P1.H = 1;
    return fail(AB_ERR_WORKSPACE, "one head needs %zu bytes of scratch; the allocation-free scorer holds %zu",
                ab::score_ws_layout_split(P1, full.split_keys).total, kScratchBytes);
  }
  if ((rc = check_device())) return rc;
  void* base = nullptr;
  if ((rc = scratch_for_current_device(&base))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t esize = P.bf16 ? 2 : 4;
  const size_t head_elems = size_t(P.N) * P.d;
  const size_t head_scores = size_t(P.nqb) * P.nkb;
  for (int h0 = 0; h0 < heads; h0 += per_chunk) {
    ab::Dims Pc = P;
    Pc.B = 1;
    Pc.H = heads - h0 < per_chunk ? heads - h0 : per_chunk;
    const ab::ScoreWs L = ab::score_ws_layout_split(Pc, full.split_keys);
    unsigned char* w = static_cast<unsigned char*>(base);
    float* cf = reinterpret_cast<float*>(w + L.centroids_f32);
    uint16_t* cb = reinterpret_cast<uint16_t*>(w + L.centroids_bf16);
    int32_t* sz = reinterpret_cast<int32_t*>(w + L.sizes);
    float* ell = reinterpret_cast<float*>(w + L.ell);
    float* lpart = reinterpret_cast<float*>(w + L.lpart);
    const void* qc = static_cast<const unsigned char*>(q) + size_t(h0) * head_elems * esize;
    const void* kc = static_cast<const unsigned char*>(k) + size_t(h0) * head_elems * esize;
    float* sc = scores + size_t(h0) * head_scores;
    hipError_t e = ab::launch_kmeans(Pc, qc, cf, Pc.bf16 ? cb : nullptr, sz, nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "k-means launch");
    e = ab::launch_score_lse(Pc, L, kc, Pc.bf16 ? static_cast<const void*>(cb) : static_cast<const void*>(cf), ell,
                             lpart, s);
    if (e != hipSuccess) return hip_fail(e, "score log-sum-exp launch");
    e = ab::launch_score_assemble(Pc, L, ell, lpart, sz, sc, s);
    if (e != hipSuccess) return hip_fail(e, "score assembly launch");
  }
  return AB_OK;
}

int32_t ab_score_debug(const ab_desc* desc, const void* q, float* centroids, int32_t* sizes, uint8_t* assign,
                       void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!q) return fail(AB_ERR_NULL, "q must be non-NULL");
  if (!centroids && !sizes && !assign) return fail(AB_ERR_NULL, "at least one of centroids, sizes, assign is needed");
  if (!aligned(q, 16)) return fail(AB_ERR_SHAPE, "q must be 16-byte aligned");
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_kmeans(P, q, centroids, nullptr, sizes, assign, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "k-means launch");
  return AB_OK;
}

int32_t ab_sample(const ab_desc* desc, const float* scores, double density, uint64_t seed, int32_t* idx,
                  float* weights, int32_t* counts, uint32_t* mask_bits, void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!scores || !idx || !weights || !counts) return fail(AB_ERR_NULL, "scores, idx, weights and counts must be non-NULL");
  if (!(density > 0.0 && density <= 1.0)) return fail(AB_ERR_DENSITY, "density %g not in (0, 1]", density);
  const int K = budget_blocks(density, P.nkb);
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_sample(P, scores, K, seed, idx, weights, counts, mask_bits,
                                   static_cast<hipStream_t>(stream), false);
  if (e != hipSuccess) return hip_fail(e, "sampler launch");
  return AB_OK;
}

int32_t ab_sample_systematic(const ab_desc* desc, const float* scores, double density, uint64_t seed, int32_t* idx,
                             float* weights, int32_t* counts, uint32_t* mask_bits, void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!scores || !idx || !weights || !counts) return fail(AB_ERR_NULL, "scores, idx, weights and counts must be non-NULL");
  if (!(density > 0.0 && density <= 1.0)) return fail(AB_ERR_DENSITY, "density %g not in (0, 1]", density);
  if (P.nkb > ab::kTopkMaxNkb)
    return fail(AB_ERR_SHAPE, "systematic sampling takes rows of at most %d sub-blocks (got %d)", ab::kTopkMaxNkb, P.nkb);
  const int K = budget_blocks(density, P.nkb);
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_sample(P, scores, K, seed, idx, weights, counts, mask_bits,
                                   static_cast<hipStream_t>(stream), true);
  if (e != hipSuccess) return hip_fail(e, "systematic sampler launch");
  return AB_OK;
}

int32_t ab_sample_topk(const ab_desc* desc, const float* scores, double density, int32_t* idx, float* weights,
                       int32_t* counts, uint32_t* mask_bits, void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!scores || !idx || !weights || !counts) return fail(AB_ERR_NULL, "scores, idx, weights and counts must be non-NULL");
  if (!(density > 0.0 && density <= 1.0)) return fail(AB_ERR_DENSITY, "density %g not in (0, 1]", density);
  if (P.nkb > ab::kTopkMaxNkb)
    return fail(AB_ERR_SHAPE, "top-K truncation takes rows of at most %d sub-blocks (got %d)", ab::kTopkMaxNkb, P.nkb);
  const int K = budget_blocks(density, P.nkb);
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_topk(P, scores, K, idx, weights, counts, mask_bits, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "top-K launch");
  return AB_OK;
}

int32_t ab_intra_lists(const ab_desc* desc, int32_t layer, int32_t partition_tokens, int32_t* idx, float* weights,
                       int32_t* counts, int32_t* row_order, void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (layer != AB_INTRA_SCATTER && layer != AB_INTRA_GATHER)
    return fail(AB_ERR_PARAM, "layer must be AB_INTRA_SCATTER or AB_INTRA_GATHER (got %d)", layer);
  const int L = partition_tokens == 0 ? ab::intra_default_partition(P) : partition_tokens;
  if (L < P.Bq || L % P.Bq != 0 || L > (1 << 30))
    return fail(AB_ERR_PARAM, "partition_tokens must be 0 or a multiple of q_block in [q_block, 2^30] (got %d)",
                partition_tokens);
  if (!idx || !weights || !counts) return fail(AB_ERR_NULL, "idx, weights and counts must be non-NULL");
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_intra_lists(P, layer, L, idx, weights, counts, row_order, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "INTRA list launch");
  return AB_OK;
}

int32_t ab_attn_fwd(const ab_desc* desc, const void* q, const void* k, const void* v, const int32_t* idx,
                    const float* weights, const int32_t* counts, void* out, float* lse, void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!q || !k || !v || !idx || !weights || !counts || !out)
    return fail(AB_ERR_NULL, "q, k, v, idx, weights, counts and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(AB_ERR_SHAPE, "q, k, v and out must be 16-byte aligned");
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_attn_fwd(P, q, k, v, idx, weights, counts, out, lse, nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return AB_OK;
}

int32_t ab_attn_fwd_ordered(const ab_desc* desc, const void* q, const void* k, const void* v, const int32_t* idx,
                            const float* weights, const int32_t* counts, const int32_t* row_order, void* out,
                            float* lse, void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!q || !k || !v || !idx || !weights || !counts || !row_order || !out)
    return fail(AB_ERR_NULL, "q, k, v, idx, weights, counts, row_order and out must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return fail(AB_ERR_SHAPE, "q, k, v and out must be 16-byte aligned");
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_attn_fwd(P, q, k, v, idx, weights, counts, out, lse, row_order,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return AB_OK;
}

size_t ab_fp8_workspace_size(const ab_desc* desc) {
  ab::Dims P;
  if (make_dims(desc, &P) != AB_OK) return 0;
  return ab::fp8_ws_bytes(P);
}

int32_t ab_fp8_prepare(const ab_desc* desc, const void* q, const void* k, const void* v, uint8_t* qcode,
                       float* qscale, uint8_t* kcode, float* kscale, uint8_t* vcode, uint16_t* vmean,
                       float* vscale, uint32_t* vmean_scaled, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!P.bf16) return fail(AB_ERR_DTYPE, "the FP8 variant takes bf16 inputs");
  if (!q || !k || !v || !qcode || !qscale || !kcode || !kscale || !vcode || !vmean || !vscale || !vmean_scaled || !ws)
    return fail(AB_ERR_NULL, "every pointer of ab_fp8_prepare must be non-NULL");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(qcode, 16) || !aligned(kcode, 16) ||
      !aligned(vcode, 16) || !aligned(vmean_scaled, 16) || !aligned(ws, 16))
    return fail(AB_ERR_SHAPE, "q, k, v, qcode, kcode, vcode, vmean_scaled and ws must be 16-byte aligned");
  const size_t need = ab::fp8_ws_bytes(P);
  if (ws_bytes < need) return fail(AB_ERR_WORKSPACE, "workspace of %zu bytes < required %zu", ws_bytes, need);
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_fp8_prepare(P, q, k, v, qcode, qscale, kcode, kscale, vcode, vmean, vscale, vmean_scaled,
                                        ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 prepare launch");
  return AB_OK;
}

int32_t ab_attn_fwd_fp8(const ab_desc* desc, const uint8_t* qcode, const float* qscale, const uint8_t* kcode,
                        const float* kscale, const uint8_t* vcode, const float* vscale, const uint32_t* vmean_scaled,
                        const int32_t* idx, const float* weights, const int32_t* counts, void* out, float* lse,
                        void* stream) {
  g_err[0] = 0;
  ab::Dims P;
  int32_t rc = make_dims(desc, &P);
  if (rc) return rc;
  if (!P.bf16) return fail(AB_ERR_DTYPE, "the FP8 variant takes bf16 inputs and writes bf16 output");
  if (P.d != 128 || P.Bq != 128) return fail(AB_ERR_PARAM, "the FP8 attention takes d = 128 and q_block = 128 (got %d, %d)", P.d, P.Bq);
  if (!qcode || !qscale || !kcode || !kscale || !vcode || !vscale || !vmean_scaled || !idx || !weights || !counts || !out)
    return fail(AB_ERR_NULL, "every pointer of ab_attn_fwd_fp8 except lse must be non-NULL");
  if (!aligned(qcode, 16) || !aligned(kcode, 16) || !aligned(vcode, 16) || !aligned(vmean_scaled, 16) || !aligned(out, 16))
    return fail(AB_ERR_SHAPE, "qcode, kcode, vcode, vmean_scaled and out must be 16-byte aligned");
  if ((rc = check_device())) return rc;
  hipError_t e = ab::launch_attn_fwd_fp8(P, qcode, qscale, kcode, kscale, vcode, vscale, vmean_scaled, idx, weights,
                                         counts, out, lse, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 attention launch");
  return AB_OK;
}

}  // extern "C"
