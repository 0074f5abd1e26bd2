/*
 * ab_attn.h - C ABI of the MI355X (gfx950) block-sparse attention library.
 *
 * The library implements the three stages of AB-Attention as described in the
 * AB-Attention abstract (paperdot search page, query "Xing Ma"):
 *
 *   ab_score     IBCS sentence: per-query-block k-means of the queries (tokens
 *                stay in place) and a block-importance estimate for every
 *                (query block, key sub-block) pair.
 *   ab_sample    SIP sentence: sample key sub-blocks in proportion to the
 *                estimates and weight each kept block by the inverse of its
 *                inclusion probability.
 *   ab_attn_fwd  kernel sentence + problem sentence: exact attention restricted
 *                to the kept sub-blocks, gathering sub-blocks smaller than a
 *                matrix-core tile into full tiles, with the inverse-probability
 *                weights applied to numerator and denominator of the softmax.
 *
 * Conventions shared by every entry point:
 *
 * - Tensors. q, k, v and out are contiguous [B, H, N, d] row-major arrays in
 *   the descriptor's dtype, with token n = (t*Hg + y)*W + x of the video latent
 *   (raster order, never permuted). Query block i covers rows
 *   [i*q_block, min(N, (i+1)*q_block)); key sub-block j covers keys
 *   [j*k_block, min(N, (j+1)*k_block)). NQB = ceil(N/q_block),
 *   NKB = ceil(N/k_block).
 * - Memory. Every tensor pointer is a DEVICE pointer owned by the caller. The
 *   library allocates no device memory and keeps no state besides a
 *   thread-local error string; scratch space is the caller's workspace.
 * - Streams. `stream` is a hipStream_t (NULL = the default stream). Calls only
 *   enqueue work and return; inputs and outputs must stay alive until the
 *   stream has drained. Outputs are deterministic run to run (no floating-point
 *   atomics).
 * - Errors. Every call validates its arguments on the host before enqueuing
 *   anything and returns 0 or one of the negative AB_ERR_* codes below;
 *   ab_last_error() then holds a thread-local description. Nothing aborts.
 */
#ifndef AB_ATTN_H
#define AB_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AB_ABI_VERSION 1

/* Return codes. */
#define AB_OK 0
#define AB_ERR_NULL (-1)      /* a required pointer is NULL */
#define AB_ERR_SHAPE (-2)     /* B, H, N < 1, d not in {64, 128}, or sizes overflow (one head of K
                                 or V must take less than 2^31 bytes) */
#define AB_ERR_PARAM (-3)     /* q_block, k_block, n_clusters or kmeans_iters out of range */
#define AB_ERR_DENSITY (-4)   /* density not in (0, 1] (NaN included) */
#define AB_ERR_DTYPE (-5)     /* dtype is not AB_BF16 or AB_F32 */
#define AB_ERR_WORKSPACE (-6) /* workspace smaller than ab_score_workspace_size() */
#define AB_ERR_HIP (-7)       /* a HIP runtime call or kernel launch failed */
#define AB_ERR_DEVICE (-8)    /* the current device is not gfx950 */

/* Element types of q, k, v and out. */
#define AB_BF16 0
#define AB_F32 1

/* Problem descriptor shared by all calls. */
typedef struct ab_desc {
  int32_t B, H, N, d;   /* batch, heads, tokens, head dim (d in {64, 128}) */
  int32_t dtype;        /* AB_BF16 or AB_F32 */
  int32_t q_block;      /* query block rows Bq, 64 or 128 */
  int32_t k_block;      /* key sub-block Bk, one of 16, 32, 64, 128 */
  int32_t n_clusters;   /* C, 1 <= C <= q_block; a block with n_i < C uses n_i */
  int32_t kmeans_iters; /* T, 1 <= T <= 64: Lloyd iterations per query block */
  float scale;          /* softmax scale; <= 0 means 1/sqrt(d) */
} ab_desc;

/* Library version of this header (AB_ABI_VERSION). */
int32_t ab_abi_version(void);

/* Static text for a return code. */
const char* ab_status_str(int32_t code);

/* Thread-local description of the last failure on this thread ("" if none). */
const char* ab_last_error(void);

/*
 * Bytes of device workspace ab_score needs for this descriptor, or 0 when the
 * descriptor is invalid (ab_last_error says why). Covers the k-means
 * centroids (fp32 and bf16 copies), cluster sizes, the per (query block,
 * key sub-block, cluster) log-sum-exp table and the per-split partial
 * log-sum-exps. The workspace must be 256-byte aligned.
 */
size_t ab_score_workspace_size(const ab_desc* desc);

/*
 * IBCS block-importance estimates (AB-Attention abstract, IBCS sentence).
 *
 * For each query block (b, h, i): k-means with C clusters and T iterations on
 * the block's queries (exact-operation fp32: a query is compared with centroid
 * mu through |mu|^2 - 2 x.mu, i.e. |mu|^2 then one fused multiply-add of
 * x_k * (-2 mu_k) per dimension in ascending order, |mu|^2 being rounded
 * products summed by a halving tree within each group of 64 dimensions and the
 * groups added in order; ties to the lowest cluster; members summed in ascending
 * row order, one correctly rounded division; strided initial centroids; empty
 * clusters keep their centroid with size 0), then
 *   scores[b,h,i,j] = sum_c (n_c/n_i) * exp(l_cj - L_c),
 *   l_cj = log sum_{k in sub-block j} exp(scale * mu_c . k_k),  L_c = log sum_j exp(l_cj),
 * where for bf16 inputs the product is taken with bf16(fl32(c2 * mu_c)),
 * c2 = fl32(scale * log2 e), as a base-2 logit (one rounding of the scaled
 * centroid). Each score row sums to 1 (up to rounding).
 *
 * q, k:    device [B, H, N, d], dtype of desc.
 * scores:  device fp32 [B, H, NQB, NKB], written in full.
 * ws:      device workspace of ws_bytes >= ab_score_workspace_size(desc),
 *          256-byte aligned; its contents are scratch.
 */
int32_t ab_score(const ab_desc* desc, const void* q, const void* k, float* scores,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): ab_score with no
 * workspace argument. Its scratch is a fixed device array inside the library,
 * AB_SCORE_NOALLOC_SCRATCH_BYTES (256 MiB) per GPU, held from the library's first
 * kernel launch on that GPU until the process ends; its address is looked up once
 * per device. It calls no allocating routine.
 *
 * Heads run in chunks that fit the scratch, each with the key splits the whole
 * problem would use in ab_score, so the scores are bit-identical to ab_score's.
 * A descriptor whose single head needs more scratch than the array holds is
 * rejected with AB_ERR_WORKSPACE before anything is enqueued (ab_last_error gives
 * both sizes). Every call on one GPU shares that GPU's array and leaves its last
 * contents there; calls that overlap on one GPU (different streams or threads)
 * race on it and must be ordered by the caller. Arguments and results are those
 * of ab_score.
 */
#define AB_SCORE_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int32_t ab_score_noalloc(const ab_desc* desc, const void* q, const void* k, float* scores, void* stream);

/*
 * The k-means stage of ab_score on its own, with every intermediate exposed
 * (the clustering of the IBCS sentence).
 *
 * centroids: device fp32 [B, H, NQB, C, d] (clusters c >= n_i are zero);
 * sizes:     device int32 [B, H, NQB, C];
 * assign:    device uint8 [B, H, N], cluster of each query after the last
 *            assignment step. Any of the three may be NULL (not written), but
 *            not all of them.
 */
int32_t ab_score_debug(const ab_desc* desc, const void* q, float* centroids, int32_t* sizes,
                       uint8_t* assign, void* stream);

/*
 * SIP sampling (AB-Attention abstract, SIP sentence), integer-exact given the
 * fp32 scores.
 *
 * Per row (b, h, i): w_j = max(1, floor(s_j * 2^24)) (NaN or s <= 0 -> 1,
 * s >= 1 -> 2^24); budget K = clamp(floor(density*NKB + 0.5), 1, NKB) in fp64;
 * thresholds t_j in [1, 2^24] by integer water-filling (inclusion probability
 * t_j/2^24 proportional to w_j, capped at 1, summing to K up to floors);
 * u_j = word (j mod 4) of Philox4x32-10(key = (seed mod 2^32, seed >> 32),
 * counter = (floor(j/4), i, h, b)) >> 8; block j is kept iff u_j < t_j, with
 * weight fp32(2^24)/fp32(t_j).
 *
 * scores:    device fp32 [B, H, NQB, NKB].
 * idx:       device int32 [B, H, NQB, NKB]; the first counts[row] entries of a
 *            row hold the kept sub-block indices in ascending order; the rest
 *            is left untouched.
 * weights:   device fp32 [B, H, NQB, NKB], aligned with idx.
 * counts:    device int32 [B, H, NQB].
 * mask_bits: device uint32 [B, H, NQB, ceil(NKB/32)], bit j%32 of word j/32
 *            set iff block j is kept; may be NULL.
 */
int32_t ab_sample(const ab_desc* desc, const float* scores, double density, uint64_t seed,
                  int32_t* idx, float* weights, int32_t* counts, uint32_t* mask_bits,
                  void* stream);

/*
 * Fixed-size (systematic) sampling with the same inclusion probabilities as
 * ab_sample: the other standard design for sampling with known inclusion
 * probabilities (AB-Attention abstract, SIP sentence, which fixes no design).
 *
 * Per row (b, h, i): thresholds t_j exactly as ab_sample; one 24-bit uniform
 * U = word 0 of Philox4x32-10(key = (seed mod 2^32, seed >> 32), counter =
 * (2^32 - 1, i, h, b)) >> 8; with C_j = t_0 + ... + t_{j-1}, block j is kept
 * iff [C_j, C_j + t_j) holds a point U + m*2^24 (m >= 0), so it is kept with
 * probability t_j/2^24 exactly and a row keeps floor(T/2^24) or one more block
 * (T = sum of t_j, about K*2^24); weight fp32(2^24)/fp32(t_j). Outputs as for
 * ab_sample. Rows of more than 16384 key sub-blocks are rejected with
 * AB_ERR_SHAPE.
 */
int32_t ab_sample_systematic(const ab_desc* desc, const float* scores, double density, uint64_t seed,
                             int32_t* idx, float* weights, int32_t* counts, uint32_t* mask_bits,
                             void* stream);

/*
 * Top-K truncation of the same score rows: the deterministic selection the SIP
 * sentence of the AB-Attention abstract sets its sampler against (kept for
 * estimator comparisons; the method itself samples with ab_sample).
 *
 * Per row (b, h, i): the same quantised scores w_j and budget K as ab_sample;
 * the K sub-blocks with the largest w_j are kept, the lower index first among
 * equal w_j, each with weight 1. Outputs as for ab_sample, with counts[row] = K.
 * Rows of more than 16384 key sub-blocks are rejected with AB_ERR_SHAPE.
 */
int32_t ab_sample_topk(const ab_desc* desc, const float* scores, double density, int32_t* idx,
                       float* weights, int32_t* counts, uint32_t* mask_bits, void* stream);

/*
 * INTRA relay patterns as kept-sub-block lists for ab_attn_fwd (INTRA page,
 * paperdot search page, query "Wenbo Lu": static sparse attention over
 * computational query sets, Scatter relay groups drawing on every local
 * neighbourhood and Gather reconnecting them, under a partition model).
 *
 * The sequence is cut into neighbourhoods of L = partition_tokens tokens (0 selects
 * q_block * ceil(sqrt(NQB))); query block i sits at offset o_i = (i * q_block) mod L
 * of neighbourhood (i * q_block) / L.
 *   AB_INTRA_SCATTER: the key sub-blocks at offsets [o_i, o_i + q_block) of every
 *                     neighbourhood (those holding real tokens);
 *   AB_INTRA_GATHER:  the key sub-blocks of query block i's own neighbourhood.
 * Every kept sub-block gets weight 1 (exact attention over the pattern). The two
 * layers in sequence connect every query token to every key token when L divides N.
 *
 * idx:      device int32 [B, H, NQB, NKB]: kept sub-blocks in ascending order, the
 *           first counts[b,h,i] entries of each row written (the rest untouched).
 * weights:  device fp32 [B, H, NQB, NKB]: 1.0 for the written entries.
 * counts:   device int32 [B, H, NQB].
 * row_order: NULL, or device int32 [B * H * NQB] receiving a processing order for
 *           ab_attn_fwd_ordered: Scatter rows ((b*H + h)*NQB + i) grouped by their
 *           offset (rows of one offset share one list, so the workgroups resident
 *           together read the same keys); Gather rows in their natural order.
 * Errors: AB_ERR_PARAM for another layer value or an L that is not a multiple of
 * q_block in [q_block, 2^30]; AB_ERR_NULL for NULL lists.
 */
#define AB_INTRA_SCATTER 0
#define AB_INTRA_GATHER 1
int32_t ab_intra_lists(const ab_desc* desc, int32_t layer, int32_t partition_tokens, int32_t* idx,
                       float* weights, int32_t* counts, int32_t* row_order, void* stream);

/*
 * ab_attn_fwd with the query-block rows taken in a given order: the same outputs
 * for every order (each row's computation is unchanged); only which rows run side
 * by side, and so share caches, changes. For callers whose lists repeat across
 * rows that are not neighbours (for instance INTRA Scatter, see ab_intra_lists).
 *
 * row_order: device int32 [B * H * NQB]: entry w is the row ((b*H + h)*NQB + i)
 *            that the w-th workgroup computes (after the XCD-aware remapping of
 *            workgroup ids). A permutation gives exactly ab_attn_fwd's result;
 *            entries outside [0, B*H*NQB) are skipped, a row not listed is not
 *            written and a row listed twice is written twice with the same values.
 * Other arguments and errors as ab_attn_fwd; AB_ERR_NULL when row_order is NULL.
 */
int32_t ab_attn_fwd_ordered(const ab_desc* desc, const void* q, const void* k, const void* v,
                            const int32_t* idx, const float* weights, const int32_t* counts,
                            const int32_t* row_order, void* out, float* lse, void* stream);

/*
 * Weighted block-sparse attention forward (AB-Attention abstract, problem,
 * SIP and kernel sentences).
 *
 * For every query row r of block i of (b, h), over the kept sub-blocks j of
 * row (b, h, i) with weights w_j:
 *   den_r = sum_j w_j sum_{k in j} exp(scale*q_r.k_k - m_r),
 *   out_r = (sum_j w_j sum_{k in j} exp(scale*q_r.k_k - m_r) v_k) / den_r,
 *   lse_r = m_r + log(den_r);
 * a block that keeps nothing gives out = 0 and lse = -inf. Sub-blocks smaller
 * than the kernel's key tile are packed together into one tile.
 *
 * q, k, v: device [B, H, N, d], dtype of desc.
 * idx, weights, counts: as written by ab_sample (indices must be ascending,
 *            unique and in [0, NKB); counts in [0, NKB]).
 * out:     device [B, H, N, d], dtype of desc.
 * lse:     device fp32 [B, H, N] natural-log log-sum-exp; may be NULL.
 * The outputs do not depend on the order in which query blocks are processed. Each
 * XCD takes one contiguous range of (b, h, i) rows, unless eight heads' K and V
 * exceed 256 MiB (the Infinity Cache; N > 65536 at d = 128): then all XCDs work on
 * the same head at a time, each on its own slice of its query blocks.
 */
int32_t ab_attn_fwd(const ab_desc* desc, const void* q, const void* k, const void* v,
                    const int32_t* idx, const float* weights, const int32_t* counts,
                    void* out, float* lse, void* stream);

/*
 * ---- FP8 variant (VC-Attention page, iitak.ru news on MiniMax-H3: the attention
 * products in 8-bit floating point, V-Smooth and ExpCast-FP8) ----
 *
 * Bytes of device workspace ab_fp8_prepare needs (per-sub-block and per-head
 * residual maxima), or 0 when the descriptor is invalid.
 */
size_t ab_fp8_workspace_size(const ab_desc* desc);

/*
 * FP8 operands of one layer for ab_attn_fwd_fp8. Codes are OCP E4M3 (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits, largest finite 448), rounded to
 * nearest even from fp32, with one fp32 scale per block: the block's largest
 * magnitude amax maps to 448, inv = 448/amax and scale = amax/448 both correctly
 * rounded, code = E4M3(x * inv); an all-zero block has scale 0 and codes 0.
 *
 * desc:     dtype must be AB_BF16 (else AB_ERR_DTYPE).
 * q, k, v:  device bf16 [B, H, N, d].
 * qcode:    device uint8 [B, H, N, d], one scale per query block -> qscale fp32 [B, H, NQB].
 * kcode:    device uint8 [B, H, N, d], one scale per key sub-block -> kscale fp32 [B, H, NKB].
 * vmean:    device bf16 [B, H, NKB, d]: V-Smooth mean of each key sub-block (fp32 sum
 *           of its real keys in ascending order, one division, rounded to bf16).
 * vcode:    device uint8 [B, H, NKB, 2, d, k_block/2]: residual v - vmean of each key
 *           quantised with one scale per head (vscale fp32 [B, H]); key t of a
 *           sub-block sits at [(t >> 2) & 1][dim][(t >> 3) * 4 + (t & 3)] (the
 *           operand order of the attention kernel); keys at or past N hold 0.
 * vmean_scaled: device uint32 [B, H, NKB, d]: vmean / vscale (1 when vscale is 0)
 *           as two bf16 halves, low 16 bits hi = bf16(x), high 16 bits lo = bf16(x - hi).
 * ws:       device workspace of ws_bytes >= ab_fp8_workspace_size(desc), 16-byte aligned.
 * q, k, v, qcode, kcode, vcode, vmean_scaled and ws must be 16-byte aligned.
 */
int32_t ab_fp8_prepare(const ab_desc* desc, const void* q, const void* k, const void* v, uint8_t* qcode,
                       float* qscale, uint8_t* kcode, float* kscale, uint8_t* vcode, uint16_t* vmean,
                       float* vscale, uint32_t* vmean_scaled, void* ws, size_t ws_bytes, void* stream);

/*
 * FP8 weighted block-sparse attention (VC-Attention page: 8-bit products,
 * V-Smooth add-back, ExpCast-FP8 probabilities) on the kept sub-blocks of
 * ab_sample, from the operands of ab_fp8_prepare. Head dim 128 and q_block 128
 * only (else AB_ERR_PARAM); k_block any of 16, 32, 64, 128.
 *
 * The kept sub-blocks of each query block are laid end to end and walked in
 * 64-slot tiles; per tile and query row (log2 units):
 *   x = qscale_i * kscale_j * scale * log2(e) * (qcode . kcode) + log2(w_j),
 *   m <- max(m, max_tile x)  (O and l rescaled by 2^(m_old - m) when m moves),
 *   p = E4M3 value of code = clamp(round_half_even(8 (x - m) + 126), 0, 126),
 *   l += sum p,  O += vscale * sum p decode(vcode) + sum_t (sum of p over sub-block t) vmean_t;
 * out = O / l (0 for an empty list), lse = (m + log2 l - 8.75) ln 2 (-inf if empty).
 * idx, weights, counts: as written by ab_sample. out: device bf16 [B, H, N, 128];
 * lse: device fp32 [B, H, N] or NULL. qcode, kcode, vcode, vmean_scaled and out
 * must be 16-byte aligned.
 */
int32_t ab_attn_fwd_fp8(const ab_desc* desc, const uint8_t* qcode, const float* qscale, const uint8_t* kcode,
                        const float* kscale, const uint8_t* vcode, const float* vscale, const uint32_t* vmean_scaled,
                        const int32_t* idx, const float* weights, const int32_t* counts, void* out, float* lse,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AB_ATTN_H */
