/* Plain C twin of two oracle steps, for checks over every row of the full-size
 * workloads (the numpy forms in oracle/ibcs.py and oracle/sip.py are the readable
 * ones; this file follows the same specification operation by operation and is
 * pinned to them, and to the same golden values, in tests/test_oracle_native.py).
 *
 * TEST INFRASTRUCTURE ONLY: built as oracle/liboracle_c.so and loaded by
 * oracle/native.py for the tests and the benchmark's CPU baseline; nothing in the
 * library under block_sparse_attention_ibcs_amd uses it.
 *
 * Build: gcc -O2 -std=c99 -fPIC -shared -fopenmp -ffp-contract=off [-mfma] oracle_c.c -lm
 * -ffp-contract=off keeps every multiply and add separately rounded unless fmaf() is
 * written; fmaf() is the correctly rounded fused multiply-add (a hardware instruction
 * with -mfma, glibc's exact routine without).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- IBCS k-means (AB-Attention abstract, IBCS sentence; readings of oracle/ibcs.py) ----
 * |mu|^2: products rounded one by one, summed by the halving tree inside each group of
 * 64 dimensions (absent dimensions 0), group sums added in order. */
static float centroid_sqnorm(const float* mu, int d) {
  float out = 0.0f;
  for (int g = 0; g * 64 < d; ++g) {
    float t[64];
    for (int k = 0; k < 64; ++k) {
      const int dk = g * 64 + k;
      t[k] = dk < d ? mu[dk] * mu[dk] : 0.0f;
    }
    for (int s = 32; s >= 1; s >>= 1)
      for (int k = 0; k < s; ++k) t[k] = t[k] + t[k + s];
    out = g == 0 ? t[0] : out + t[0];
  }
  return out;
}

/* One query block X [n][d]: T Lloyd iterations on C_i = min(C, n) clusters initialised
 * at X[floor(c n / C_i)]; comparison |mu_c|^2 - 2 x.mu_c with one fused multiply-add
 * per dimension in ascending order; ties to the lowest cluster; members summed in
 * ascending row order, one division; an empty cluster keeps its centroid and gets size
 * 0. Outputs mu [C][d] (clusters >= C_i stay 0), sizes [C], assign [n]. */
static void kmeans_block(const float* X, int n, int d, int C, int T, float* mu, int32_t* sizes, uint8_t* assign,
                         float* work /* C*d + C*d floats */) {
  const int Ci = C < n ? C : n;
  float* m2 = work;         /* -2 mu */
  float* sums = work + (size_t)C * d;
  int32_t cnt[256];
  float nrm[256];
  memset(mu, 0, sizeof(float) * (size_t)C * d);
  memset(sizes, 0, sizeof(int32_t) * (size_t)C);
  for (int c = 0; c < Ci; ++c) memcpy(mu + (size_t)c * d, X + (size_t)((int64_t)c * n / Ci) * d, sizeof(float) * d);
  for (int it = 0; it < T; ++it) {
    for (int c = 0; c < Ci; ++c) {
      nrm[c] = centroid_sqnorm(mu + (size_t)c * d, d);
      for (int k = 0; k < d; ++k) m2[(size_t)c * d + k] = -2.0f * mu[(size_t)c * d + k];
    }
    for (int r = 0; r < n; ++r) {
      const float* x = X + (size_t)r * d;
      int best = 0;
      float bd = 0.0f;
      for (int c = 0; c < Ci; ++c) {
        float D = nrm[c];
        const float* w = m2 + (size_t)c * d;
        for (int k = 0; k < d; ++k) D = fmaf(x[k], w[k], D);
        if (c == 0 || D < bd) {
          bd = D;
          best = c;
        }
      }
      assign[r] = (uint8_t)best;
    }
    memset(sums, 0, sizeof(float) * (size_t)Ci * d);
    for (int c = 0; c < Ci; ++c) cnt[c] = 0;
    for (int r = 0; r < n; ++r) {
      const int a = assign[r];
      const float* x = X + (size_t)r * d;
      float* s = sums + (size_t)a * d;
      for (int k = 0; k < d; ++k) s[k] = s[k] + x[k];
      cnt[a] += 1;
    }
    for (int c = 0; c < Ci; ++c) {
      if (cnt[c] > 0) {
        const float den = (float)cnt[c];
        for (int k = 0; k < d; ++k) mu[(size_t)c * d + k] = sums[(size_t)c * d + k] / den;
      }
      sizes[c] = cnt[c];
    }
  }
}

/* Every query block of every head: Q [BH][N][d] (float32 values), blocks of q_block
 * rows (the last one ragged). Outputs mu [BH][NQB][C][d], sizes [BH][NQB][C],
 * assign [BH][N]. Returns 0, or -1 for an unsupported size. */
int oc_kmeans_all(const float* Q, int BH, int N, int d, int q_block, int C, int T, float* mu, int32_t* sizes,
                  uint8_t* assign) {
  if (C < 1 || C > 256 || d < 1 || q_block < 1) return -1;
  const int nqb = (N + q_block - 1) / q_block;
  const int64_t total = (int64_t)BH * nqb;
  int bad = 0;
#pragma omp parallel
  {
    float* work = (float*)malloc(sizeof(float) * 2 * (size_t)C * d);
    if (!work) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t t = 0; t < total; ++t) {
        const int bh = (int)(t / nqb), i = (int)(t % nqb);
        const int r0 = i * q_block;
        const int n = (N - r0) < q_block ? (N - r0) : q_block;
        kmeans_block(Q + ((size_t)bh * N + r0) * d, n, d, C, T, mu + (size_t)t * C * d, sizes + (size_t)t * C,
                     assign + (size_t)bh * N + r0, work);
      }
      free(work);
    }
  }
  return bad ? -1 : 0;
}

/* ---- SIP sampler (AB-Attention abstract, SIP sentence; readings of oracle/sip.py) ---- */
#define SIP_ONE (1u << 24)

/* Philox4x32-10 as published by Salmon, Moraes, Dror and Shaw (SC'11). */
static void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c[2] * 0xCD9E8D57u;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c[0] = n0;
    c[1] = n1;
    c[2] = n2;
    c[3] = n3;
  }
}

void oc_philox(const uint32_t* ctr, const uint32_t* key, int64_t n, uint32_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t c[4] = {ctr[4 * i], ctr[4 * i + 1], ctr[4 * i + 2], ctr[4 * i + 3]};
    philox4x32_10(c, key[2 * i], key[2 * i + 1]);
    memcpy(out + 4 * i, c, sizeof c);
  }
}

/* w = max(1, floor(s 2^24)); NaN and s <= 0 give 1, s >= 1 gives 2^24. */
static uint64_t quantise(float s) {
  if (s >= 1.0f) return SIP_ONE;
  if (!(s > 0.0f)) return 1;
  const double v = floor((double)s * 16777216.0); /* exact: a power-of-two scaling */
  return v < 1.0 ? 1 : (uint64_t)v;
}

/* K = clamp(floor(density NKB + 0.5), 1, NKB), two separately rounded fp64 operations */
int oc_budget(double density, int nkb) {
  volatile double prod = density * (double)nkb;
  const double t = prod + 0.5;
  long long K = (long long)floor(t);
  if (K < 1) K = 1;
  if (K > nkb) K = nkb;
  return (int)K;
}

/* Integer water-filling of one row: thresholds t (pi_j = t_j / 2^24). */
static void thresholds(const float* s, int nkb, int K, uint64_t* w, uint8_t* capped, uint32_t* t) {
  for (int j = 0; j < nkb; ++j) {
    w[j] = quantise(s[j]);
    capped[j] = 0;
  }
  if (K >= nkb) {
    for (int j = 0; j < nkb; ++j) t[j] = SIP_ONE;
    return;
  }
  uint64_t room = 0, S = 0;
  for (;;) {
    uint64_t m = 0;
    S = 0;
    for (int j = 0; j < nkb; ++j) {
      if (capped[j]) ++m;
      else S += w[j];
    }
    room = (uint64_t)K - m;
    int any = 0;
    for (int j = 0; j < nkb; ++j)
      if (!capped[j] && room * w[j] >= S) any = 1;
    if (!any) break;
    for (int j = 0; j < nkb; ++j)
      if (!capped[j] && room * w[j] >= S) capped[j] = 1;
  }
  for (int j = 0; j < nkb; ++j) {
    if (capped[j]) {
      t[j] = SIP_ONE;
    } else {
      const uint64_t v = room * w[j] * (uint64_t)SIP_ONE / S;
      t[j] = (uint32_t)(v < 1 ? 1 : v);
    }
  }
}

/* SIP on rows of a score matrix: scores [rows][nkb]; row r is (b, h, i) = bhi[3r..3r+2].
 * Per row: counts[r]; idx[r][0..count) ascending; weights[r][0..count) = fp32(2^24) /
 * fp32(t_j); mask[r][ceil(nkb/32)] bit words; thresh[r][nkb] (may be NULL); uniforms
 * u[r][nkb] (may be NULL). Entries of idx/weights past the count are left untouched. */
void oc_sip_rows(const float* scores, int64_t rows, int nkb, int K, uint64_t seed, const int32_t* bhi, int32_t* counts,
                 int32_t* idx, float* weights, uint32_t* mask, uint32_t* thresh, uint32_t* uniforms) {
  const int words = (nkb + 31) / 32;
  const uint32_t key0 = (uint32_t)(seed & 0xFFFFFFFFu), key1 = (uint32_t)(seed >> 32);
#pragma omp parallel
  {
    uint64_t* w = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)nkb);
    uint8_t* capped = (uint8_t*)malloc((size_t)nkb);
    uint32_t* t = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)nkb);
#pragma omp for schedule(dynamic, 8)
    for (int64_t r = 0; r < rows; ++r) {
      thresholds(scores + (size_t)r * nkb, nkb, K, w, capped, t);
      uint32_t* mk = mask + (size_t)r * words;
      memset(mk, 0, sizeof(uint32_t) * (size_t)words);
      int c = 0;
      for (int g = 0; 4 * g < nkb; ++g) {
        uint32_t x[4] = {(uint32_t)g, (uint32_t)bhi[3 * r + 2], (uint32_t)bhi[3 * r + 1], (uint32_t)bhi[3 * r]};
        philox4x32_10(x, key0, key1);
        for (int e = 0; e < 4 && 4 * g + e < nkb; ++e) {
          const int j = 4 * g + e;
          const uint32_t u = x[e] >> 8;
          if (uniforms) uniforms[(size_t)r * nkb + j] = u;
          if (u < t[j]) {
            idx[(size_t)r * nkb + c] = j;
            weights[(size_t)r * nkb + c] = (float)SIP_ONE / (float)t[j];
            mk[j >> 5] |= 1u << (j & 31);
            ++c;
          }
        }
      }
      counts[r] = c;
      if (thresh) memcpy(thresh + (size_t)r * nkb, t, sizeof(uint32_t) * (size_t)nkb);
    }
    free(w);
    free(capped);
    free(t);
  }
}
