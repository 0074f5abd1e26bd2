"""IBCS: intra-block clustering selector (oracle side).

AB-Attention abstract (paperdot search page, query "Xing Ma"), IBCS sentence:
block importance is estimated by clustering the queries of each query block on
their own, with tokens left in place. The pages give neither the clustering
algorithm nor the estimate's formula. Readings used here:

* Query block i holds rows [i*Bq, min(N, (i+1)*Bq)); key sub-block j holds keys
  [j*Bk, min(N, (j+1)*Bk)); both are contiguous ranges of the raster order.
* Clustering is Lloyd's k-means with a fixed number T of iterations on raw
  queries, squared Euclidean distance, C_i = min(C, n_i) clusters initialised at
  the strided queries X[floor(c*n_i/C_i)]. Each iteration assigns every query
  to its nearest centroid (ties to the lowest index) and then replaces each
  centroid by the mean of its members; an empty cluster keeps its centroid and
  gets size 0.
* It is specified operation by operation in fp32 so that any correct
  implementation reproduces it bit for bit. Queries are compared through
  |mu_c|^2 - 2 x.mu_c, the squared distance less the query's own |x|^2, which
  leaves the nearest centroid unchanged: starting from |mu_c|^2, each dimension
  k in ascending order adds x_k * (-2 mu_ck) with one fused multiply-add
  (-2 mu is exact). |mu_c|^2 rounds each product mu_k^2 to fp32 and sums them
  within each group of 64 dimensions by the halving tree (k with k+32, then k
  with k+16, ..., then k with k+1; absent dimensions count as 0), then adds
  the group sums left to right. A centroid is the fp32 sum of its members in
  ascending row order, divided by the member count with one correctly rounded
  fp32 division.
* Each cluster stands in for its members by its centroid. For bf16 inputs the
  centroid meets the keys at the keys' precision: it is multiplied in fp32 by
  c2 = fl32(fl32(scale) * fl32(log2 e)) and the product is rounded to bf16 (ties
  to even), so the logit in base-2 units is the exact dot product of that bf16
  vector with the key (one rounding of the scaled centroid, as one rounding of
  the centroid itself would be; the pages fix neither).
* Estimate: s_ij = sum_c (n_c / n_i) * exp(l_cj - L_c) with
  l_cj = log sum_{k in j} exp(scale * mu_c . k_k) and L_c = log sum_j exp(l_cj),
  i.e. the mean softmax mass that block i's queries put on sub-block j when
  every query is replaced by its cluster centroid. sum_j s_ij = 1.
"""

import numpy as np


def round_bf16(x):
    """Round float32 values to the nearest bf16 value (ties to even), as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return (r & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32).reshape(np.shape(x))


def fma_f32(a, b, c):
    """fp32 fused multiply-add a*b + c with a single rounding (nearest, ties to even).

    The product of two fp32 values is exact in float64 (at most 48 significant
    bits). The float64 sum p + c is made exact-or-odd: its rounding error e comes
    from Knuth's TwoSum, and an inexact sum whose last bit is even is moved one
    float64 step towards the exact value. Rounding to odd with two or more spare
    bits, then to nearest at the narrower precision, gives the correctly rounded
    result (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
    proved algorithms using rounding to odd", IEEE Trans. Computers, 2008).
    """
    a64 = np.asarray(a, dtype=np.float32).astype(np.float64)
    b64 = np.asarray(b, dtype=np.float32).astype(np.float64)
    c64 = np.asarray(c, dtype=np.float32).astype(np.float64)
    p = a64 * b64
    with np.errstate(invalid="ignore", over="ignore"):
        s = p + c64
        bv = s - p
        e = (p - (s - bv)) + (c64 - bv)
        s = np.array(s, dtype=np.float64, copy=True)
        even = (s.view(np.int64) & 1) == 0
        fix = np.isfinite(s) & (e != 0) & even
        if np.any(fix):
            s[fix] = np.nextafter(s[fix], np.where(e[fix] > 0, np.inf, -np.inf))
        return s.astype(np.float32)


def centroid_sqnorm(mu):
    """|mu|^2 over the last axis, as the clustering computes it (fp32).

    Products rounded one by one; halving-tree sum inside each group of 64
    dimensions (zero-padded); group sums added left to right.
    """
    mu = np.asarray(mu, dtype=np.float32)
    d = mu.shape[-1]
    G = -(-d // 64)
    t = np.zeros(mu.shape[:-1] + (G * 64,), dtype=np.float32)
    t[..., :d] = mu * mu
    t = t.reshape(mu.shape[:-1] + (G, 64))
    for s in (32, 16, 8, 4, 2, 1):
        t[..., :s] = t[..., :s] + t[..., s:2 * s]
    out = t[..., 0, 0].copy()
    for g in range(1, G):
        out = out + t[..., g, 0]
    return out


def kmeans_distances(X, mu):
    """Comparison distances |mu_c|^2 - 2 x_r.mu_c, fp32 [..., n, C].

    X: float32 [..., n, d]; mu: float32 [..., C, d]. Each entry starts at the
    centroid's norm and takes one fused multiply-add per dimension, ascending.
    """
    X = np.asarray(X, dtype=np.float32)
    mu = np.asarray(mu, dtype=np.float32)
    m2 = (np.float32(-2.0) * mu).astype(np.float32)
    D = np.broadcast_to(centroid_sqnorm(mu)[..., None, :], X.shape[:-1] + (mu.shape[-2],)).astype(np.float32)
    for k in range(X.shape[-1]):
        D = fma_f32(X[..., :, None, k], m2[..., None, :, k], D)
    return D


def kmeans_fp32(X, n_clusters, iters, return_history=False):
    """Fixed-iteration k-means of each query block, exact-operation fp32.

    X: float32 [nb, n, d] (a batch of equal-length blocks) or [n, d].
    Returns (mu float32 [nb, C, d], sizes int32 [nb, C], assign uint8 [nb, n]),
    without the leading axis when X was 2-D. With return_history the list of
    the clustering objective (sum of each query's distance to its assigned
    centroid, float64) after every assignment step is appended.
    """
    X = np.asarray(X, dtype=np.float32)
    squeeze = X.ndim == 2
    if squeeze:
        X = X[None]
    nb, n, d = X.shape
    C = int(n_clusters)
    T = int(iters)
    if C < 1 or T < 1 or n < 1:
        raise ValueError("need n_clusters >= 1, iters >= 1 and a non-empty block")
    Ci = min(C, n)
    bidx = np.arange(nb)
    mu = np.zeros((nb, C, d), dtype=np.float32)
    for c in range(Ci):
        mu[:, c, :] = X[:, (c * n) // Ci, :]
    sizes = np.zeros((nb, C), dtype=np.int32)
    assign = np.zeros((nb, n), dtype=np.int64)
    history = []
    for _ in range(T):
        # assignment: nearest centroid by |mu|^2 - 2 x.mu
        D = kmeans_distances(X, mu[:, :Ci])
        assign = np.argmin(D, axis=2)  # first minimum, i.e. lowest cluster index on ties
        if return_history:
            diff = X.astype(np.float64) - np.take_along_axis(mu[:, :Ci], assign[:, :, None], 1).astype(np.float64)
            history.append(float((diff * diff).sum()))
        # update: members summed in ascending row order, one division per coordinate
        sums = np.zeros((nb, Ci, d), dtype=np.float32)
        counts = np.zeros((nb, Ci), dtype=np.int64)
        for r in range(n):
            a = assign[:, r]
            sums[bidx, a] = sums[bidx, a] + X[:, r]
            counts[bidx, a] += 1
        nz = counts > 0
        denom = np.where(nz, counts, 1).astype(np.float32)
        newmu = sums / denom[:, :, None]
        mu[:, :Ci] = np.where(nz[:, :, None], newmu, mu[:, :Ci])
        sizes[:, :Ci] = counts.astype(np.int32)
    out = (mu, sizes, assign.astype(np.uint8))
    if squeeze:
        out = (mu[0], sizes[0], out[2][0])
    if return_history:
        out = out + (history,)
    return out


def _logsumexp(x, axis):
    m = np.max(x, axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    return np.squeeze(m, axis=axis) + np.log(np.sum(np.exp(x - m), axis=axis))


def block_scores(mu, sizes, n_rows, K, k_block, scale, bf16, dtype=np.float64):
    """Block-importance estimates of one query block, float64 math, fp32 result
    (dtype=np.float32: the same steps in float32, the CPU timing mode).

    mu: float32 [C, d] centroids; sizes: [C] member counts; n_rows: rows in the
    query block; K: [N, d] keys (the exact values the GPU sees); k_block: Bk.
    Returns float32 [NKB].
    """
    mu = np.asarray(mu, dtype=np.float32)
    K = np.asarray(K, dtype=dtype)
    N = K.shape[0]
    nkb = -(-N // k_block)
    if bf16:
        c2 = np.float32(np.float32(scale) * np.float32(np.log2(np.e)))
        mu2 = round_bf16((mu * c2).astype(np.float32))  # scale * log2(e) * mu at bf16
        logits = dtype(np.log(2.0)) * (mu2.astype(dtype) @ K.T)  # base-2 logits in natural units
    else:
        logits = dtype(scale) * (mu.astype(dtype) @ K.T)  # [C, N]
    pad = nkb * k_block - N
    if pad:
        logits = np.concatenate([logits, np.full((logits.shape[0], pad), -np.inf)], axis=1)
    ell = _logsumexp(logits.reshape(logits.shape[0], nkb, k_block), axis=2)  # [C, NKB]
    L = _logsumexp(ell, axis=1)  # [C]
    w = np.asarray(sizes, dtype=dtype) / dtype(n_rows)
    s = (w[:, None] * np.exp(ell - L[:, None])).sum(axis=0)
    return s.astype(np.float32)


def block_scores_many(mu, sizes, n_rows, K, k_block, scale, bf16, chunk=64):
    """block_scores for many query blocks of one head at once (the same definition, the
    centroids of several blocks stacked into one matrix product).

    mu: float32 [nb, C, d]; sizes: [nb, C]; n_rows: [nb] rows per block; K: [N, d] keys.
    Returns float32 [nb, NKB]. chunk: blocks per matrix product (memory bound only)."""
    mu = np.asarray(mu, dtype=np.float32)
    nb, C, d = mu.shape
    K = np.asarray(K, dtype=np.float64)
    N = K.shape[0]
    nkb = -(-N // k_block)
    pad = nkb * k_block - N
    out = np.zeros((nb, nkb), np.float32)
    if bf16:
        c2 = np.float32(np.float32(scale) * np.float32(np.log2(np.e)))
    for b0 in range(0, nb, chunk):
        m = mu[b0:b0 + chunk]
        nbc = m.shape[0]
        flat = m.reshape(nbc * C, d)
        if bf16:
            logits = np.log(2.0) * (round_bf16((flat * c2).astype(np.float32)).astype(np.float64) @ K.T)
        else:
            logits = float(scale) * (flat.astype(np.float64) @ K.T)
        if pad:
            logits = np.concatenate([logits, np.full((logits.shape[0], pad), -np.inf)], axis=1)
        ell = _logsumexp(logits.reshape(nbc * C, nkb, k_block), axis=2)  # [nbc*C, NKB]
        L = _logsumexp(ell, axis=1)
        w = np.asarray(sizes[b0:b0 + chunk], dtype=np.float64).reshape(nbc * C) / np.repeat(
            np.asarray(n_rows[b0:b0 + chunk], dtype=np.float64), C)
        s = (w[:, None] * np.exp(ell - L[:, None])).reshape(nbc, C, nkb).sum(axis=1)
        out[b0:b0 + nbc] = s.astype(np.float32)
    return out
