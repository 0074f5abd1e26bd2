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
  implementation reproduces it bit for bit: a distance is the left-to-right
  fp32 sum over dimensions of fl(fl(x - mu)^2) starting from 0 with separate
  multiply and add (no fused multiply-add); a centroid is the fp32 sum of its
  members in ascending row order, divided by the member count with one
  correctly rounded fp32 division.
* Each cluster stands in for its members by its centroid. For bf16 inputs the
  centroid is rounded to bf16 (ties to even) before it meets the keys, since
  that is the precision the keys have.
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
        # assignment: D(r, c) = (((0 + e_0) + e_1) + ...) with e_k = fl(fl(x_k - mu_k)^2)
        D = np.zeros((nb, n, Ci), dtype=np.float32)
        for k in range(d):
            diff = X[:, :, None, k] - mu[:, None, :Ci, k]
            D = D + diff * diff
        assign = np.argmin(D, axis=2)  # first minimum, i.e. lowest cluster index on ties
        if return_history:
            history.append(float(np.take_along_axis(D, assign[:, :, None], 2).astype(np.float64).sum()))
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


def block_scores(mu, sizes, n_rows, K, k_block, scale, bf16):
    """Block-importance estimates of one query block, float64 math, fp32 result.

    mu: float32 [C, d] centroids; sizes: [C] member counts; n_rows: rows in the
    query block; K: [N, d] keys (the exact values the GPU sees); k_block: Bk.
    Returns float32 [NKB].
    """
    mu = np.asarray(mu, dtype=np.float32)
    if bf16:
        mu = round_bf16(mu)
    K = np.asarray(K, dtype=np.float64)
    N = K.shape[0]
    nkb = -(-N // k_block)
    logits = float(scale) * (mu.astype(np.float64) @ K.T)  # [C, N]
    pad = nkb * k_block - N
    if pad:
        logits = np.concatenate([logits, np.full((logits.shape[0], pad), -np.inf)], axis=1)
    ell = _logsumexp(logits.reshape(logits.shape[0], nkb, k_block), axis=2)  # [C, NKB]
    L = _logsumexp(ell, axis=1)  # [C]
    w = np.asarray(sizes, dtype=np.float64) / float(n_rows)
    s = (w[:, None] * np.exp(ell - L[:, None])).sum(axis=0)
    return s.astype(np.float32)
