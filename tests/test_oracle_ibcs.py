"""Pins for the oracle's IBCS scorer (k-means + block-importance estimate).

* P2 - one cluster per query: the estimate equals the brute-force block mass of
  the dense softmax, averaged over the block's queries.
* P3 - one cluster: the estimate equals the block softmax mass of the block's
  mean query (the pooled "coarse summary").
* P4 - k-means invariants: centroids are the means of their members; the
  objective does not increase; assignments are nearest-centroid; T iterations
  are taken; the result matches scikit-learn's Lloyd iterations from the same
  initial centroids.
* Score rows sum to 1, and bf16 rounding matches torch's.
"""

import math

import numpy as np
import pytest
import torch

from oracle.ibcs import block_scores, kmeans_fp32, round_bf16


def _dense_block_mass(q, k, k_block, scale):
    s = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    N = k.shape[0]
    nkb = -(-N // k_block)
    mass = np.zeros((q.shape[0], nkb))
    for j in range(nkb):
        mass[:, j] = p[:, j * k_block:(j + 1) * k_block].sum(axis=1)
    return mass


def test_p2_single_query_clusters_give_block_mass(tiny_inputs):
    w, q, k, v = tiny_inputs
    scale = 1.0 / math.sqrt(w.d)
    for i in range(w.nqb):
        X = q[0, 0, i * 64:(i + 1) * 64]
        mu, sizes, assign = kmeans_fp32(X, 64, 3)
        assert np.array_equal(assign, np.arange(64))
        assert np.all(sizes == 1)
        np.testing.assert_array_equal(mu, X)
        s = block_scores(mu, sizes, 64, k[0, 0], w.k_block, scale, bf16=False)
        brute = _dense_block_mass(X, k[0, 0], w.k_block, scale).mean(axis=0)
        np.testing.assert_allclose(s, brute, rtol=2e-6, atol=1e-9)


def test_p3_one_cluster_is_pooled_query(tiny_inputs):
    w, q, k, v = tiny_inputs
    scale = 1.0 / math.sqrt(w.d)
    for i in range(w.nqb):
        X = q[0, 0, i * 64:(i + 1) * 64]
        mu, sizes, _ = kmeans_fp32(X, 1, 2)
        assert sizes[0] == 64
        pooled = X.astype(np.float64).mean(axis=0, keepdims=True)
        np.testing.assert_allclose(mu[0], pooled[0], rtol=0, atol=1e-5)
        s = block_scores(mu, sizes, 64, k[0, 0], w.k_block, scale, bf16=False)
        brute = _dense_block_mass(pooled, k[0, 0], w.k_block, scale)[0]
        np.testing.assert_allclose(s, brute, rtol=1e-4, atol=1e-9)


def test_scores_sum_to_one_and_tail_blocks(tiny_inputs):
    w, q, k, v = tiny_inputs
    scale = 1.0 / math.sqrt(w.d)
    # a ragged key count: drop the last 5 keys so the last sub-block has 11 keys
    K = k[0, 0, :251]
    X = q[0, 0, 192:256]
    mu, sizes, _ = kmeans_fp32(X, 4, 4)
    s = block_scores(mu, sizes, 64, K, 16, scale, bf16=False)
    assert s.shape == (16,)
    assert abs(float(s.astype(np.float64).sum()) - 1.0) < 1e-6
    # with C = n the ragged sub-block still equals the brute-force mass
    mu1, sz1, _ = kmeans_fp32(X, 64, 1)
    s1 = block_scores(mu1, sz1, 64, K, 16, scale, bf16=False)
    brute = _dense_block_mass(X, K, 16, scale).mean(axis=0)
    np.testing.assert_allclose(s1, brute, rtol=2e-6, atol=1e-9)


def _objective(X, mu, assign):
    return float(((X.astype(np.float64) - mu.astype(np.float64)[assign]) ** 2).sum())


def test_p4_kmeans_invariants():
    rng = np.random.default_rng(3)
    for n, d, C, T in [(64, 64, 4, 4), (128, 128, 8, 4), (37, 16, 8, 6), (5, 8, 8, 2)]:
        X = (rng.standard_normal((n, d)) + 3 * rng.integers(0, 3, size=(n, 1))).astype(np.float32)
        mu, sizes, assign, hist = kmeans_fp32(X, C, T, return_history=True)
        Ci = min(C, n)
        assert len(hist) == T
        assert sizes.sum() == n and np.all(sizes[Ci:] == 0)
        assert np.array_equal(np.bincount(assign, minlength=C)[:C], sizes)
        # centroids are the means of their members (fp32 sequential sum, within rounding)
        for c in range(Ci):
            if sizes[c]:
                ref = X[assign == c].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(mu[c], ref, rtol=0, atol=1e-5 * (1 + np.abs(ref).max()))
        # objective non-increasing across iterations (exact arithmetic; fp32 slack)
        for a, b in zip(hist, hist[1:]):
            assert b <= a * (1 + 1e-5) + 1e-6
        # the last assignment is nearest-centroid w.r.t. the centroids before the final update
        mu_prev, _, assign_prev = kmeans_fp32(X, C, T - 1)[:3] if T > 1 else (None, None, None)
        if T > 1:
            D = ((X.astype(np.float64)[:, None, :] - mu_prev.astype(np.float64)[None, :Ci, :]) ** 2).sum(axis=2)
            best = D.min(axis=1)
            chosen = D[np.arange(n), assign]
            assert np.all(chosen <= best * (1 + 1e-5) + 1e-6)
        # T matters: one more iteration changes nothing only if converged
        mu2, _, assign2 = kmeans_fp32(X, C, T + 1)
        if not np.array_equal(assign2, assign):
            assert not np.array_equal(mu2, mu)


def test_p4_matches_sklearn_lloyd():
    sk = pytest.importorskip("sklearn.cluster")
    rng = np.random.default_rng(11)
    checked = 0
    for trial in range(6):
        n, d, C, T = 128, 32, 8, 3
        X = (rng.standard_normal((n, d)) + 2.5 * rng.integers(0, 4, size=(n, 1))).astype(np.float32)
        mu, sizes, assign = kmeans_fp32(X, C, T)
        if np.any(sizes == 0):
            continue  # scikit-learn relocates empty clusters; the readings keep them
        init = X[[(c * n) // C for c in range(C)]].astype(np.float64)
        km = sk.KMeans(n_clusters=C, init=init, n_init=1, max_iter=T, tol=0.0, algorithm="lloyd")
        km.fit(X.astype(np.float64))
        np.testing.assert_allclose(mu.astype(np.float64), km.cluster_centers_, rtol=0, atol=2e-5)
        checked += 1
    assert checked >= 3


def test_kmeans_tie_goes_to_lowest_cluster_and_empty_cluster_kept():
    # init: rows floor(0*4/2)=0 and floor(1*4/2)=2 -> mu = [1,0], [5,0]; the query
    # [3,0] is at squared distance 4 from both and must go to cluster 0
    X = np.array([[1.0, 0.0], [3.0, 0.0], [5.0, 0.0], [6.0, 0.0]], dtype=np.float32)
    mu, sizes, assign = kmeans_fp32(X, 2, 1)
    assert assign.tolist() == [0, 0, 1, 1]
    np.testing.assert_array_equal(mu, np.array([[2.0, 0.0], [5.5, 0.0]], dtype=np.float32))
    X2 = np.array([[0.0, 0.0], [0.0, 0.0], [0.0, 0.0], [0.0, 0.0]], dtype=np.float32)
    mu2, sizes2, assign2 = kmeans_fp32(X2, 2, 2)
    assert assign2.tolist() == [0, 0, 0, 0]
    assert sizes2.tolist() == [4, 0]
    np.testing.assert_array_equal(mu2[1], X2[2])  # the empty cluster keeps its centroid


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10, np.array([0.0, -0.0, 1.0, 3.0039062, 1e-40], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)


@pytest.mark.parametrize("dim", [64, 128])
def test_kmeans_rounds_multiply_and_add_separately(dim):
    """On a block built so that one row's two distances are equal in exact arithmetic,
    the oracle's assignment is the one of separately rounded multiplies and adds
    (computed here term by term) and not the one of a fused multiply-add (computed
    with exact rationals): the spec's rounding is what decides it."""
    import kmeans_rounding_case as case

    X, row, separate, fused = case.build(dim)
    assert separate != fused
    _, _, assign = kmeans_fp32(X, 2, 1)
    assert int(assign[row]) == separate
