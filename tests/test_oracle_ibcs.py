"""Pins for the oracle's IBCS scorer (k-means + block-importance estimate).

* P2 - one cluster per query: the estimate equals the brute-force block mass of
  the dense softmax, averaged over the block's queries.
* P3 - one cluster: the estimate equals the block softmax mass of the block's
  mean query (the pooled summary the problem sentence criticises).
* P4 - k-means invariants: centroids are the means of their members; the
  objective does not increase; assignments are nearest-centroid; T iterations
  are taken; the result matches scikit-learn's Lloyd iterations from the same
  initial centroids.
* Score rows sum to 1, and bf16 rounding matches torch's.
* The clustering's fp32 arithmetic: the fused multiply-add against hand-worked
  values (one where separate rounding gives 0, one where rounding the float64
  sum directly to fp32 rounds twice) and against exact rationals; the centroid
  norm's halving tree and the comparison distances against exact-rational
  step-by-step evaluation; a block where only fused arithmetic gives the
  oracle's assignment.
"""

import math

import numpy as np
import pytest
import torch

from oracle.ibcs import block_scores, centroid_sqnorm, fma_f32, kmeans_distances, kmeans_fp32, round_bf16


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
        # the last assignment is nearest-centroid w.r.t. the centroids before the final
        # update, up to the rounding of the fp32 comparison: each compared value is an
        # fp32 chain of d fused multiply-adds plus a norm of at most d + 7 rounded
        # steps, so its error is below (2d + 8) u (|mu|^2 + 2 sum |x mu|), u = 2^-24
        if T > 1:
            mu_prev = kmeans_fp32(X, C, T - 1)[0].astype(np.float64)[:Ci]
            X64 = X.astype(np.float64)
            D = ((X64[:, None, :] - mu_prev[None, :, :]) ** 2).sum(axis=2)
            bound = (2 * d + 8) * 2.0 ** -24 * ((mu_prev ** 2).sum(axis=1)[None, :] + 2 * np.abs(X64) @ np.abs(mu_prev).T)
            best = D.argmin(axis=1)
            rows = np.arange(n)
            assert np.all(D[rows, assign] <= D[rows, best] + bound[rows, assign] + bound[rows, best])
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


def test_bf16_estimate_uses_the_scaled_centroid_at_bf16(tiny_inputs):
    """For bf16 inputs the centroid meets the keys as bf16(fl32(c2 * mu)) with
    c2 = fl32(scale * log2 e), the logits being base-2. Centroids chosen so that
    c2 * mu rounds to a given bf16 vector t make that rounding the identity: the
    estimate must then equal the unrounded fp32 estimate at mu = t / (scale log2 e)
    (the two differ only by mu's own fp32 rounding). Rounding mu before scaling,
    a missing ln 2 or a wrong constant moves the scores well past that comparison's tolerance."""
    w, q, k, v = tiny_inputs
    scale = 1.0 / math.sqrt(w.d)
    rng = np.random.default_rng(11)
    c2 = np.float32(np.float32(scale) * np.float32(1.4426950408889634))
    t = round_bf16((rng.standard_normal((4, w.d)) * 4.0).astype(np.float32))
    mu = (t.astype(np.float64) / float(c2)).astype(np.float32)
    assert np.array_equal(round_bf16((mu * c2).astype(np.float32)), t)
    sizes = np.array([30, 20, 10, 4], dtype=np.int32)
    K = k[0, 0]
    s_bf16 = block_scores(mu, sizes, 64, K, w.k_block, scale, bf16=True).astype(np.float64)
    exact = (t.astype(np.float64) / (np.float64(np.float32(scale)) * np.log2(np.e))).astype(np.float32)
    s_ref = block_scores(exact, sizes, 64, K, w.k_block, scale, bf16=False).astype(np.float64)
    np.testing.assert_allclose(s_bf16, s_ref, rtol=1e-5, atol=1e-9)
    # the reading that rounds mu itself fails the same comparison
    s_other = block_scores(round_bf16(mu), sizes, 64, K, w.k_block, scale, bf16=False).astype(np.float64)
    assert not np.allclose(s_other, s_ref, rtol=1e-5, atol=1e-9)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10, np.array([0.0, -0.0, 1.0, 3.0039062, 1e-40], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)


def test_fma_f32_hand_worked():
    a = np.float32(1 + 2.0 ** -12)  # a*a = 1 + 2^-11 + 2^-24 exactly
    # separate rounding loses the 2^-24 (a tie at 1 + 2^-11, kept even), the fused form keeps it
    assert fma_f32(a, a, np.float32(-(1 + 2.0 ** -11))) == np.float32(2.0 ** -24)
    assert np.float32(np.float32(a * a) - np.float32(1 + 2.0 ** -11)) == 0.0
    # exact value 1 + 2^-11 + 2^-24 + 2^-80 lies just above the fp32 midpoint: correct
    # rounding goes up; the float64 sum is the midpoint itself and would round down to even
    got = fma_f32(a, a, np.float32(2.0 ** -80))
    assert got == np.float32(1 + 2.0 ** -11 + 2.0 ** -23)
    assert np.float32(np.float64(a) * np.float64(a) + 2.0 ** -80) == np.float32(1 + 2.0 ** -11)
    # same below the midpoint: the exact value rounds down
    assert fma_f32(a, a, np.float32(-(2.0 ** -80))) == np.float32(1 + 2.0 ** -11)
    # signs, zero and an exact result
    assert fma_f32(np.float32(-3.0), np.float32(0.5), np.float32(1.5)) == 0.0
    assert fma_f32(np.float32(2.0), np.float32(3.0), np.float32(-1.0)) == np.float32(5.0)


def test_fma_f32_against_exact_rationals():
    import kmeans_rounding_case as case

    rng = np.random.default_rng(21)
    n = 3000
    a = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32)
    b = (rng.standard_normal(n) * 2.0 ** rng.integers(-20, 20, n)).astype(np.float32)
    c = (rng.standard_normal(n) * 2.0 ** rng.integers(-40, 40, n)).astype(np.float32)
    # a third of the cases cancel the product almost exactly, where rounding matters most
    k = n // 3
    c[:k] = (-(a[:k].astype(np.float64) * b[:k].astype(np.float64))).astype(np.float32)
    got = fma_f32(a, b, c)
    for i in range(n):
        assert got[i] == case.fma_exact(a[i], b[i], c[i]), (a[i], b[i], c[i])


@pytest.mark.parametrize("d", [8, 64, 100, 128])
def test_centroid_sqnorm_tree(d):
    import kmeans_rounding_case as case

    rng = np.random.default_rng(d)
    mu = (rng.standard_normal((3, d)) * 10.0 ** rng.uniform(-2, 2, size=(3, d))).astype(np.float32)
    got = centroid_sqnorm(mu)
    for c in range(3):
        assert got[c] == case.sqnorm_exact(mu[c])
        np.testing.assert_allclose(float(got[c]), float((mu[c].astype(np.float64) ** 2).sum()), rtol=1e-5)


@pytest.mark.parametrize("d", [16, 70])
def test_kmeans_distances_stepwise(d):
    import kmeans_rounding_case as case

    rng = np.random.default_rng(100 + d)
    X = rng.standard_normal((6, d)).astype(np.float32)
    mu = (rng.standard_normal((3, d)) + 0.5).astype(np.float32)
    D = kmeans_distances(X, mu)
    for r in range(6):
        for c in range(3):
            assert D[r, c] == case.distance_fused(X[r], mu[c])
    # and it is the squared distance less |x|^2, up to rounding
    ref = ((X.astype(np.float64)[:, None, :] - mu.astype(np.float64)[None]) ** 2).sum(-1) - (X.astype(np.float64) ** 2).sum(-1)[:, None]
    np.testing.assert_allclose(D, ref, rtol=0, atol=1e-4 * (1 + np.abs(ref).max()))


@pytest.mark.parametrize("dim", [64, 128])
def test_kmeans_distance_uses_fused_multiply_add(dim):
    """On a block built so that one row's two comparisons are equal in exact arithmetic,
    the oracle's assignment is the one of the fused chain and not the one of separately
    rounded multiplies and adds (both computed with exact rationals)."""
    import kmeans_rounding_case as case

    X, row, fused, separate = case.build(dim)
    assert fused != separate
    _, _, assign = kmeans_fp32(X, 2, 1)
    assert int(assign[row]) == fused


def test_block_scores_many_equals_block_scores():
    """The batched form used by the full-size checks is the same definition: per block
    it equals block_scores up to the last bit of the fp32 result (matrix products of
    different shapes may sum in another order)."""
    from oracle.ibcs import block_scores_many

    rng = np.random.default_rng(11)
    N, d = 700, 64
    K = rng.standard_normal((N, d)).astype(np.float32)
    Q = rng.standard_normal((N, d)).astype(np.float32)
    mus, szs, ns = [], [], []
    for i in range(6):
        lo, hi = i * 128, min(N, (i + 1) * 128)
        mu, sz, _ = kmeans_fp32(Q[lo:hi], 8, 2)
        mus.append(mu)
        szs.append(sz)
        ns.append(hi - lo)
    for bf in (True, False):
        many = block_scores_many(np.stack(mus), np.stack(szs), np.array(ns), K, 32, 0.125, bf, chunk=4)
        for i in range(6):
            one = block_scores(mus[i], szs[i], ns[i], K, 32, 0.125, bf)
            ulp = np.spacing(np.maximum(np.abs(one), np.float32(1e-30)))
            assert np.all(np.abs(one - many[i]) <= ulp), (bf, i)
