"""Pins for the oracle's attention and for the whole oracle pipeline.

* P8 - dense fp64 attention equals torch's scaled_dot_product_attention (CPU, float64).
* P1 - at density 1 every block is kept with weight 1, so the sparse weighted
  attention equals dense attention.
* P7 - unbiasedness on the tiny workload at density 0.25:
  (i) closed form: sum_j pi_j * omega_j * A_j equals the dense numerator and
      denominator (pi_j * omega_j = 1 up to one fp32 rounding);
  (ii) Monte-Carlo means of the numerator O*exp(LSE) and denominator exp(LSE)
      over 1000 sampling seeds lie within 5 standard errors of the dense values;
  (iii) the exact expectation of the normalised output over all 2^16 keep
      patterns of each query block, enumerated by brute force, matches the
      Monte-Carlo mean within 5 standard errors. The ratio bias E[O] - O_dense
      is reported, not asserted to vanish.
"""

import math

import numpy as np
import pytest
import torch

from oracle import Params, dense_attention, run_blocks, sparse_ht_attention
from oracle.sip import SIP_ONE


def test_p8_dense_matches_torch_sdpa(tiny_inputs):
    w, q, k, v = tiny_inputs
    o, lse = dense_attention(q[0, 0], k[0, 0], v[0, 0], 1 / math.sqrt(w.d))
    qt, kt, vt = (torch.from_numpy(x[0, 0].astype(np.float64))[None, None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, 0].numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = (qt[0, 0] @ kt[0, 0].T / math.sqrt(w.d))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


def test_p1_density_one_is_dense(tiny_inputs):
    w, q, k, v = tiny_inputs
    p = Params(w.q_block, w.k_block, w.n_clusters, w.kmeans_iters, 1.0, bf16=False)
    res = run_blocks(q, k, v, p, seed=123, blocks=[(0, 0, i) for i in range(w.nqb)])
    o_dense, lse_dense = dense_attention(q[0, 0], k[0, 0], v[0, 0], 1 / math.sqrt(w.d))
    for i in range(w.nqb):
        r = res[(0, 0, i)]
        assert r["count"] == w.nkb
        assert np.all(r["thresh"] == SIP_ONE) and np.all(r["weight"] == 1.0)
        np.testing.assert_allclose(r["O"], o_dense[i * 64:(i + 1) * 64], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["LSE"], lse_dense[i * 64:(i + 1) * 64], rtol=0, atol=1e-12)


def test_sparse_empty_and_partial_blocks():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((5, 8))
    k = rng.standard_normal((21, 8))
    v = rng.standard_normal((21, 8))
    o, lse = sparse_ht_attention(q, k, v, [], [], 4, 0.3)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # kept blocks {1, 5} with weights; block 5 is the ragged tail (key 20 only)
    o, lse = sparse_ht_attention(q, k, v, [1, 5], [2.0, 3.0], 4, 0.3)
    keys = [4, 5, 6, 7, 20]
    wts = np.array([2.0] * 4 + [3.0])
    a = np.exp(0.3 * q @ k[keys].T) * wts
    np.testing.assert_allclose(o, (a @ v[keys]) / a.sum(1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(lse, np.log(a.sum(1)), rtol=1e-12)


def _block_terms(q, k, v, k_block, scale):
    """Per-row, per-block dense terms A_j = sum_k a_k and N_j = sum_k a_k v_k (stabiliser = row max)."""
    s = scale * (q.astype(np.float64) @ k.astype(np.float64).T)
    M = s.max(axis=1, keepdims=True)
    a = np.exp(s - M)
    nkb = k.shape[0] // k_block
    A = a.reshape(q.shape[0], nkb, k_block).sum(axis=2)
    Nm = np.einsum("rjk,jkd->rjd", a.reshape(q.shape[0], nkb, k_block), v.astype(np.float64).reshape(nkb, k_block, -1))
    return M[:, 0], A, Nm


@pytest.mark.slow
def test_p7_unbiasedness(tiny_inputs):
    w, q, k, v = tiny_inputs
    scale = 1 / math.sqrt(w.d)
    p = Params(w.q_block, w.k_block, w.n_clusters, w.kmeans_iters, 0.25, bf16=False)
    blocks = [(0, 0, i) for i in range(w.nqb)]
    seeds = 1000
    res0 = run_blocks(q, k, v, p, seed=0, blocks=blocks, with_attention=False)
    thresh = {b: res0[b]["thresh"] for b in blocks}
    o_dense, lse_dense = dense_attention(q[0, 0], k[0, 0], v[0, 0], scale)
    num_sum = np.zeros((256, 64))
    num_sq = np.zeros((256, 64))
    den_sum = np.zeros(256)
    den_sq = np.zeros(256)
    o_sum = np.zeros((256, 64))
    o_sq = np.zeros((256, 64))
    for seed in range(seeds):
        res = run_blocks(q, k, v, p, seed=seed, blocks=blocks)
        for (b, h, i) in blocks:
            r = res[(b, h, i)]
            assert np.array_equal(r["thresh"], thresh[(b, h, i)])  # thresholds do not depend on the seed
            sl = slice(i * 64, (i + 1) * 64)
            den = np.exp(r["LSE"] - lse_dense[sl])  # relative to the dense denominator
            num = r["O"] * den[:, None]
            num_sum[sl] += num
            num_sq[sl] += num * num
            den_sum[sl] += den
            den_sq[sl] += den * den
            o_sum[sl] += r["O"]
            o_sq[sl] += r["O"] ** 2
    # (ii) numerator and denominator are unbiased: relative to the dense denominator,
    # E[den] = 1 and E[num] = O_dense
    den_mean = den_sum / seeds
    den_se = np.sqrt(np.maximum(den_sq / seeds - den_mean**2, 0) / seeds)
    assert np.all(np.abs(den_mean - 1.0) <= 5 * den_se + 1e-9)
    num_mean = num_sum / seeds
    num_se = np.sqrt(np.maximum(num_sq / seeds - num_mean**2, 0) / seeds)
    assert np.all(np.abs(num_mean - o_dense) <= 5 * num_se + 1e-9)

    # (i) closed form and (iii) exact enumeration of E[O]
    subsets = ((np.arange(1 << 16)[:, None] >> np.arange(16)[None, :]) & 1).astype(np.float64)
    worst_bias = 0.0
    for (b, h, i) in blocks:
        sl = slice(i * 64, (i + 1) * 64)
        t = thresh[(b, h, i)].astype(np.float64)
        pi = t / SIP_ONE
        omega = (np.float32(SIP_ONE) / thresh[(b, h, i)].astype(np.float32)).astype(np.float64)
        M, A, Nm = _block_terms(q[0, 0, sl], k[0, 0], v[0, 0], w.k_block, scale)
        # (i) E[sum_j I_j omega_j A_j] = sum_j pi_j omega_j A_j = sum_j A_j
        np.testing.assert_allclose((pi * omega * A).sum(1), A.sum(1), rtol=1e-7)
        mag = np.abs(Nm).sum(1)  # cancellation-free magnitude of each numerator entry
        assert np.all(np.abs(np.einsum("j,rjd->rd", pi * omega, Nm) - Nm.sum(1)) <= 1e-7 * mag + 1e-15)
        # (iii) enumerate the 2^16 keep patterns
        logp = (subsets * np.log(pi) + (1 - subsets) * np.log1p(-np.minimum(pi, 1 - 1e-300))).sum(1)
        logp = np.where(np.any((subsets == 0) & (pi[None, :] >= 1), axis=1), -np.inf, logp)
        prob = np.exp(logp)
        assert abs(prob.sum() - 1) < 1e-9
        sw = subsets * omega[None, :]  # [S, 16]
        EO = np.zeros((64, 64))
        for r0 in range(0, 64, 16):
            den = sw @ A[r0:r0 + 16].T  # [S, 16 rows]
            num = np.einsum("sj,rjd->srd", sw, Nm[r0:r0 + 16])
            with np.errstate(invalid="ignore", divide="ignore"):
                O = np.where(den[:, :, None] > 0, num / den[:, :, None], 0.0)
            EO[r0:r0 + 16] = np.einsum("s,srd->rd", prob, O)
        o_mean = o_sum[sl] / seeds
        o_se = np.sqrt(np.maximum(o_sq[sl] / seeds - o_mean**2, 0) / seeds)
        assert np.all(np.abs(o_mean - EO) <= 5 * o_se + 1e-9)
        worst_bias = max(worst_bias, float(np.abs(EO - o_dense[sl]).max()))
    print(f"ratio-estimator bias max |E[O] - O_dense| = {worst_bias:.3e}")
