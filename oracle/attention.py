"""Dense attention and Horvitz-Thompson sparse attention (oracle side), float64.

AB-Attention abstract (paperdot search page, query "Xing Ma"): 3D full
attention is the dense target (opening sentence); dynamic block-sparse
attention computes exact attention on the selected key/value blocks only
(problem sentence); each kept block carries weight 1/pi_j, pi_j its inclusion
probability, so the single weighted pass is an unbiased estimate of the dense
numerator and denominator (SIP sentence).

Readings: non-causal attention with softmax scale 1/sqrt(d) and no positional
transform inside the op; the weight omega_j multiplies block j's terms in both
the numerator sum_k a_k v_k and the denominator sum_k a_k; a query block that
keeps no key block returns O = 0 and LSE = -inf.
"""

import numpy as np


def dense_attention(q, k, v, scale):
    """softmax(scale * q k^T) v for one head. q [n, d], k/v [N, d]. Returns (O, LSE)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = float(scale) * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    a = np.exp(s - m)
    den = a.sum(axis=1, keepdims=True)
    out = (a @ v) / den
    lse = m[:, 0] + np.log(den[:, 0])
    return out, lse


def sparse_ht_attention(q, k, v, idx, weight, k_block, scale, dtype=np.float64):
    """Weighted attention of one query block over its kept key sub-blocks.

    q [n, d]; k, v [N, d] of the same (b, h); idx: kept sub-block indices;
    weight: omega_j per kept sub-block. Returns (O [n, d], LSE [n]) in float64
    (dtype=np.float32: the same steps in float32, the CPU timing mode).
    """
    q = np.asarray(q, dtype=dtype)
    n, d = q.shape
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size == 0:
        return np.zeros((n, d), dtype), np.full(n, -np.inf, dtype)
    k = np.asarray(k, dtype=dtype)
    v = np.asarray(v, dtype=dtype)
    N = k.shape[0]
    keys = []
    omega = []
    for j, w in zip(idx.tolist(), np.asarray(weight, dtype=dtype).tolist()):
        lo, hi = j * k_block, min(N, (j + 1) * k_block)
        keys.append(np.arange(lo, hi))
        omega.append(np.full(hi - lo, w))
    keys = np.concatenate(keys)
    omega = np.concatenate(omega).astype(dtype)
    s = dtype(scale) * (q @ k[keys].T)  # [n, kept keys]
    m = s.max(axis=1, keepdims=True)
    a = np.exp(s - m) * omega[None, :]
    den = a.sum(axis=1, keepdims=True)
    num = a @ v[keys]
    return num / den, m[:, 0] + np.log(den[:, 0])
