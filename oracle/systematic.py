"""Fixed-size (systematic) sampling with SIP's inclusion probabilities (oracle side).

AB-Attention abstract (paperdot search page, query "Xing Ma"), SIP sentence:
blocks are sampled with known inclusion probabilities and reweighted by their
inverse. The abstract does not fix the sampling design; independent (Poisson)
trials are the reading of ``oracle/sip.py``. This module is the other standard
design with the same probabilities, systematic sampling, which keeps a nearly
fixed number of blocks per row. Reading:

* thresholds t_j exactly as SIP (same quantised scores, budget K and integer
  water-filling), so pi_j = t_j / 2^24;
* one 24-bit uniform U per row: word 0 of Philox4x32-10 with key
  (seed mod 2^32, seed >> 32) and counter (2^32 - 1, i, h, b), shifted right by
  8 (the per-block draws of SIP use counter words below 2^14, never this one);
* with C_j = t_0 + ... + t_{j-1} (exact integers), sub-block j is kept iff the
  half-open interval [C_j, C_j + t_j) holds a point U + m * 2^24 (m >= 0). As
  t_j <= 2^24 and U takes each of its 2^24 values equally often, j is kept for
  exactly t_j of them: pi_j = t_j / 2^24 exactly, so the inverse weights stay
  unbiased, and a row keeps floor(T / 2^24) or that plus one block
  (T = sum of t_j, which is K * 2^24 up to the floors of the thresholds);
* weight fp32(2^24) / fp32(t_j), as in SIP.
"""

import numpy as np

from .philox import philox4x32_10
from .sip import SIP_ONE, budget, inclusion_thresholds, quantize_scores

ROW_COUNTER = 0xFFFFFFFF


def row_uniform24(seed, b, h, i):
    """The row's 24-bit uniform U."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)
    ctr = np.array([[ROW_COUNTER, i, h, b]], dtype=np.uint32)
    return int(philox4x32_10(ctr, key)[0, 0]) >> 8


def points_below(x, U):
    """Number of points U + m * 2^24 (m >= 0) strictly below x (x, U non-negative integers)."""
    x = np.asarray(x, dtype=np.int64)
    return np.where(x > U, (x - 1 - U) // SIP_ONE + 1, 0)


def keep_systematic(t, U):
    """Kept mask of one row from its thresholds t (uint32 [NKB]) and uniform U."""
    t = np.asarray(t, dtype=np.int64)
    c = np.concatenate([[0], np.cumsum(t)[:-1]])
    return points_below(c + t, U) > points_below(c, U)


def sample_rows_systematic(scores, density, seed, rows):
    """Systematic sampling on a set of rows; same output dict as ``sample_rows``."""
    rows = list(rows)
    if not rows:
        return {}
    nkb = scores.shape[-1]
    K = budget(density, nkb)
    S = np.stack([np.asarray(scores[b, h, i], dtype=np.float32) for (b, h, i) in rows])
    t = inclusion_thresholds(quantize_scores(S), K)
    words = -(-nkb // 32)
    out = {}
    for r, (b, h, i) in enumerate(rows):
        keep = keep_systematic(t[r], row_uniform24(seed, b, h, i))
        idx = np.nonzero(keep)[0].astype(np.int32)
        wgt = (np.float32(SIP_ONE) / t[r, idx].astype(np.float32)).astype(np.float32)
        bits = np.zeros(words * 32, dtype=np.uint64)
        bits[:nkb] = keep
        mask = (bits.reshape(words, 32) << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
        out[(b, h, i)] = {"count": int(idx.size), "idx": idx, "weight": wgt, "thresh": t[r], "mask": mask}
    return out
