"""Top-K truncation (oracle side): the deterministic selection SIP is set against.

AB-Attention abstract (paperdot search page, query "Xing Ma"), SIP sentence:
sampling blocks with inverse-inclusion-probability weights lets one pass
estimate dense attention, where keeping only the best-scoring blocks truncates
it. For the estimator comparison the truncating rule is read as the plainest
deterministic counterpart of the sampler, on the same integers:

* the same quantised scores w_j = max(1, floor(s_j * 2^24)) and the same budget
  K = clamp(floor(rho * NKB + 0.5), 1, NKB) as SIP;
* keep the K sub-blocks with the largest w_j; among equal w_j the lower index
  is kept first, so exactly K are kept;
* every kept block has weight 1 (plain attention over the kept blocks).
"""

import numpy as np

from .sip import budget, quantize_scores


def topk_rows(scores, density, rows):
    """Top-K truncation on a set of rows of the score matrix.

    scores: float32 [B, H, NQB, NKB] (or anything indexable by (b, h, i) with a
    .shape). Returns a dict keyed by (b, h, i) with 'count', 'idx' (int32
    ascending), 'weight' (float32 ones) and 'mask' (uint32 bit words).
    """
    rows = list(rows)
    nkb = scores.shape[-1]
    K = budget(density, nkb)
    words = -(-nkb // 32)
    out = {}
    for (b, h, i) in rows:
        w = quantize_scores(np.asarray(scores[b, h, i], dtype=np.float32)).astype(np.int64)
        # primary key: larger w first; secondary key: lower index first
        order = np.lexsort((np.arange(nkb), -w))
        idx = np.sort(order[:K]).astype(np.int32)
        keep = np.zeros(words * 32, dtype=np.uint64)
        keep[idx] = 1
        mask = (keep.reshape(words, 32) << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
        out[(b, h, i)] = {"count": int(K), "idx": idx, "weight": np.ones(K, dtype=np.float32), "mask": mask}
    return out
