"""The whole path on selected query blocks: IBCS scores, SIP draw, weighted attention.

Every query block (b, h, i) is independent through all three stages, so the
oracle can run any subset of them. The order of steps is the one the
AB-Attention abstract (paperdot search page, query "Xing Ma") gives: IBCS
estimates, SIP sampling and reweighting, then attention on the kept blocks.
"""

import dataclasses
import math

import numpy as np

from .attention import sparse_ht_attention
from .ibcs import block_scores, kmeans_fp32
from .sip import sample_rows


@dataclasses.dataclass(frozen=True)
class Params:
    q_block: int
    k_block: int
    n_clusters: int
    kmeans_iters: int
    density: float
    bf16: bool
    scale: float = 0.0  # <= 0 means 1/sqrt(d)

    def softmax_scale(self, d):
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(d)


def run_blocks(q, k, v, p, seed, blocks, with_attention=True, precision="fp64"):
    """Run the path on query blocks `blocks` = [(b, h, i), ...].

    q, k, v: float32 [B, H, N, d] holding exactly the values the GPU sees.
    Returns a dict keyed by (b, h, i) with centroids/sizes/assign, the fp32
    score row, the SIP draw (count/idx/weight/thresh/mask) and, when asked,
    O (float64 [n_i, d]) and LSE (float64 [n_i]).
    precision: "fp64" (parity) or "fp32" (the same steps with the score and
    attention arithmetic in float32: the CPU timing mode).
    """
    dt = np.float64 if precision == "fp64" else np.float32
    B, H, N, d = q.shape
    scale = p.softmax_scale(d)
    nkb = -(-N // p.k_block)
    blocks = list(blocks)
    res = {}
    scores = {}
    for (b, h, i) in blocks:
        lo, hi = i * p.q_block, min(N, (i + 1) * p.q_block)
        mu, sizes, assign = kmeans_fp32(q[b, h, lo:hi], p.n_clusters, p.kmeans_iters)
        s = block_scores(mu, sizes, hi - lo, k[b, h], p.k_block, scale, p.bf16, dtype=dt)
        res[(b, h, i)] = {"mu": mu, "sizes": sizes, "assign": assign, "scores": s}
        scores[(b, h, i)] = s

    class _Rows:
        shape = (B, H, -(-N // p.q_block), nkb)

        def __getitem__(self, key):
            return scores[key]

    draws = sample_rows(_Rows(), p.density, seed, blocks)
    for key, dr in draws.items():
        res[key].update(dr)
        if with_attention:
            b, h, i = key
            lo, hi = i * p.q_block, min(N, (i + 1) * p.q_block)
            o, lse = sparse_ht_attention(q[b, h, lo:hi], k[b, h], v[b, h], dr["idx"], dr["weight"], p.k_block, scale,
                                         dtype=dt)
            res[key]["O"] = o
            res[key]["LSE"] = lse
    return res
