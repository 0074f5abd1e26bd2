"""SIP: sampling with inclusion-probability weighting (oracle side).

AB-Attention abstract (paperdot search page, query "Xing Ma"), SIP sentence:
blocks are drawn with probabilities proportional to the IBCS estimates and
each kept block carries weight 1/pi_j, pi_j its inclusion probability; the
weighted single pass is then an unbiased (Horvitz-Thompson) estimate of the
dense softmax numerator and denominator, where dropping the unkept blocks
would bias both. The pages fix neither the
sampling design nor the budget. Readings used here, all in integer arithmetic
on the fp32 scores so that any correct implementation reproduces them bit for
bit:

* Quantise: w_j = max(1, floor(s_j * 2^24)); NaN or non-positive scores give 1
  and scores >= 1 give 2^24. The floor of 1 keeps every inclusion probability
  positive, which the inverse-probability estimate needs.
* Budget: the target density rho is the expected kept fraction of key
  sub-blocks per query block, K = clamp(floor(rho * NKB + 0.5), 1, NKB) in fp64.
* Inclusion probabilities proportional to w, capped at 1, summing to K (the
  standard water-filling for probability-proportional-to-size designs): grow
  a capped set until no uncapped block has (K - m) * w_j >= S, where m is the
  capped count and S the uncapped weight total; capped blocks get
  t_j = 2^24, the rest t_j = max(1, floor((K - m) * w_j * 2^24 / S)). The
  inclusion probability is exactly pi_j = t_j / 2^24.
* Draw: independent Bernoulli trials (Poisson sampling). Word (j mod 4) of
  Philox4x32-10 with key (seed mod 2^32, seed >> 32) and counter
  (floor(j/4), i, h, b), shifted right by 8, is a 24-bit uniform u_j; block j
  is kept iff u_j < t_j.
* Weight: omega_j = fp32(2^24) / fp32(t_j), one correctly rounded division;
  capped blocks get exactly 1.
* No extra rules: no always-kept diagonal block, no sink tokens, no per-row
  minimum (the pages name none). A row may therefore keep nothing.
"""

import math

import numpy as np

from .philox import philox4x32_10

SIP_ONE = 1 << 24  # probability 1 in 24-bit fixed point


def quantize_scores(s):
    """w = max(1, floor(s * 2^24)) as uint64, on fp32 scores (any shape)."""
    s = np.asarray(s, dtype=np.float32)
    v = s * np.float32(SIP_ONE)  # exact: scaling by a power of two
    with np.errstate(invalid="ignore"):
        pos = s > 0
        ge1 = s >= 1
    fl = np.floor(np.where(pos & ~ge1, v, np.float32(1.0))).astype(np.uint64)
    w = np.where(ge1, np.uint64(SIP_ONE), np.maximum(fl, np.uint64(1)))
    return w.astype(np.uint64)


def budget(density, nkb):
    """K = clamp(floor(rho * NKB + 0.5), 1, NKB), evaluated in fp64."""
    density = float(density)
    if not (0.0 < density <= 1.0):
        raise ValueError("density must lie in (0, 1]")
    t = density * float(nkb)
    t = t + 0.5
    return int(min(max(math.floor(t), 1), nkb))


def inclusion_thresholds(w, K):
    """Integer water-filling. w: uint64 [rows, NKB]; K: int. Returns uint32 thresholds t."""
    w = np.asarray(w, dtype=np.uint64)
    squeeze = w.ndim == 1
    if squeeze:
        w = w[None]
    rows, nkb = w.shape
    one = np.uint64(SIP_ONE)
    if K >= nkb:
        t = np.full((rows, nkb), SIP_ONE, dtype=np.uint32)
        return t[0] if squeeze else t
    capped = np.zeros((rows, nkb), dtype=bool)
    while True:
        m = capped.sum(axis=1).astype(np.uint64)
        S = np.where(capped, np.uint64(0), w).sum(axis=1, dtype=np.uint64)
        room = np.uint64(K) - m
        new = (~capped) & (room[:, None] * w >= S[:, None])
        if not new.any():
            break
        capped |= new
    num = room[:, None] * w * one  # < 2^61
    t_unc = np.maximum(num // S[:, None], np.uint64(1))
    t = np.where(capped, one, t_unc).astype(np.uint32)
    return t[0] if squeeze else t


def uniforms24(seed, b, h, i, nkb):
    """24-bit uniforms u_j for j in [0, NKB) of row (b, h, i), uint32 [NKB]."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)
    groups = -(-nkb // 4)
    ctr = np.zeros((groups, 4), dtype=np.uint32)
    ctr[:, 0] = np.arange(groups, dtype=np.uint32)
    ctr[:, 1] = i
    ctr[:, 2] = h
    ctr[:, 3] = b
    x = philox4x32_10(ctr, key).reshape(-1)[:nkb]
    return x >> np.uint32(8)


def sample_rows(scores, density, seed, rows):
    """SIP on a set of rows of the score matrix.

    scores: float32 [B, H, NQB, NKB] (or any array indexable by (b, h, i)).
    rows: iterable of (b, h, i). Returns a dict keyed by (b, h, i) with
    'count' (int), 'idx' (int32 ascending), 'weight' (float32, aligned with idx),
    'thresh' (uint32 [NKB]) and 'mask' (uint32 bit words, bit j%32 of word j//32).
    """
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
        u = uniforms24(seed, b, h, i, nkb)
        keep = u < t[r]
        idx = np.nonzero(keep)[0].astype(np.int32)
        wgt = (np.float32(SIP_ONE) / t[r, idx].astype(np.float32)).astype(np.float32)
        bits = np.zeros(words * 32, dtype=np.uint64)
        bits[:nkb] = keep
        mask = (bits.reshape(words, 32) << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
        out[(b, h, i)] = {"count": int(idx.size), "idx": idx, "weight": wgt, "thresh": t[r], "mask": mask}
    return out
