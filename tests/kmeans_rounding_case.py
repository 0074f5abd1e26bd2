"""A k-means input on which separately rounded and fused distance arithmetic disagree.

The clustering is specified with a separately rounded multiply and add per
term: distance = (((0 + e_0) + e_1) + ...) with e_k = fl(fl(x_k - mu_k)^2). A
fused multiply-add, acc = fl(t * t + acc), rounds once per term instead of
twice, which is a different function. The block built here makes that
difference decide an assignment: the two initial centroids (rows 0 and 32 of a
64-row block, the strided initialisation for two clusters) differ only by a
swap of two coordinates, and row ROW equals itself in those two coordinates,
so its two distances are equal in exact arithmetic and only the rounding of
the running sums tells them apart. A seeded search keeps the first candidate
whose first assignment differs between the two arithmetics, checked with exact
rational arithmetic.

Only inputs come from here; the expected assignment is the oracle's.
"""

from fractions import Fraction

import numpy as np

N_ROWS, ROW = 64, 5
SWAP = (3, 40)


def _bf16(x):
    """Round float32 values to bfloat16 (nearest, ties to even), kept as float32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _round_f32(q):
    """Exact rational -> nearest float32, ties to even mantissa."""
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(c)) - q)
        key = (err, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def distance_separate(x, mu):
    acc = np.float32(0.0)
    for k in range(len(x)):
        t = np.float32(x[k] - mu[k])
        acc = np.float32(acc + np.float32(t * t))
    return acc


def distance_fused(x, mu):
    acc = np.float32(0.0)
    for k in range(len(x)):
        t = np.float32(x[k] - mu[k])
        acc = _round_f32(Fraction(float(t)) * Fraction(float(t)) + Fraction(float(acc)))
    return acc


def _screen(xs, a, b, dim):
    """Vectorised first pass: (separate d0 <= d1, fused-by-fp64 d0 <= d1) per candidate row."""
    res = []
    for mu in (a, b):
        sep = np.zeros(len(xs), dtype=np.float32)
        fus = np.zeros(len(xs), dtype=np.float32)
        for k in range(dim):
            t = (xs[:, k] - mu[k]).astype(np.float32)
            sep = (sep + (t * t).astype(np.float32)).astype(np.float32)
            t64 = t.astype(np.float64)
            fus = (t64 * t64 + fus.astype(np.float64)).astype(np.float32)
        res.append((sep, fus))
    (s0, f0), (s1, f1) = res
    return s0 <= s1, f0 <= f1


def build(dim=64, seed=7):
    """Return (X float32 [64, dim] of bfloat16 values, row, separate choice, fused choice)."""
    rng = np.random.default_rng(seed)
    i, j = SWAP
    for _ in range(200):
        a = _bf16(rng.standard_normal(dim).astype(np.float32))
        if a[i] == a[j]:
            continue
        b = a.copy()
        b[i], b[j] = a[j], a[i]
        xs = _bf16(rng.standard_normal((512, dim)).astype(np.float32))
        xs[:, j] = xs[:, i]
        sep_le, fus_le = _screen(xs, a, b, dim)
        for r in np.nonzero(sep_le != fus_le)[0]:
            x = xs[r]
            d0s, d1s = distance_separate(x, a), distance_separate(x, b)
            d0f, d1f = distance_fused(x, a), distance_fused(x, b)
            sep_choice = 0 if d0s <= d1s else 1
            fus_choice = 0 if d0f <= d1f else 1
            if sep_choice != fus_choice:
                X = _bf16(3.0 * rng.standard_normal((N_ROWS, dim)).astype(np.float32))
                X[0], X[N_ROWS // 2], X[ROW] = a, b, x
                return X, ROW, sep_choice, fus_choice
    raise RuntimeError("no distinguishing candidate found")
