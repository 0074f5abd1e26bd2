"""Exact-rational references for the clustering's fp32 arithmetic, and a k-means
input on which fused and separately rounded distance arithmetic disagree.

The clustering compares a query x with a centroid mu through
|mu|^2 - 2 x.mu: start at |mu|^2 (products rounded one by one, halving-tree sum
in groups of 64 dimensions, group sums left to right), then one fused
multiply-add acc = fl(x_k * (-2 mu_k) + acc) per dimension in ascending order.
The functions here compute every step with exact rationals and one rounding to
fp32 per step, independently of numpy's float arithmetic.

The block built by ``build`` (fp32 values: with bf16 queries and bf16 initial
centroids every product is exact in fp32 and the two arithmetics agree) makes
the rounding decide an assignment: the two
initial centroids (rows 0 and 32 of a 64-row block, the strided initialisation
for two clusters) differ only by a swap of two coordinates, and row ROW equals
itself in those two coordinates, so x.a == x.b exactly and only rounding tells
the two comparisons apart. A seeded search keeps the first candidate whose
first assignment under the fused chain differs from the one under separately
rounded multiplies and adds, both computed here with exact rationals.

Only inputs and those two alternative choices come from here; the expected
assignment in the tests is the oracle's.
"""

from fractions import Fraction

import numpy as np

N_ROWS, ROW = 64, 5
SWAP = (3, 40)


def round_f32(q):
    """Exact rational -> nearest float32, ties to the even mantissa."""
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        err = abs(Fraction(float(c)) - q)
        key = (err, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def fma_exact(a, b, c):
    """fl(a*b + c) with one rounding, from exact rationals."""
    return round_f32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def sqnorm_exact(mu):
    """|mu|^2 by the clustering's rule, every step rounded from exact rationals."""
    d = len(mu)
    G = -(-d // 64)
    t = [round_f32(Fraction(float(m)) * Fraction(float(m))) for m in mu] + [np.float32(0.0)] * (G * 64 - d)
    sums = []
    for g in range(G):
        v = t[64 * g:64 * g + 64]
        s = 32
        while s >= 1:
            for k in range(s):
                v[k] = round_f32(Fraction(float(v[k])) + Fraction(float(v[k + s])))
            s //= 2
        sums.append(v[0])
    out = sums[0]
    for g in sums[1:]:
        out = round_f32(Fraction(float(out)) + Fraction(float(g)))
    return out


def distance_fused(x, mu):
    """|mu|^2 - 2 x.mu with one fused multiply-add per dimension (the specification)."""
    acc = sqnorm_exact(mu)
    for k in range(len(x)):
        acc = fma_exact(x[k], np.float32(-2.0) * np.float32(mu[k]), acc)
    return acc


def distance_separate(x, mu):
    """The same chain with the multiply and the add rounded separately."""
    acc = sqnorm_exact(mu)
    for k in range(len(x)):
        prod = round_f32(Fraction(float(x[k])) * Fraction(float(np.float32(-2.0) * np.float32(mu[k]))))
        acc = round_f32(Fraction(float(acc)) + Fraction(float(prod)))
    return acc


def _screen(xs, a, b, dim):
    """Vectorised first pass: per candidate row and centroid, the difference between
    a float64-then-fp32 chain (nearly always the fused result) and the separately
    rounded one. Both start from 0 here (the norms are common to both arithmetics);
    candidates are confirmed with exact rationals afterwards."""
    res = []
    for mu in (a, b):
        m2 = (np.float32(-2.0) * mu).astype(np.float32)
        sep = np.zeros(len(xs), dtype=np.float32)
        fus = np.zeros(len(xs), dtype=np.float32)
        for k in range(dim):
            sep = (sep + (xs[:, k] * m2[k]).astype(np.float32)).astype(np.float32)
            fus = (xs[:, k].astype(np.float64) * np.float64(m2[k]) + fus.astype(np.float64)).astype(np.float32)
        res.append((sep, fus))
    (s0, f0), (s1, f1) = res
    return f0 - s0, f1 - s1


def build(dim=64, seed=7):
    """Return (X float32 [64, dim], row, fused choice, separate choice)."""
    rng = np.random.default_rng(seed)
    i, j = SWAP
    for _ in range(400):
        a = rng.standard_normal(dim).astype(np.float32)
        if a[i] == a[j]:
            continue
        b = a.copy()
        b[i], b[j] = a[j], a[i]
        xs = rng.standard_normal((512, dim)).astype(np.float32)
        xs[:, j] = xs[:, i]
        da, db = _screen(xs, a, b, dim)
        # rows whose two chains round differently for at least one of the centroids
        for r in np.nonzero((da != 0) | (db != 0))[0][:16]:
            x = xs[r]
            fa, fb = distance_fused(x, a), distance_fused(x, b)
            sa, sb = distance_separate(x, a), distance_separate(x, b)
            fused_choice = 0 if fa <= fb else 1
            sep_choice = 0 if sa <= sb else 1
            if fused_choice != sep_choice:
                X = (3.0 * rng.standard_normal((N_ROWS, dim))).astype(np.float32)
                X[0], X[N_ROWS // 2], X[ROW] = a, b, x
                return X, ROW, fused_choice, sep_choice
    raise RuntimeError("no distinguishing candidate found")
