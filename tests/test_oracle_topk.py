"""Pins of the oracle's top-K truncation (oracle/topk.py): hand-worked examples and
properties that hold for any row (exactly K kept, every kept quantised score at least
every dropped one, ties cut in index order, weights 1)."""

import os

import numpy as np
import pytest

from oracle import budget, quantize_scores, topk_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topk_truncation.txt")


def _cases():
    cases, cur = [], {}
    for line in open(GOLDEN):
        line = line.strip()
        if line.startswith("#") or not line:
            continue
        if line == "---":
            cases.append(cur)
            cur = {}
            continue
        k, v = (x.strip() for x in line.split("=", 1))
        cur[k] = v
    if cur:
        cases.append(cur)
    return cases


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["scores"])
def test_topk_golden(case):
    s = np.array([float(x) for x in case["scores"].split()], dtype=np.float32)
    res = topk_rows(s.reshape(1, 1, 1, -1), float(case["density"]), [(0, 0, 0)])[(0, 0, 0)]
    want = np.array([int(x) for x in case["idx"].split()], dtype=np.int32)
    assert np.array_equal(res["idx"], want)
    assert res["count"] == want.size
    assert np.all(res["weight"] == 1.0)
    bits = np.unpackbits(res["mask"].view(np.uint8), bitorder="little")[: s.size]
    assert np.array_equal(np.nonzero(bits)[0], want)


@pytest.mark.parametrize("nkb", [1, 7, 64, 300, 1037])
def test_topk_properties(nkb):
    rng = np.random.default_rng(nkb)
    for trial in range(20):
        # coarse values so that ties are common
        s = (rng.integers(0, 6, size=nkb) / 8.0).astype(np.float32)
        rho = float(rng.choice([0.02, 0.1, 0.3, 0.77, 1.0]))
        res = topk_rows(s.reshape(1, 1, 1, -1), rho, [(0, 0, 0)])[(0, 0, 0)]
        K = budget(rho, nkb)
        idx = res["idx"]
        assert idx.size == K == res["count"]
        assert np.all(np.diff(idx) > 0)
        w = quantize_scores(s).astype(np.int64)
        kept = np.zeros(nkb, bool)
        kept[idx] = True
        if K < nkb:
            assert w[kept].min() >= w[~kept].max()
            cut = w[kept].min()
            tied = np.nonzero(w == cut)[0]
            n_above = int((w > cut).sum())
            # the tied blocks that are kept are the lowest-indexed ones
            assert np.array_equal(np.nonzero(kept & (w == cut))[0], tied[: K - n_above])
