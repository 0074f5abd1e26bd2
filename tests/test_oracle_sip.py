"""Pins for the oracle's SIP sampler.

* A hand-worked water-filling example (derivation in tests/golden/sip_waterfill.txt).
* P5 invariants: capped iff t = 2^24; uncapped thresholds proportional to the
  quantised score; sum of inclusion probabilities equals the budget up to the
  floors; quantisation edge cases; budget rounding.
* P5 statistics: the keep frequency of every block over many seeds lies within
  a binomial 5-sigma band of t / 2^24.
"""

import os

import numpy as np
import pytest

from oracle.sip import SIP_ONE, budget, inclusion_thresholds, quantize_scores, sample_rows

HERE = os.path.dirname(os.path.abspath(__file__))


def _load_golden(name):
    examples = [{}]
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line == "---":
                examples.append({})
                continue
            key, rest = line.split("=", 1)
            examples[-1][key.strip()] = [float(t) if ("." in t or "e" in t) else int(t) for t in rest.split()]
    return examples


def test_waterfill_worked_examples():
    examples = _load_golden("sip_waterfill.txt")
    assert len(examples) == 3
    for g in examples:
        s = np.array(g["scores"], dtype=np.float32)
        K = budget(g["density"][0], s.size)
        assert K == g["budget"][0]
        w = quantize_scores(s)
        assert w.tolist() == g["quantised"]
        t = inclusion_thresholds(w, K)
        assert t.tolist() == g["thresholds"]
        if "weights" in g:
            omega = np.float32(SIP_ONE) / t.astype(np.float32)
            assert omega.tolist() == [float(x) for x in g["weights"]]


def test_quantize_edges():
    s = np.array([0.0, -1.0, np.nan, 1e-30, 2.0**-24, 0.5, 1.0, 1.5, np.inf, np.float32(1) - np.float32(2**-24)], dtype=np.float32)
    w = quantize_scores(s)
    assert w.tolist() == [1, 1, 1, 1, 1, 2**23, 2**24, 2**24, 2**24, 2**24 - 1]


def test_budget_rounding():
    assert budget(1.0, 16) == 16
    assert budget(0.25, 16) == 4
    assert budget(0.10, 1024) == 102  # 102.4 + 0.5 -> 102
    assert budget(0.08, 2363) == 189  # 189.04
    assert budget(0.08, 7425) == 594  # 594.0
    assert budget(1e-9, 100) == 1
    assert budget(0.5, 3) == 2  # 1.5 + 0.5 = 2.0
    with pytest.raises(ValueError):
        budget(0.0, 10)
    with pytest.raises(ValueError):
        budget(1.5, 10)


def test_p5_threshold_invariants():
    rng = np.random.default_rng(0)
    for nkb, K, skew in [(16, 4, 1.0), (1024, 102, 3.0), (2363, 189, 4.0), (300, 299, 2.0), (50, 1, 0.5), (7, 7, 1.0)]:
        raw = rng.lognormal(0.0, skew, size=(8, nkb))
        s = (raw / raw.sum(axis=1, keepdims=True)).astype(np.float32)
        w = quantize_scores(s)
        t = inclusion_thresholds(w, K).astype(np.int64)
        assert t.min() >= 1 and t.max() <= SIP_ONE
        for r in range(8):
            capped = t[r] == SIP_ONE
            pi_sum = t[r].sum() / SIP_ONE
            assert K - nkb / SIP_ONE <= pi_sum <= K + 1e-12
            if K == nkb:
                assert capped.all()
                continue
            unc = ~capped
            m = int(capped.sum())
            S = int(w[r][unc].sum())
            # every capped block has weight >= every uncapped block
            if capped.any() and unc.any():
                assert w[r][capped].min() >= w[r][unc].max()
            # uncapped: t = floor((K - m) w 2^24 / S), and strictly below 1
            ref = np.maximum(((K - m) * w[r][unc].astype(object) * SIP_ONE) // S, 1).astype(np.int64)
            np.testing.assert_array_equal(t[r][unc], ref)
            assert np.all((K - m) * w[r][unc].astype(np.int64) < S)


def test_p5_keep_frequency_matches_probability():
    rng = np.random.default_rng(1)
    nkb, K = 16, 4
    raw = rng.lognormal(0, 1.5, size=(2, nkb))
    s = (raw / raw.sum(axis=1, keepdims=True)).astype(np.float32)
    scores = s.reshape(1, 1, 2, nkb)
    seeds = 10000
    hits = np.zeros((2, nkb))
    counts = np.zeros((2, seeds))
    t = None
    for seed in range(seeds):
        out = sample_rows(scores, K / nkb, seed, [(0, 0, 0), (0, 0, 1)])
        for r in range(2):
            o = out[(0, 0, r)]
            hits[r, o["idx"]] += 1
            counts[r, seed] = o["count"]
            t = o["thresh"] if r == 1 else t
            if seed == 0 and r == 0:
                t0 = o["thresh"]
    for r, tr in ((0, t0), (1, t)):
        p = tr.astype(np.float64) / SIP_ONE
        freq = hits[r] / seeds
        sd = np.sqrt(p * (1 - p) / seeds)
        assert np.all(np.abs(freq - p) <= 5 * sd + 1e-12), (freq, p)
        # expected kept count is K
        assert abs(counts[r].mean() - p.sum()) < 5 * np.sqrt((p * (1 - p)).sum() / seeds)


def test_sample_outputs_consistent():
    rng = np.random.default_rng(2)
    raw = rng.lognormal(0, 2, size=(1, 2, 3, 70))
    s = (raw / raw.sum(axis=-1, keepdims=True)).astype(np.float32)
    out = sample_rows(s, 0.2, 99, [(0, h, i) for h in range(2) for i in range(3)])
    for (b, h, i), o in out.items():
        assert np.all(np.diff(o["idx"]) > 0)
        assert o["count"] == o["idx"].size
        bits = np.unpackbits(o["mask"].view(np.uint8), bitorder="little")[:70]
        assert np.array_equal(np.nonzero(bits)[0], o["idx"])
        np.testing.assert_array_equal(o["weight"], np.float32(SIP_ONE) / o["thresh"][o["idx"]].astype(np.float32))
    # different rows draw different streams
    assert not all(np.array_equal(out[(0, 0, 0)]["mask"], out[(0, h, i)]["mask"]) for h in range(2) for i in range(3) if (h, i) != (0, 0))
