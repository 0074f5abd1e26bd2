"""Pins of the oracle's systematic sampler (oracle/systematic.py): a hand-worked draw,
inclusion probabilities equal to t_j / 2^24 exactly (every value of the row uniform
enumerated), a nearly fixed count, and the row uniform against an independent Philox."""

import numpy as np
import pytest

from oracle import philox4x32_10
from oracle.sip import SIP_ONE, inclusion_thresholds, quantize_scores
from oracle.systematic import keep_systematic, points_below, row_uniform24, sample_rows_systematic


def test_hand_worked_draw():
    # thresholds of the SIP golden example A (s = 1/2, 1/4, 1/8, 1/16, 1/16 at density 0.6):
    # t = 2^24, 2^24, 2^23, 2^22, 2^22; prefix C = 0, 2^24, 2^25, 2^25 + 2^23, 2^25 + 2^23 + 2^22.
    # With U = 2^23 + 5 the points are U, U + 2^24, U + 2^25 = 2^25 + 2^23 + 5: the first lies in
    # block 0's interval [0, 2^24), the second in block 1's, the third in block 3's
    # [2^25 + 2^23, 2^25 + 2^23 + 2^22), and block 2's [2^25, 2^25 + 2^23) holds none.
    t = np.array([1 << 24, 1 << 24, 1 << 23, 1 << 22, 1 << 22], dtype=np.uint32)
    keep = keep_systematic(t, (1 << 23) + 5)
    assert np.nonzero(keep)[0].tolist() == [0, 1, 3]
    # U = 0: points 0, 2^24, 2^25 -> blocks 0, 1, 2
    assert np.nonzero(keep_systematic(t, 0))[0].tolist() == [0, 1, 2]
    # U = 2^24 - 1: points end on the last unit of blocks 0, 1 and at 2^25 + 2^24 - 1 in block 4
    assert np.nonzero(keep_systematic(t, SIP_ONE - 1))[0].tolist() == [0, 1, 4]


def test_points_below():
    assert points_below(0, 0) == 0 and points_below(1, 0) == 1
    assert points_below(SIP_ONE, 0) == 1 and points_below(SIP_ONE + 1, 0) == 2
    assert points_below(7, 7) == 0 and points_below(8, 7) == 1


@pytest.mark.parametrize("seed", [1, 2])
def test_inclusion_probabilities_are_exact(seed):
    """Over all 2^24 values of U, block j is kept exactly t_j times."""
    rng = np.random.default_rng(seed)
    s = rng.random(7).astype(np.float32)
    s /= s.sum()
    t = inclusion_thresholds(quantize_scores(s), 3).astype(np.int64)
    c = np.concatenate([[0], np.cumsum(t)[:-1]])
    U = np.arange(SIP_ONE, dtype=np.int64)
    hits = np.zeros(t.size, dtype=np.int64)
    counts = np.zeros(SIP_ONE, dtype=np.int64)
    for j in range(t.size):
        kj = points_below(c[j] + t[j], U[:, None])[:, 0] > points_below(c[j], U[:, None])[:, 0]
        hits[j] = kj.sum()
        counts += kj
    assert np.array_equal(hits, t)
    T = int(t.sum())
    assert set(np.unique(counts).tolist()) <= {T // SIP_ONE, T // SIP_ONE + 1}


def test_row_uniform_counter():
    seed = 0x1234567890ABCDEF
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)
    want = int(philox4x32_10(np.array([[0xFFFFFFFF, 5, 3, 1]], dtype=np.uint32), key)[0, 0]) >> 8
    assert row_uniform24(seed, 1, 3, 5) == want < SIP_ONE


def test_rows_dict_and_density_one():
    rng = np.random.default_rng(0)
    sc = rng.random((1, 2, 3, 50)).astype(np.float32)
    out = sample_rows_systematic(sc, 1.0, 9, [(0, 1, 2)])[(0, 1, 2)]
    assert out["count"] == 50 and np.all(out["weight"] == 1.0)
    out = sample_rows_systematic(sc, 0.2, 9, [(0, 0, 0), (0, 1, 1)])
    for o in out.values():
        assert o["count"] in (9, 10)  # T is 10 * 2^24 up to the floors of the thresholds
        assert np.all(np.diff(o["idx"]) > 0)
        bits = np.unpackbits(o["mask"].view(np.uint8), bitorder="little")[:50]
        assert np.array_equal(np.nonzero(bits)[0], o["idx"])
