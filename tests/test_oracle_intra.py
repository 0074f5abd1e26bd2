"""Pins for the INTRA relay patterns (oracle/intra.py).

* Token-level definitions, written independently of the list construction: a key
  token y is in query token x's Scatter set iff y sits at an offset of its
  neighbourhood that x's query block covers in its own; in x's Gather set iff it
  shares x's neighbourhood. The lists must give exactly these masks (sizes with
  Bk | Bq | L make the selection sub-block aligned), ragged sequence ends included.
* Global reachability of the two-layer relay, in both orders: every query token
  reaches every key token through one intermediate token when L divides N; with a
  partial last neighbourhood, exactly the paths through its missing offsets are lost.
* Counts: Scatter keeps Bq/Bk sub-blocks per neighbourhood, Gather L/Bk.
* Degenerate neighbourhoods: L >= N makes Gather dense and Scatter block-diagonal.
"""

import numpy as np
import pytest

from oracle.intra import default_partition, intra_lists, intra_row_order, token_mask

SHAPES = [
    # (N, Bq, Bk, L)
    (512, 64, 16, 128),
    (500, 64, 16, 128),   # ragged last neighbourhood and sub-block
    (777, 128, 32, 256),
    (1000, 64, 32, 320),
    (640, 128, 64, 384),
    (300, 64, 16, 64),    # L = Bq: Scatter keeps one block per neighbourhood, Gather the block itself
]


def _scatter_def(N, Bq, L):
    x = np.arange(N)
    o = ((x // Bq) * Bq) % L  # offset of x's query block in its neighbourhood
    y = np.arange(N) % L
    return (y[None, :] >= o[:, None]) & (y[None, :] < o[:, None] + Bq)


def _gather_def(N, Bq, L):
    x = np.arange(N)
    return ((x // Bq) * Bq // L)[:, None] == (np.arange(N) // L)[None, :]


@pytest.mark.parametrize("N,Bq,Bk,L", SHAPES)
def test_lists_match_token_definitions(N, Bq, Bk, L):
    for layer, ref in (("scatter", _scatter_def(N, Bq, L)), ("gather", _gather_def(N, Bq, L))):
        lists = intra_lists(N, Bq, Bk, L, layer)
        idx, wts, cnt = lists
        for i in range(idx.shape[0]):
            row = idx[i, :cnt[i]]
            assert np.all(np.diff(row) > 0), (layer, i)  # ascending, unique
            assert np.all(wts[i, :cnt[i]] == 1.0) and not wts[i, cnt[i]:].any()
        assert np.array_equal(token_mask(N, Bq, Bk, lists), ref), layer


@pytest.mark.parametrize("N,Bq,Bk,L", SHAPES + [(768, 64, 16, 256), (1024, 128, 32, 256)])
def test_two_layer_relay_reaches_every_token(N, Bq, Bk, L):
    S = token_mask(N, Bq, Bk, intra_lists(N, Bq, Bk, L, "scatter")).astype(np.int64)
    G = token_mask(N, Bq, Bk, intra_lists(N, Bq, Bk, L, "gather")).astype(np.int64)
    SG = (G @ S) > 0  # Scatter, then Gather: x -> z in x's neighbourhood -> y at z's offsets
    GS = (S @ G) > 0  # Gather, then Scatter: x -> z at x's offsets -> y in z's neighbourhood
    if N % L == 0:
        assert SG.all() and GS.all()
    else:
        # a partial last neighbourhood of r tokens has no tokens at offsets >= r, so
        # relay paths through those offsets do not exist: queries of the full
        # neighbourhoods still reach everything through Scatter then Gather, and
        # queries whose block offset exists in the last neighbourhood through Gather
        # then Scatter
        r = N % L
        x = np.arange(N)
        assert SG[x < N - r].all()
        assert GS[((x // Bq) * Bq) % L < r].all()
    # neither layer does it alone, unless a neighbourhood is the whole sequence
    # (Gather) or one query block wide (Scatter)
    if L < N:
        assert not G.all()
    if Bq < L:
        assert not S.all()


def test_counts_and_defaults():
    N, Bq, Bk = 32760, 128, 32
    L = default_partition(N, Bq)
    assert L == 128 * 16  # 256 query blocks -> 16 blocks a neighbourhood
    _, _, cs = intra_lists(N, Bq, Bk, L, "scatter")
    _, _, cg = intra_lists(N, Bq, Bk, L, "gather")
    nfull = N // L  # 15 full neighbourhoods and a partial one of 1960 tokens
    tail = N - nfull * L
    for i in range(len(cs)):
        o = (i * Bq) % L
        covered = nfull + (1 if o < tail else 0)
        assert cs[i] == covered * (Bq // Bk) - (1 if (o < tail < o + Bq) else 0) * ((o + Bq - tail) // Bk)
        p = (i * Bq) // L
        assert cg[i] == (L // Bk if p < nfull else -(-tail // Bk))


def test_whole_sequence_neighbourhood():
    N, Bq, Bk = 300, 64, 16
    L = 320  # >= N
    idx, _, cnt = intra_lists(N, Bq, Bk, L, "gather")
    nkb = -(-N // Bk)
    assert np.all(cnt == nkb)
    S = token_mask(N, Bq, Bk, intra_lists(N, Bq, Bk, L, "scatter"))
    blocks = (np.arange(N) // Bq)
    assert np.array_equal(S, blocks[:, None] == blocks[None, :])


def test_rejects_bad_partitions():
    with pytest.raises(ValueError):
        intra_lists(512, 64, 16, 96, "scatter")
    with pytest.raises(ValueError):
        intra_lists(512, 64, 16, 0, "gather")
    with pytest.raises(ValueError):
        intra_lists(512, 64, 16, 128, "relay")


@pytest.mark.parametrize("N,Bq,Bk,L", SHAPES + [(32760, 128, 32, 2048), (5000, 128, 16, 4096)])
def test_scatter_row_order_groups_shared_lists(N, Bq, Bk, L):
    """The Scatter processing order lists every query block once, and the blocks that
    share a list (equal offsets) form consecutive runs in ascending neighbourhood order."""
    order = intra_row_order(N, Bq, L, "scatter")
    nqb = -(-N // Bq)
    assert sorted(order.tolist()) == list(range(nqb))
    idx, _, cnt = intra_lists(N, Bq, Bk, L, "scatter")
    offs = (order * Bq) % L
    assert np.all(np.diff(offs) >= 0)  # runs of equal offset, offsets ascending
    for a, b in zip(order[:-1], order[1:]):
        if (a * Bq) % L == (b * Bq) % L:  # same run: next neighbourhood, same list
            assert b > a
            assert np.array_equal(idx[a, :cnt[a]], idx[b, :cnt[b]])
    assert np.array_equal(intra_row_order(N, Bq, L, "gather"), np.arange(nqb))
