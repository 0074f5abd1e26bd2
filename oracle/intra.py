"""INTRA's static relay patterns as kept-sub-block lists (oracle side).

INTRA page (paperdot search page, query "Wenbo Lu"; abstract): static sparse
attention whose patterns respect computational query sets (the queries computed
together share one key set), built from complementary sparse groups under a
partition model: Scatter forms relay groups that draw broadly across local
neighbourhoods, Gather reconnects those groups in a later layer, and the two
together reach every token. The abstract fixes no formula. Readings used here:

* The computational query set is the query block (rows [i*Bq, (i+1)*Bq)); keys are
  selected in key sub-blocks of Bk tokens, the unit the gather kernel loads.
* Partition model: the token sequence is cut into contiguous neighbourhoods of L
  tokens (L a multiple of Bq); token n lies in neighbourhood n // L at offset n % L.
* Scatter: query block i, at offsets [o_i, o_i + Bq) of its neighbourhood, attends
  to the keys at those same offsets in every neighbourhood (one slice of each:
  the relay group of offset o_i).
* Gather: query block i attends to every key of its own neighbourhood.
* Every kept sub-block has weight 1 (exact attention over the pattern); lists are
  ascending. A sub-block is kept when any of its real tokens is selected.

Scatter followed by Gather (or Gather by Scatter) connects every query token to
every key token when L divides N: that two-layer reachability is the property the
pins check. A partial last neighbourhood (N not a multiple of L) has no tokens at
its missing offsets, so the relay paths through them do not exist.
"""

import numpy as np


def default_partition(n_tokens, q_block):
    """L = q_block * ceil(sqrt(NQB)): both layers then keep about sqrt(q_block / N) of the keys."""
    nqb = -(-int(n_tokens) // int(q_block))
    return int(q_block) * int(np.ceil(np.sqrt(nqb)))


def intra_lists(n_tokens, q_block, k_block, partition, layer):
    """Kept sub-block lists of every query block for one INTRA layer.

    layer: "scatter" or "gather". Returns (idx int32 [NQB, NKB], weights float32
    [NQB, NKB], counts int32 [NQB]); the first counts[i] entries of row i are valid.
    """
    N, Bq, Bk, L = int(n_tokens), int(q_block), int(k_block), int(partition)
    if L < Bq or L % Bq:
        raise ValueError("the neighbourhood size must be a positive multiple of q_block")
    if layer not in ("scatter", "gather"):
        raise ValueError("layer is 'scatter' or 'gather'")
    nqb, nkb = -(-N // Bq), -(-N // Bk)
    idx = np.zeros((nqb, nkb), np.int32)
    wts = np.zeros((nqb, nkb), np.float32)
    cnt = np.zeros(nqb, np.int32)
    for i in range(nqb):
        p, o = divmod(i * Bq, L)
        if layer == "gather":
            first = p * L
            last = min(N, (p + 1) * L)  # exclusive token bound
            js = range(first // Bk, -(-last // Bk))
        else:
            js = []
            for q0 in range(0, N, L):  # start of every neighbourhood
                lo, hi = q0 + o, min(N, q0 + o + Bq)
                if lo >= N:
                    continue
                js.extend(range(lo // Bk, -(-hi // Bk)))
            js = sorted(set(js))
        js = list(js)
        cnt[i] = len(js)
        idx[i, :len(js)] = js
        wts[i, :len(js)] = 1.0
    return idx, wts, cnt


def token_mask(n_tokens, q_block, k_block, lists):
    """Query-token x key-token boolean mask of a layer's lists (each query token gets
    its block's list; each kept sub-block contributes its real tokens)."""
    idx, _, cnt = lists
    N = int(n_tokens)
    M = np.zeros((N, N), dtype=bool)
    for i in range(idx.shape[0]):
        rows = slice(i * q_block, min(N, (i + 1) * q_block))
        for j in idx[i, :cnt[i]]:
            M[rows, j * k_block:min(N, (j + 1) * k_block)] = True
    return M


def intra_row_order(n_tokens, q_block, partition, layer):
    """Processing order of one head's query blocks for the attention: Scatter blocks
    grouped by their offset (blocks of one offset share one list), within an offset
    by neighbourhood; Gather blocks in their natural order."""
    nqb = -(-int(n_tokens) // int(q_block))
    if layer == "gather":
        return np.arange(nqb, dtype=np.int32)
    U = int(partition) // int(q_block)
    return np.array([p * U + u for u in range(U) for p in range(-(-nqb // U)) if p * U + u < nqb], dtype=np.int32)
