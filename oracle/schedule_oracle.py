"""Split-KV schedule, stated unit by unit -- TEST INFRASTRUCTURE ONLY.

The FlashMLA interface page (docstring of ``get_mla_metadata``) fixes only the
shapes: a (num_sm_parts, TileSchedulerMetaDataSize) int32 table "for the tile
scheduler" and num_splits of shape (batch + 1,) -- "splits per sample".  The
rule below is this repository's own, written here as a plain walk over cost
units so the GPU scheduler kernel can be compared with it bit for bit:

  * Sequence b costs ``fixed_cost`` overhead units followed by one unit per
    page, nblk_b = ceil(L_b / page).  Units of all sequences are laid end to end
    in batch order; total = sum_b (fixed_cost + nblk_b).
  * Payload W = ceil(total / num_parts).  Unit u belongs to part u // W.
  * Part p works on sequence b if it owns at least one of b's page units, or,
    for a sequence with no pages, if it owns b's first overhead unit.  Each
    such (part, sequence) pair is one split of b; the splits of b are numbered
    k = 0, 1, ... in part order.
  * num_splits is the exclusive prefix sum of the split counts:
    num_splits[0] = 0, num_splits[b+1] - num_splits[b] >= 1.
  * The table has batch + num_parts - 1 rows (the most splits possible).  Row
    s = num_splits[b] + k describes split k of sequence b as 8 int32:
    [b, first page, end page (exclusive), k, split count of b, W, fixed_cost,
    part].  Rows past the last split are [-1, 0, 0, 0, 0, W, fixed_cost, -1].
"""
from __future__ import annotations

import numpy as np

TILE_MD_INTS = 8


def table_rows(batch: int, num_parts: int) -> int:
    return batch + num_parts - 1


def schedule(cache_seqlens, num_parts: int, fixed_cost: int, page: int = 64):
    """Returns (tile_md (batch + num_parts - 1, 8) int32, num_splits (B+1,) int32)."""
    L = [int(x) for x in cache_seqlens]
    B = len(L)
    if num_parts < 1 or fixed_cost < 1 or B < 1:
        raise ValueError("need num_parts >= 1, fixed_cost >= 1, batch >= 1")
    nblk = [-(-x // page) for x in L]
    units = []                                   # (b, page index or -1 for overhead)
    for b in range(B):
        units += [(b, -1)] * fixed_cost
        units += [(b, j) for j in range(nblk[b])]
    total = len(units)
    W = max(1, -(-total // num_parts))
    pages = [dict() for _ in range(num_parts)]   # pages[p][b] = ordered pages of b owned by p
    first_seen = set()
    for u, (b, j) in enumerate(units):
        p = u // W
        if j >= 0:
            pages[p].setdefault(b, []).append(j)
        elif nblk[b] == 0 and b not in first_seen:
            pages[p].setdefault(b, [])
        first_seen.add(b)
    parts_of = [[p for p in range(num_parts) if b in pages[p]] for b in range(B)]
    num_splits = np.zeros(B + 1, dtype=np.int32)
    for b in range(B):
        num_splits[b + 1] = num_splits[b] + len(parts_of[b])
    rows = table_rows(B, num_parts)
    md = np.zeros((rows, TILE_MD_INTS), dtype=np.int32)
    md[:] = [-1, 0, 0, 0, 0, W, fixed_cost, -1]
    for b in range(B):
        n = len(parts_of[b])
        for k, p in enumerate(parts_of[b]):
            pg = pages[p][b]
            first, end = (pg[0], pg[-1] + 1) if pg else (0, 0)
            md[num_splits[b] + k] = [b, first, end, k, n, W, fixed_cost, p]
    return md, num_splits


def check_schedule(tile_md, num_splits, cache_seqlens, num_parts, fixed_cost, page=64):
    """Invariants any valid table must satisfy (raises AssertionError).

    Every page of every sequence is covered exactly once and in order by its
    splits, which occupy consecutive rows starting at num_splits[b] with
    k = 0, 1, ...; the parts of one sequence's splits are consecutive; every
    sequence gets >= 1 split; total splits <= B + num_parts - 1; each part's
    real cost (its pages plus fixed_cost per sequence whose pages it touches)
    is at most W + fixed_cost; rows past the last split are empty.
    """
    md = np.asarray(tile_md)
    ns = np.asarray(num_splits)
    L = [int(x) for x in cache_seqlens]
    B = len(L)
    nblk = [-(-x // page) for x in L]
    rows = table_rows(B, num_parts)
    assert md.shape == (rows, TILE_MD_INTS)
    assert ns.shape == (B + 1,) and ns[0] == 0
    counts = np.diff(ns)
    assert (counts >= 1).all()
    total = int(ns[-1])
    assert total <= rows
    W = int(md[0, 5])
    assert (md[:, 5] == W).all() and (md[:, 6] == fixed_cost).all()
    cost = {}
    for b in range(B):
        seen = []
        parts = []
        for k in range(counts[b]):
            r = md[ns[b] + k]
            assert r[0] == b and r[3] == k and r[4] == counts[b], (b, k, r)
            assert 0 <= r[1] <= r[2] <= nblk[b]
            assert r[2] > r[1] or nblk[b] == 0
            seen.extend(range(r[1], r[2]))
            parts.append(int(r[7]))
            if r[2] > r[1]:
                cost[int(r[7])] = cost.get(int(r[7]), 0) + fixed_cost + int(r[2] - r[1])
        assert seen == list(range(nblk[b])), b
        assert parts == list(range(parts[0], parts[0] + len(parts))), (b, parts)
        assert all(0 <= p < num_parts for p in parts)
    for p, c in cost.items():
        assert c <= W + fixed_cost, (p, c, W)
    for r in md[total:]:
        assert r[0] == -1 and r[7] == -1
    return True
