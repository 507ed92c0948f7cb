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
  * Part p takes part in sequence b if it owns at least one of b's page units,
    or, for a sequence with no pages, if it owns b's first overhead unit.
  * num_splits is the exclusive prefix sum of the number of parts taking part
    in each sequence: num_splits[0] = 0, num_splits[b+1] - num_splits[b] >= 1.
  * Table row of part p (8 int32): [begin_b, begin_page, end_b (inclusive),
    end_page (exclusive, within end_b), index of p among the parts of begin_b,
    W, fixed_cost, 0].  A part with no work has begin_b = B, end_b = B - 1.
"""
from __future__ import annotations

import numpy as np

TILE_MD_INTS = 8


def schedule(cache_seqlens, num_parts: int, fixed_cost: int, page: int = 64):
    """Returns (tile_md (num_parts, 8) int32, num_splits (B+1,) int32)."""
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
    # pages[p][b] = ordered page list of sequence b owned by part p
    pages = [dict() for _ in range(num_parts)]
    first_unit_seen = set()
    for u, (b, j) in enumerate(units):
        p = u // W
        if j >= 0:
            pages[p].setdefault(b, []).append(j)
        elif nblk[b] == 0 and b not in first_unit_seen:
            pages[p].setdefault(b, [])
        first_unit_seen.add(b)
    parts_of = [[] for _ in range(B)]
    for p in range(num_parts):
        for b in sorted(pages[p]):
            parts_of[b].append(p)
    num_splits = np.zeros(B + 1, dtype=np.int32)
    for b in range(B):
        num_splits[b + 1] = num_splits[b] + len(parts_of[b])
    md = np.zeros((num_parts, TILE_MD_INTS), dtype=np.int32)
    for p in range(num_parts):
        seqs = sorted(pages[p])
        if not seqs:
            md[p] = [B, 0, B - 1, 0, 0, W, fixed_cost, 0]
            continue
        b0, b1 = seqs[0], seqs[-1]
        begin_page = pages[p][b0][0] if pages[p][b0] else 0
        end_page = pages[p][b1][-1] + 1 if pages[p][b1] else 0
        md[p] = [b0, begin_page, b1, end_page, parts_of[b0].index(p), W, fixed_cost, 0]
    return md, num_splits


def check_schedule(tile_md, num_splits, cache_seqlens, num_parts, fixed_cost, page=64):
    """Invariants any valid table must satisfy (raises AssertionError).

    Every page of every sequence is processed exactly once and in order, by
    consecutive parts; every sequence gets >= 1 split and the split count is
    what num_splits says; a part's recorded index within its first sequence is
    its rank there; total splits <= B + num_parts - 1; each part's real cost
    (its pages plus fixed_cost per sequence whose pages it touches) is at most
    W + fixed_cost.
    """
    md = np.asarray(tile_md)
    ns = np.asarray(num_splits)
    L = [int(x) for x in cache_seqlens]
    B = len(L)
    nblk = [-(-x // page) for x in L]
    assert md.shape == (num_parts, TILE_MD_INTS)
    assert ns.shape == (B + 1,) and ns[0] == 0
    counts = np.diff(ns)
    assert (counts >= 1).all()
    assert ns[-1] <= B + num_parts - 1
    seen = [[] for _ in range(B)]
    parts_of = [[] for _ in range(B)]
    W = int(md[0, 5])
    for p in range(num_parts):
        b0, pg0, b1, pg1, k0, w, fc = (int(v) for v in md[p, :7])
        assert w == W and fc == fixed_cost
        if b0 > b1:
            continue
        cost = 0
        for b in range(b0, b1 + 1):
            lo = pg0 if b == b0 else 0
            hi = pg1 if b == b1 else nblk[b]
            assert 0 <= lo <= hi <= nblk[b]
            assert hi > lo or nblk[b] == 0
            seen[b].extend(range(lo, hi))
            parts_of[b].append(p)
            if hi > lo:                   # an empty sequence only needs its zero output written
                cost += fixed_cost + (hi - lo)
        assert k0 == parts_of[b0].index(p)
        assert cost <= W + fixed_cost, (p, cost, W)
    for b in range(B):
        assert seen[b] == list(range(nblk[b])), b
        assert len(parts_of[b]) == counts[b]
        assert parts_of[b] == list(range(parts_of[b][0], parts_of[b][0] + len(parts_of[b])))
    return True
