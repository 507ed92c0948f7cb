"""Split-KV schedule, stated unit by unit -- TEST INFRASTRUCTURE ONLY.

The FlashMLA interface page (docstring of ``get_mla_metadata``) fixes only the
shapes: a (num_sm_parts, TileSchedulerMetaDataSize) int32 table "for the tile
scheduler" and num_splits of shape (batch + 1,) -- "splits per sample".  The
rule below is this repository's own, written here as a plain walk over cost
units so the GPU scheduler kernel can be compared with it bit for bit:

  * Sequence b costs ``fixed_cost`` overhead units and one unit per page,
    nblk_b = ceil(L_b / page), laid out as ceil(fixed_cost / 2) overhead
    units, the page units, then the other floor(fixed_cost / 2) overhead units
    (a split's overhead is its q load at the start and its result stores at
    the end).  Units of all sequences are laid end to end in batch order;
    total = sum_b (fixed_cost + nblk_b).
  * Part p owns units [floor(p * total / num_parts), floor((p+1) * total /
    num_parts)): parts differ by at most one unit and none is left idle
    while total >= num_parts.  W = ceil(total / num_parts) is the most units
    a part owns.
  * Part p works on sequence b if it owns at least one of b's page units, or,
    for a sequence with no pages, if it owns b's first overhead unit.  Each
    such (part, sequence) pair is one split of b; the splits of b are numbered
    k = 0, 1, ... in part order.
  * num_splits is the exclusive prefix sum of the split counts:
    num_splits[0] = 0, num_splits[b+1] - num_splits[b] >= 1.
  * The table has one row per part (num_parts rows of 8 int32).  A part works
    on a run of consecutive sequences b0..b1: its first split is split k0 of
    b0 over pages [first, nblk_b0) (or [first, end) when b0 == b1), the
    sequences strictly between are whole, and its last split covers pages
    [0, end) of b1.  Row p = [b0, first, b1, end, k0, W, fixed_cost, number of
    splits of the part].  A part with no split has [-1, 0, -1, 0, 0, W,
    fixed_cost, 0].
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
    lead = (fixed_cost + 1) // 2
    for b in range(B):
        units += [(b, -1)] * lead
        units += [(b, j) for j in range(nblk[b])]
        units += [(b, -1)] * (fixed_cost - lead)
    total = len(units)
    W = max(1, -(-total // num_parts))
    bounds = [p * total // num_parts for p in range(num_parts + 1)]
    owner = []
    for p in range(num_parts):
        owner += [p] * (bounds[p + 1] - bounds[p])
    pages = [dict() for _ in range(num_parts)]   # pages[p][b] = ordered pages of b owned by p
    first_seen = set()
    for u, (b, j) in enumerate(units):
        p = owner[u]
        if j >= 0:
            pages[p].setdefault(b, []).append(j)
        elif nblk[b] == 0 and b not in first_seen:
            pages[p].setdefault(b, [])
        first_seen.add(b)
    parts_of = [[p for p in range(num_parts) if b in pages[p]] for b in range(B)]
    num_splits = np.zeros(B + 1, dtype=np.int32)
    for b in range(B):
        num_splits[b + 1] = num_splits[b] + len(parts_of[b])
    md = np.zeros((num_parts, TILE_MD_INTS), dtype=np.int32)
    md[:] = [-1, 0, -1, 0, 0, W, fixed_cost, 0]
    for p in range(num_parts):
        seqs = sorted(pages[p])
        if not seqs:
            continue
        b0, b1 = seqs[0], seqs[-1]
        pg0, pg1 = pages[p][b0], pages[p][b1]
        first = pg0[0] if pg0 else 0
        end = pg1[-1] + 1 if pg1 else 0
        k0 = parts_of[b0].index(p)
        md[p] = [b0, first, b1, end, k0, W, fixed_cost, len(seqs)]
    return md, num_splits


def expand_splits(tile_md, cache_seqlens, page: int = 64):
    """Lists the splits a per-part table describes, in table order, as tuples
    (part, b, k, first page, end page).  Sequences strictly inside a part's
    run are whole; the run's first and last sequences are cut as the row says."""
    md = np.asarray(tile_md)
    L = [int(x) for x in cache_seqlens]
    out = []
    for p, r in enumerate(md):
        b0, first, b1, end, k0 = (int(x) for x in r[:5])
        if b0 < 0:
            continue
        for b in range(b0, b1 + 1):
            nblk = -(-L[b] // page)
            lo = first if b == b0 else 0
            hi = end if b == b1 else nblk
            out.append((p, b, k0 if b == b0 else 0, lo, hi))
    return out


def check_schedule(tile_md, num_splits, cache_seqlens, num_parts, fixed_cost, page=64):
    """Invariants any valid table must satisfy (raises AssertionError).

    Every page of every sequence is covered exactly once and in order by its
    splits, numbered k = 0, 1, ... in part order; every sequence gets >= 1
    split and num_splits counts them; total splits <= B + num_parts - 1; the
    parts of one sequence's splits increase with only idle parts between
    them; each part's real cost (its
    pages plus fixed_cost per sequence whose pages it touches) is at most
    W + fixed_cost; idle rows are empty; the split count field is right.
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
    assert int(ns[-1]) <= B + num_parts - 1
    W = int(md[0, 5])
    assert (md[:, 5] == W).all() and (md[:, 6] == fixed_cost).all()
    for r in md:
        if r[0] < 0:
            assert r.tolist() == [-1, 0, -1, 0, 0, W, fixed_cost, 0]
        else:
            assert 0 <= r[0] <= r[2] < B and r[7] == r[2] - r[0] + 1
    splits = expand_splits(md, L, page)
    seen = {b: [] for b in range(B)}
    ks = {b: [] for b in range(B)}
    parts = {b: [] for b in range(B)}
    cost = {}
    prev_b = -1
    for p, b, k, lo, hi in splits:
        assert b >= prev_b                # sequences appear in batch order
        prev_b = b
        assert 0 <= lo <= hi <= nblk[b], (p, b, lo, hi)
        assert hi > lo or nblk[b] == 0, (p, b, lo, hi)
        seen[b].extend(range(lo, hi))
        ks[b].append(k)
        parts[b].append(p)
        if hi > lo:
            cost[p] = cost.get(p, 0) + fixed_cost + (hi - lo)
    for b in range(B):
        assert seen[b] == list(range(nblk[b])), b
        assert ks[b] == list(range(counts[b])), (b, ks[b], counts[b])
        # a sequence's parts increase, and any part between two of them is idle
        for p0, p1 in zip(parts[b], parts[b][1:]):
            assert p1 > p0, (b, parts[b])
            assert all(md[q, 0] < 0 for q in range(p0 + 1, p1)), (b, parts[b])
    for p, c in cost.items():
        assert c <= W + fixed_cost, (p, c, W)
    return True
