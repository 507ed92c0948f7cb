"""Pins of the split-KV schedule rule (the oracle side of the scheduler).

The pages fix only the table shapes (FlashMLA interface page, docstring of
get_mla_metadata); the rule is ours.  It is pinned by the invariants any
correct schedule must meet (coverage exactly once and in order, per-part cost
bound, split counts, split-index bookkeeping), and the invariant checker is
itself pinned by planting mistakes in valid tables.
"""
import numpy as np
import pytest

from oracle import check_schedule, expand_splits, schedule
from workloads import make_config


def _cases():
    rng = np.random.default_rng(0)
    yield [127, 300], 4, 2
    yield [0], 1, 1
    yield [0, 0, 0], 8, 2
    yield [1] * 10, 3, 1
    yield [65536] + [512] * 31, 256, 3
    for _ in range(60):
        B = int(rng.integers(1, 40))
        L = rng.integers(0, 3000, size=B)
        L[rng.random(B) < 0.2] = 0
        yield L.tolist(), int(rng.integers(1, 300)), int(rng.integers(1, 6))


@pytest.mark.parametrize("L,parts,fc", list(_cases()))
def test_schedule_invariants(L, parts, fc):
    md, ns = schedule(L, parts, fc)
    assert check_schedule(md, ns, L, parts, fc)


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_schedule_on_config_lengths(cfg):
    L = make_config(cfg).cache_seqlens if cfg != 4 else make_config(4).cache_seqlens
    for parts in (1, 7, 64, 256, 1024):
        md, ns = schedule(L, parts, 2)
        check_schedule(md, ns, L, parts, 2)
        W = int(md[0, 5])
        total = int(sum(-(-int(x) // 64) for x in L)) + 2 * len(L)
        assert W == -(-total // parts)


def test_single_part_takes_everything_in_one_split_each():
    L = [5, 700, 0, 64]
    md, ns = schedule(L, 1, 2)
    assert ns.tolist() == [0, 1, 2, 3, 4]
    assert md.tolist() == [[0, 0, 3, 1, 0, 2 * 4 + 1 + 11 + 0 + 1, 2, 4]]
    assert expand_splits(md, L) == [(0, 0, 0, 0, 1), (0, 1, 0, 0, 11), (0, 2, 0, 0, 0), (0, 3, 0, 0, 1)]


def test_hand_worked_two_part_table():
    # Units (fixed_cost 1): b0 = [o, p0, p1], b1 = [o, p0, p1, p2, p3]; total 8,
    # W = 4: part 0 owns b0 whole and b1's overhead unit (no page of b1), part 1
    # owns b1's pages 0..3.
    md, ns = schedule([128, 256], 2, 1)
    assert ns.tolist() == [0, 1, 2]
    assert md.tolist() == [[0, 0, 0, 2, 0, 4, 1, 1], [1, 0, 1, 4, 0, 4, 1, 1]]
    # Three parts: boundaries floor(p * 8 / 3) = 0, 2, 5, 8.  Part 0 = units
    # 0-1 (b0's overhead, page 0); part 1 = units 2-4 (b0's page 1, b1's
    # overhead and page 0); part 2 = units 5-7 (b1's pages 1-3).
    md, ns = schedule([128, 256], 3, 1)
    assert ns.tolist() == [0, 2, 4]
    assert md.tolist() == [[0, 0, 0, 1, 0, 3, 1, 1], [0, 1, 1, 1, 1, 3, 1, 2], [1, 1, 1, 4, 1, 3, 1, 1]]
    # More parts than units: boundaries floor(p * 2 / 5) = 0, 0, 0, 1, 1, 2, so
    # part 2 owns the overhead unit (no page: it does not work on b0), part 4
    # owns page 0, and the others own nothing.
    md, ns = schedule([64], 5, 1)
    assert ns.tolist() == [0, 1]
    assert [r[0] for r in md.tolist()] == [-1, -1, -1, -1, 0]


def test_hand_worked_overhead_before_and_after_pages():
    # fixed_cost 2: one overhead unit before a sequence's pages and one after.
    # Units: b0 = [o, p0, p1, o], b1 = [o, p0, p1, p2, p3, o]; total 10.
    # Two parts (boundaries 0, 5, 10): part 0 owns b0 whole and b1's leading
    # unit (no page of b1); part 1 owns b1's pages and its trailing unit.
    md, ns = schedule([128, 256], 2, 2)
    assert ns.tolist() == [0, 1, 2]
    assert md.tolist() == [[0, 0, 0, 2, 0, 5, 2, 1], [1, 0, 1, 4, 0, 5, 2, 1]]
    # Three parts (boundaries 0, 3, 6, 10; W = 4): part 0 = b0's leading unit
    # and pages; part 1 = b0's trailing unit, b1's leading unit and page 0;
    # part 2 = b1's pages 1-3 and trailing unit.  b1 has two splits.
    md, ns = schedule([128, 256], 3, 2)
    assert ns.tolist() == [0, 1, 3]
    assert md.tolist() == [[0, 0, 0, 2, 0, 4, 2, 1], [1, 0, 1, 1, 0, 4, 2, 1], [1, 1, 1, 4, 1, 4, 2, 1]]


def test_uniform_lengths_split_evenly():
    # 128 sequences of 128 pages over 256 parts: with the overhead on both
    # sides of the pages every part gets exactly 64 pages.
    md, ns = schedule([8192] * 128, 256, 4)
    pages = [hi - lo for _, _, _, lo, hi in expand_splits(md, [8192] * 128)]
    assert len(pages) == 256 and set(pages) == {64}


def test_long_sequence_is_spread_over_many_parts():
    L = make_config(4).cache_seqlens
    md, ns = schedule(L, 256, 2)
    assert ns[1] - ns[0] > 100          # the 65536-token sequence is split widely


@pytest.mark.parametrize("mutation", ["drop_page", "dup_page", "bad_rank", "bad_count", "overload", "part_gap",
                                      "stray_row", "bad_nsplit"])
def test_checker_catches_planted_mistakes(mutation):
    L = [300, 129, 64, 1000]
    md, ns = schedule(L, 6, 2)
    md = md.copy()
    ns = ns.copy()
    cut = next(p for p in range(len(md)) if md[p, 4] > 0)      # a part starting mid-sequence
    if mutation == "drop_page":
        md[cut, 1] += 1
    elif mutation == "dup_page":
        md[cut, 1] -= 1
    elif mutation == "bad_rank":
        md[cut, 4] += 1
    elif mutation == "bad_count":
        ns[2:] += 1
    elif mutation == "overload":
        md[:, 5] = 1                      # claimed payload too small for the real costs
    elif mutation == "part_gap":
        md[cut - 1:cut + 1] = md[[cut, cut - 1]]    # two parts swapped
    elif mutation == "stray_row":
        md[-1] = [2, 0, 2, 1, 0, md[0, 5], 2, 1]
    elif mutation == "bad_nsplit":
        md[cut, 7] += 1
    with pytest.raises(AssertionError):
        check_schedule(md, ns, L, 6, 2)
