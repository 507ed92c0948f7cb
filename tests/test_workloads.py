"""The seeded input builders that both the oracle and the HIP path consume."""
import numpy as np
import pytest

from workloads import batch_share, make_workload


def _pages(w, b):
    n = (int(w.cache_seqlens[b]) + w.page_block_size - 1) // w.page_block_size
    return [w.kv[w.block_table[b, j]] for j in range(n)]


def test_batch_shares_partition_the_batch():
    w = make_workload(seqlens=[300, 1, 0, 64, 65, 700, 128, 5], num_heads_q=16, seed=4, extra_pages=3)
    shares = [batch_share(w, 4, i) for i in range(4)]
    assert np.array_equal(np.concatenate([s.cache_seqlens for s in shares]), w.cache_seqlens)
    assert np.array_equal(np.concatenate([s.q_bits for s in shares]), w.q_bits)
    for i, s in enumerate(shares):
        assert s.batch == 2
        # only the share's own blocks, each once
        assert s.num_blocks == max(1, int(s.nblk().sum()))
        for b in range(s.batch):
            got, want = _pages(s, b), _pages(w, 2 * i + b)
            assert len(got) == len(want) and all(np.array_equal(x, y) for x, y in zip(got, want))


def test_batch_share_of_one_is_the_workload():
    w = make_workload(seqlens=[100, 3], num_heads_q=16, seed=5)
    s = batch_share(w, 1)
    assert np.array_equal(s.cache_seqlens, w.cache_seqlens) and np.array_equal(s.q_bits, w.q_bits)
    for b in range(w.batch):
        assert all(np.array_equal(x, y) for x, y in zip(_pages(s, b), _pages(w, b)))


@pytest.mark.parametrize("n,index", [(3, 0), (0, 0), (2, 2), (2, -1)])
def test_batch_share_rejects_uneven_or_missing_shares(n, index):
    w = make_workload(seqlens=[10, 20, 30, 40], num_heads_q=16, seed=6)
    with pytest.raises(ValueError):
        batch_share(w, n, index)
