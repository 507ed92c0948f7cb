"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded bytes, at the stated tolerances."""
import numpy as np
import pytest
import torch

from oracle import check_schedule, schedule
from workloads import make_config, make_workload

from gpu_util import compare, run_gpu, run_oracle, to_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [1, 101, 102, 103])
def test_config1_tiny(gpu_lib, seed):
    w = make_config(1, seed)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label=f"c1 seed {seed}")


@pytest.mark.parametrize("L", [[1], [64], [65], [127, 300], [0, 5], [1, 0, 63, 64, 65, 129, 700]])
def test_lengths_and_page_edges(gpu_lib, L):
    w = make_workload(seqlens=L, num_heads_q=16, seed=sum(L) + 7)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label=f"L={L}")


@pytest.mark.parametrize("H,s_q,causal", [(128, 1, False), (20, 1, False), (64, 2, True), (128, 2, True),
                                          (16, 3, True), (96, 3, True)])
def test_head_layouts(gpu_lib, H, s_q, causal):
    w = make_workload(seqlens=[2, 70, 500, 1], s_q=s_q, num_heads_q=H, causal=causal, seed=H + s_q)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label=f"H={H} s_q={s_q} causal={causal}")


def test_grouped_kv_heads(gpu_lib):
    w = make_workload(seqlens=[300, 64, 5], num_heads_q=32, num_heads_k=2, seed=5)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label="H_k=2")


def test_config2_full(gpu_lib):
    w = make_config(2)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label="c2 full")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("parts", [1, 7, 64, 256, 1024])
def test_split_count_does_not_change_result(gpu_lib, parts, kv_dtype):
    """Any split count (down to one page per split, where an fp8 split's PV
    steps are its first page's and the closing one only) gives the oracle's
    result."""
    w = make_workload(seqlens=[3000, 65, 1, 1800, 640], num_heads_q=128, kv_dtype=kv_dtype, seed=31)
    out, lse, md, ns = run_gpu(w, num_parts=parts)
    compare(w, out, lse, run_oracle(w), label=f"parts={parts} {kv_dtype}")


@pytest.mark.parametrize("parts,fc", [(1, 1), (7, 2), (256, 9), (300, 3)])
def test_scheduler_kernel_matches_schedule_rule(gpu_lib, parts, fc):
    L = make_config(4).cache_seqlens.copy()
    L[3] = 0
    w = make_workload(seqlens=L, num_heads_q=16, seed=3)
    sl = torch.from_numpy(w.cache_seqlens).cuda()
    import mla_paged_kv_metadata_amd as mla
    md, ns = mla.mla_get_metadata(sl, 16, 1, num_parts=parts, fixed_cost=fc)
    assert md.shape == (parts, 8)
    torch.cuda.synchronize()
    ref_md, ref_ns = schedule(w.cache_seqlens, parts, fc)
    assert np.array_equal(ns.cpu().numpy(), ref_ns)
    assert np.array_equal(md.cpu().numpy(), ref_md)
    check_schedule(md.cpu().numpy(), ns.cpu().numpy(), w.cache_seqlens, parts, fc)


@pytest.mark.parametrize("parts", [1100, 3])
def test_scheduler_kernel_on_huge_lengths(gpu_lib, parts):
    """About 2.1M page units: times 1100 parts that passes 2^31 (the kernel's
    64-bit path); 3 parts stays on the 32-bit path.  The table needs only
    cache_seqlens, so no cache is allocated."""
    L = np.array([1 << 24] * 7 + [5, 0, (1 << 24) + 1, 64], dtype=np.int32)
    sl = torch.from_numpy(L).cuda()
    import mla_paged_kv_metadata_amd as mla
    md, ns = mla.mla_get_metadata(sl, 128, 1, num_parts=parts, fixed_cost=4)
    torch.cuda.synchronize()
    ref_md, ref_ns = schedule(L, parts, 4)
    assert np.array_equal(ns.cpu().numpy(), ref_ns)
    assert np.array_equal(md.cpu().numpy(), ref_md)


@pytest.mark.parametrize("B,parts,fc", [(65, 256, 4), (129, 256, 2), (300, 97, 4), (5000, 256, 3), (8192, 1024, 4)])
def test_scheduler_kernel_on_large_batches(gpu_lib, B, parts, fc):
    """Batches past one wave (65, 129), past one value per thread (300 over
    256 threads) and up to the batch limit: the block scans cross waves and
    chunks; the table must still be the schedule rule's, bit for bit."""
    rng = np.random.default_rng(B)
    L = rng.integers(0, 9000, size=B).astype(np.int32)
    L[rng.integers(0, B, size=max(1, B // 10))] = 0
    sl = torch.from_numpy(L).cuda()
    import mla_paged_kv_metadata_amd as mla
    md, ns = mla.mla_get_metadata(sl, 128, 1, num_parts=parts, fixed_cost=fc)
    torch.cuda.synchronize()
    ref_md, ref_ns = schedule(L, parts, fc)
    assert np.array_equal(ns.cpu().numpy(), ref_ns)
    assert np.array_equal(md.cpu().numpy(), ref_md)
