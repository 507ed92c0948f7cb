"""GPU parity on the five decode workloads at full size, invariances, and
special inputs.  Every case runs the HIP library through its C ABI and
compares with the fp64 oracle on the same bytes."""
import math

import numpy as np
import pytest
import torch

import mla_paged_kv_metadata_amd as mla
from oracle import bf16_bits_to_f64
from workloads import batch_share, bf16_bits_from_f32, make_config, make_workload

from gpu_util import compare, run_gpu, run_oracle, to_gpu

pytestmark = pytest.mark.gpu


def _sample(B, n, seed):
    if n >= B:
        return list(range(B))
    rng = np.random.default_rng(seed)
    return sorted(set([0, B - 1] + rng.choice(B, n, replace=False).tolist()))


@pytest.mark.parametrize("cfg,nsample", [(2, 64), (3, 24), (4, 32), (5, 16)])
def test_config_full_size(gpu_lib, cfg, nsample):
    print(f"config {cfg}: generating", flush=True)
    w = make_config(cfg)
    out, lse, md, ns = run_gpu(w)
    bs = _sample(w.batch, nsample, cfg)
    compare(w, out, lse, run_oracle(w, batches=bs), batches=bs, label=f"c{cfg} full size, batches {len(bs)}")


@pytest.mark.parametrize("cfg,n,nsample", [(2, 8, 8), (3, 8, 6), (5, 8, 4)])
def test_batch_share_of_one_gpu(gpu_lib, cfg, n, nsample):
    """One GPU's share of a batch split over n GPUs (its first B/n sequences
    and their blocks, on the default number of parts): few sequences over
    every compute unit, so each is cut into many short splits."""
    print(f"config {cfg} share 1/{n}: generating", flush=True)
    w = batch_share(make_config(cfg), n)
    out, lse, md, ns = run_gpu(w)
    assert int(ns[-1]) > 4 * w.batch                    # the case this covers: many splits per sequence
    bs = _sample(w.batch, nsample, cfg)
    compare(w, out, lse, run_oracle(w, batches=bs), batches=bs, label=f"c{cfg} share 1/{n}, batches {len(bs)}")


def test_config4_long_sequence_last(gpu_lib):
    w = make_config(4, seed=104, long_at_end=True)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label="c4 long at end")


@pytest.mark.parametrize("seed", [101, 102])
def test_fp8_small(gpu_lib, seed):
    w = make_workload(seqlens=[1, 64, 200, 1000], num_heads_q=128, kv_dtype="fp8_e4m3fn", seed=seed)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label=f"fp8 seed {seed}")


def test_fp8_causal_mtp(gpu_lib):
    w = make_workload(seqlens=[3, 129, 700], s_q=2, num_heads_q=64, causal=True, kv_dtype="fp8_e4m3fn", seed=7)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label="fp8 causal")


def test_page_placement_is_bitwise_invisible(gpu_lib):
    w = make_workload(seqlens=[700, 64, 3, 1290], num_heads_q=128, seed=41, extra_pages=5)
    out1, lse1, _, _ = run_gpu(w)
    nblk = w.nblk()
    order = np.concatenate([w.block_table[b, :nblk[b]] for b in range(w.batch)])
    kv2 = w.kv[order]                                   # contiguous pool, sequences in order
    bt2 = np.zeros_like(w.block_table)
    o = 0
    for b in range(w.batch):
        bt2[b, :nblk[b]] = np.arange(o, o + nblk[b])
        o += nblk[b]
    w2 = make_workload(seqlens=w.cache_seqlens, num_heads_q=128, seed=41, block_table=bt2, num_blocks=len(kv2))
    w2.q_bits, w2.kv = w.q_bits, kv2
    out2, lse2, _, _ = run_gpu(w2)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_repeat_runs_are_bitwise_equal(gpu_lib):
    w = make_config(2)
    t = to_gpu(w)
    a = run_gpu(w, tensors=t)
    b = run_gpu(w, tensors=t)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_poisoned_tail_rows_and_padding_do_not_matter(gpu_lib):
    w = make_workload(seqlens=[100, 65, 1, 64, 300], num_heads_q=64, seed=9, padding="zero")
    out1, lse1, _, _ = run_gpu(w)
    kv = w.kv.copy()
    bt = w.block_table.copy()
    for b in range(w.batch):
        L = int(w.cache_seqlens[b])
        n = -(-L // 64)
        if L % 64:
            kv[bt[b, n - 1], L % 64:] = 0x7FC0              # bf16 NaN in rows past the end
        bt[b, n:] = 0x7FFFFFF0                              # padding never read
    w.kv, w.block_table = kv, bt
    out2, lse2, _, _ = run_gpu(w)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_causal_two_queries_reduce_to_noncausal(gpu_lib):
    w = make_workload(seqlens=[1, 2, 65, 333], s_q=2, num_heads_q=16, causal=True, seed=12)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label="causal s_q=2")
    # query 0 of a length-1 sequence sees nothing
    assert (out[0, 0].float() == 0).all() and torch.isinf(lse[0, :, 0]).all() and (lse[0, :, 0] < 0).all()


def test_identical_keys_closed_form(gpu_lib):
    rng = np.random.default_rng(5)
    k = bf16_bits_from_f32(rng.standard_normal(576).astype(np.float32))
    w = make_workload(seqlens=[777], num_heads_q=32, seed=5)
    w.kv[:] = k
    out, lse, _, _ = run_gpu(w)
    kd = bf16_bits_to_f64(k)
    qd = bf16_bits_to_f64(w.q_bits[0, 0])
    ref_out = np.broadcast_to(kd[:512], (32, 512))
    ref_lse = math.log(777) + (qd @ kd) / 24.0
    assert np.abs(out[0, 0].float().cpu().numpy() - ref_out).max() <= 1e-2 * np.abs(ref_out).max() + 1e-3
    assert np.abs(lse[0, :, 0].cpu().numpy() - ref_lse).max() <= 2e-3


@pytest.mark.parametrize("H", [16, 64])
def test_late_scores_far_above_the_first_keys(gpu_lib, H):
    """A later key scores ~86 (base-2 units) above the first ones: exercises
    the re-run with a raised reference max (16 heads: two waves per page,
    one token tile each; 64 heads: one wave per 32 rows)."""
    w = make_workload(seqlens=[300, 150], num_heads_q=H, seed=21)
    w.q_bits[:] = 0
    w.q_bits[..., 0] = bf16_bits_from_f32(np.array([24.0 * 60.0], dtype=np.float32))[0]
    kv = np.zeros_like(w.kv)
    for b, t_big in [(0, 250), (1, 70)]:
        L = int(w.cache_seqlens[b])
        for t in range(L):
            page, r = w.block_table[b, t // 64], t % 64
            kv[page, r, 0, 1] = bf16_bits_from_f32(np.array([float(t % 7 - 3)], dtype=np.float32))[0]
        page, r = w.block_table[b, t_big // 64], t_big % 64
        kv[page, r, 0, 0] = bf16_bits_from_f32(np.array([1.0], dtype=np.float32))[0]
    w.kv = kv
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label="late large score")


def _e4m3_codes(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("H,parts", [(16, None), (64, None), (64, 1)])
def test_late_scores_far_above_the_first_keys_fp8(gpu_lib, H, parts):
    """The re-run with a raised reference max on the fp8 path, whose PV steps
    carry each page's second token tile into the next step: a key ~86 base-2
    units above the first ones on a middle page (unit scales)."""
    w = make_workload(seqlens=[300, 150, 600], num_heads_q=H, kv_dtype="fp8_e4m3fn", seed=22)
    w.k_scale, w.v_scale = 1.0, 1.0
    w.q_bits[:] = 0
    w.q_bits[..., 0] = bf16_bits_from_f32(np.array([24.0 * 60.0], dtype=np.float32))[0]
    w.q_bits[..., 1] = bf16_bits_from_f32(np.array([0.5], dtype=np.float32))[0]
    kv = np.zeros_like(w.kv)
    for b, t_big in [(0, 250), (1, 70), (2, 390)]:
        L = int(w.cache_seqlens[b])
        for t in range(L):
            page, r = w.block_table[b, t // 64], t % 64
            kv[page, r, 0, 1] = _e4m3_codes([float(t % 7 - 3)])[0]
            kv[page, r, 0, 2 + t % 500] = _e4m3_codes([float(t % 5 - 2) * 0.5])[0]
        page, r = w.block_table[b, t_big // 64], t_big % 64
        kv[page, r, 0, 0] = _e4m3_codes([1.0])[0]
    w.kv = kv
    out, lse, _, _ = run_gpu(w, num_parts=parts)
    compare(w, out, lse, run_oracle(w), label=f"fp8 late large score H={H} parts={parts}")
