"""More GPU parity cases through the C ABI against the fp64 oracle: every
workload at the parity seeds 101-103, the scale-0 closed form, grouped KV
heads with several row tiles, and the optional inputs of mla_decode_fwd_ext
(device-held scales, split cache and query) checked directly against the
oracle rather than only against another HIP path."""
import numpy as np
import pytest
import torch

import mla_paged_kv_metadata_amd as mla
from oracle import bf16_bits_to_f64, decode_kv, gather_rows
from oracle import mla_decode as oracle_decode
from workloads import make_config, make_workload

from gpu_util import DV, compare, run_gpu, run_oracle, scales, to_gpu

pytestmark = pytest.mark.gpu


def _sample(B, n, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, B - 1] + rng.choice(B, min(n, B), replace=False).tolist()))


@pytest.mark.parametrize("seed", [101, 102, 103])
@pytest.mark.parametrize("cfg,nsample", [(2, 12), (3, 6), (4, 8), (5, 6)])
def test_configs_at_parity_seeds(gpu_lib, cfg, nsample, seed):
    print(f"config {cfg} seed {seed}: generating", flush=True)
    w = make_config(cfg, seed)
    out, lse, _, _ = run_gpu(w)
    bs = _sample(w.batch, nsample, seed)
    compare(w, out, lse, run_oracle(w, batches=bs), batches=bs, label=f"c{cfg} seed {seed}")


@pytest.mark.parametrize("kv_dtype,causal,s_q", [("bf16", False, 1), ("bf16", True, 2), ("fp8_e4m3fn", False, 1)])
@pytest.mark.parametrize("parts", [1, 24])
def test_scale_zero_is_the_mean_of_visible_values(gpu_lib, kv_dtype, causal, s_q, parts):
    """softmax_scale = 0: out is the plain mean of the visible V rows (times
    v_scale) and lse = ln n, whatever q holds (closed form P6)."""
    w = make_workload(seqlens=[1, 63, 64, 65, 900, 2], s_q=s_q, num_heads_q=32, causal=causal, kv_dtype=kv_dtype,
                      seed=81)
    q, kv, bt, sl = to_gpu(w)
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, 1, num_parts=parts)
    vs = 0.5 if kv_dtype == "bf16" else w.v_scale
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=0.0, v_scale=vs, causal=causal)
    torch.cuda.synchronize()
    ref_o = np.zeros((w.batch, s_q, 32, DV))
    ref_l = np.full((w.batch, 32, s_q), -np.inf)
    for b in range(w.batch):
        L = int(w.cache_seqlens[b])
        rows = decode_kv(gather_rows(w.kv, w.block_table[b], L, 64), w.kv_dtype)[:, 0, :DV]
        for i in range(s_q):
            n = max(0, min(L, L - s_q + 1 + i)) if causal else L
            if n:
                ref_o[b, i] = vs * rows[:n].mean(axis=0)
                ref_l[b, :, i] = np.log(n)
    compare(w, out, lse, (ref_o, ref_l), label=f"scale 0 {kv_dtype} causal={causal} parts={parts}")
    compare(w, out, lse, oracle_decode(w.q_bits, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, 0.0,
                                       causal, vs), label="scale 0 vs oracle")


@pytest.mark.parametrize("H,s_q,causal", [(256, 1, False), (256, 2, True), (128, 1, False)])
def test_grouped_kv_heads_with_several_row_tiles(gpu_lib, H, s_q, causal):
    """Two KV heads: 128 or 256 query rows per KV head, so whole 128-row tiles
    (whose q rows are staged through LDS) exist for both KV heads, with one or
    more tiles per head."""
    w = make_workload(seqlens=[700, 1, 130, 2000], s_q=s_q, num_heads_q=H, num_heads_k=2, causal=causal,
                      seed=H + s_q)
    out, lse, _, _ = run_gpu(w)
    compare(w, out, lse, run_oracle(w), label=f"H_k=2 H={H} s_q={s_q}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("parts", [1, 32])
def test_device_scales_match_the_oracle(gpu_lib, kv_dtype, parts):
    w = make_workload(seqlens=[500, 1, 2000, 64], num_heads_q=128, kv_dtype=kv_dtype, seed=59)
    q, kv, bt, sl = to_gpu(w)
    s1, s2 = scales(w)
    s1, s2 = s1 * 1.3, s2 * 0.75          # scales other than the defaults, so a dropped scale shows
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, 1, num_parts=parts)
    b1 = torch.tensor([s1], dtype=torch.float32, device="cuda")
    b2 = torch.tensor([s2], dtype=torch.float32, device="cuda")
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=9.0, v_scale=3.0,
                                  bmm1_scale_tensor=b1, bmm2_scale_tensor=b2)
    torch.cuda.synchronize()
    ref = oracle_decode(w.q_bits, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV,
                        float(np.float32(s1)), False, float(np.float32(s2)))
    compare(w, out, lse, ref, label=f"device scales {kv_dtype} parts={parts}")


@pytest.mark.parametrize("kv_dtype,causal,s_q,bs", [("bf16", False, 1, 64), ("bf16", True, 2, 32),
                                                    ("fp8_e4m3fn", False, 1, 64)])
def test_split_cache_and_query_match_the_oracle(gpu_lib, kv_dtype, causal, s_q, bs):
    w = make_workload(seqlens=[1, 64, 65, 777, 0, 300], s_q=s_q, num_heads_q=64, causal=causal,
                      kv_dtype=kv_dtype, seed=47, page_block_size=bs)
    q, kv, bt, sl = to_gpu(w)
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, 1, num_parts=8)
    s1, s2 = scales(w)
    out, lse = mla.mla_decode_fwd(q[..., :DV].contiguous(), kv[..., :DV].contiguous(), bt, sl, DV, md, ns,
                                  softmax_scale=s1, v_scale=s2, causal=causal, kv_rope=kv[..., DV:].contiguous(),
                                  q_rope=q[..., DV:].contiguous())
    torch.cuda.synchronize()
    compare(w, out, lse, run_oracle(w), label=f"split cache/query {kv_dtype} bs={bs}")


@pytest.mark.parametrize("bad", [float("nan"), -1.0, float("inf")])
@pytest.mark.parametrize("parts", [1, 16])
def test_invalid_device_bmm1_gives_nan(gpu_lib, bad, parts):
    """A device-held bmm1 scale cannot be checked on the host: a NaN, negative
    or infinite value turns every output row into NaN (out and lse) instead of
    a plausible finite result."""
    w = make_workload(seqlens=[300, 5, 1200], num_heads_q=64, seed=83)
    q, kv, bt, sl = to_gpu(w)
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, 1, num_parts=parts)
    b1 = torch.tensor([bad], dtype=torch.float32, device="cuda")
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, bmm1_scale_tensor=b1)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()


def test_lds_dma_read_calibration_runs(gpu_lib):
    """The counter-calibration read (mla_lds_dma_read) runs on sizes that do
    and do not fill its grid, and refuses a size that is not whole KiB."""
    for kib in (1, 3, 4096, 65536):
        src = torch.ones(kib * 1024, dtype=torch.uint8, device="cuda")
        mla.lds_dma_read(src)
    torch.cuda.synchronize()
    with pytest.raises(mla.MlaError):
        mla.lds_dma_read(torch.ones(1000, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("H,s_q,causal", [(1, 1, False), (16, 1, False), (20, 1, False), (32, 1, False),
                                          (16, 2, True), (8, 3, True)])
@pytest.mark.parametrize("parts", [1, 64])
def test_two_waves_per_page_for_few_rows(gpu_lib, H, s_q, causal, parts):
    """At most 32 rows per workgroup: two waves take the two token tiles of
    every page and merge their states at the end of each split.  Lengths put
    the last visible key in either tile, leave tile 1 empty (L <= 32) and
    cut splits mid-sequence (64 parts)."""
    w = make_workload(seqlens=[1, 31, 32, 33, 63, 64, 65, 700, 0, 4000, 97], s_q=s_q, num_heads_q=H,
                      causal=causal, seed=107 + H)
    out, lse, _, _ = run_gpu(w, num_parts=parts)
    compare(w, out, lse, run_oracle(w), label=f"few rows H={H} s_q={s_q} parts={parts}")


@pytest.mark.parametrize("kv_dtype,num_heads_k,parts", [("bf16", 1, None), ("fp8_e4m3fn", 1, None), ("bf16", 2, 16)])
def test_the_most_rows_per_kv_head(gpu_lib, kv_dtype, num_heads_k, parts):
    """s_q x heads per KV head at the boundary's limit (1024 rows: eight
    128-row tiles per KV head, MTP with 8 query tokens, causal), on the
    default and on few parts."""
    H = 128 * num_heads_k
    w = make_workload(seqlens=[700, 9, 1500], s_q=8, num_heads_q=H, num_heads_k=num_heads_k, causal=True,
                      kv_dtype=kv_dtype, seed=81 + num_heads_k)
    assert w.heads_per_head_k == 1024
    out, lse, _, _ = run_gpu(w, num_parts=parts)
    compare(w, out, lse, run_oracle(w), label=f"1024 rows {kv_dtype} H_k={num_heads_k}")
