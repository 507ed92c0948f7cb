"""GPU parity of the optional decode inputs (mla_decode_fwd_ext): per-head
attention sinks and device-held fused scales (FlashInfer MLA page), and the
split cache / split query layouts (Ascend ATB MLA page), through the C ABI."""
import numpy as np
import pytest
import torch

import mla_paged_kv_metadata_amd as mla
from oracle import mla_decode as oracle_decode
from workloads import make_config, make_workload

from gpu_util import DV, compare, scales, to_gpu

pytestmark = pytest.mark.gpu


def _run(w, t, parts=None, **kw):
    q, kv, bt, sl = t
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, w.num_heads_k, num_parts=parts)
    s1, s2 = scales(w)
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=s1, causal=w.causal, v_scale=s2, **kw)
    torch.cuda.synchronize()
    return out, lse


def _oracle(w, sinks=None, batches=None):
    s1, s2 = scales(w)
    return oracle_decode(w.q_bits, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, s1, w.causal, s2,
                         batches=batches, sinks=sinks)


# One-split sequences apply the sink in the decode kernel, split sequences in
# the combine: 1 part puts every sequence in one split; 64 parts split the long ones.
@pytest.mark.parametrize("parts", [1, 64])
@pytest.mark.parametrize("kv_dtype,causal,s_q,H", [("bf16", False, 1, 128), ("bf16", True, 2, 16),
                                                   ("fp8_e4m3fn", False, 1, 64)])
def test_sinks_match_oracle(gpu_lib, parts, kv_dtype, causal, s_q, H):
    w = make_workload(seqlens=[0, 1, 65, 700, 2000, 130], s_q=s_q, num_heads_q=H, causal=causal,
                      kv_dtype=kv_dtype, seed=41 + H)
    sinks = np.linspace(-2.0, 6.0, H).astype(np.float32)
    t = to_gpu(w)
    out, lse = _run(w, t, parts, sinks=torch.from_numpy(sinks).cuda())
    compare(w, out, lse, _oracle(w, sinks.astype(np.float64)), label=f"sinks {kv_dtype} parts={parts}")


def test_sinks_of_minus_inf_are_bitwise_no_sinks(gpu_lib):
    w = make_workload(seqlens=[900, 3, 0, 1500], num_heads_q=128, seed=43)
    t = to_gpu(w)
    o1, l1 = _run(w, t, 16)
    o2, l2 = _run(w, t, 16, sinks=torch.full((128,), float("-inf"), device="cuda"))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_sinks_full_size_sampled(gpu_lib):
    """The standard B=64 H=128 decode in its default launch configuration, checked
    on three whole sequences."""
    w = make_config(2)
    sinks = np.linspace(-1.0, 3.0, 128).astype(np.float32)
    out, lse = _run(w, to_gpu(w), sinks=torch.from_numpy(sinks).cuda())
    bs = [0, 31, 63]
    compare(w, out, lse, _oracle(w, sinks.astype(np.float64), batches=bs), batches=bs, label="c2 sinks")


@pytest.mark.parametrize("kv_dtype,causal,s_q", [("bf16", False, 1), ("bf16", True, 2), ("fp8_e4m3fn", False, 1)])
@pytest.mark.parametrize("split_q", [False, True])
def test_split_cache_and_query_are_bitwise_the_joined_layout(gpu_lib, kv_dtype, causal, s_q, split_q):
    w = make_workload(seqlens=[1, 64, 65, 777, 0, 300], s_q=s_q, num_heads_q=64, num_heads_k=1, causal=causal,
                      kv_dtype=kv_dtype, seed=47)
    q, kv, bt, sl = to_gpu(w)
    o1, l1 = _run(w, (q, kv, bt, sl), 8)
    kv_nope, kv_rope = kv[..., :DV].contiguous(), kv[..., DV:].contiguous()
    kw = {"kv_rope": kv_rope}
    qq = q
    if split_q:
        qq = q[..., :DV].contiguous()
        kw["q_rope"] = q[..., DV:].contiguous()
    o2, l2 = _run(w, (qq, kv_nope, bt, sl), 8, **kw)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_query_alone_and_grouped_heads(gpu_lib):
    w = make_workload(seqlens=[400, 90, 5], num_heads_q=32, num_heads_k=2, seed=53)
    q, kv, bt, sl = to_gpu(w)
    o1, l1 = _run(w, (q, kv, bt, sl), 4)
    o2, l2 = _run(w, (q[..., :DV].contiguous(), kv, bt, sl), 4, q_rope=q[..., DV:].contiguous())
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    kv_nope, kv_rope = kv[..., :DV].contiguous(), kv[..., DV:].contiguous()
    o3, l3 = _run(w, (q, kv_nope, bt, sl), 4, kv_rope=kv_rope)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_device_scales_are_bitwise_the_host_scales(gpu_lib, kv_dtype):
    w = make_workload(seqlens=[500, 1, 2000], num_heads_q=128, kv_dtype=kv_dtype, seed=59)
    t = to_gpu(w)
    s1, s2 = scales(w)
    if kv_dtype == "bf16":
        s2 = 0.75                       # a bmm2 scale other than 1 exercises the combine's copy too
    q, kv, bt, sl = t
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, 1, num_parts=32)
    o1, l1 = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=s1, v_scale=s2)
    b1 = torch.tensor([s1], dtype=torch.float32, device="cuda")
    b2 = torch.tensor([s2], dtype=torch.float32, device="cuda")
    o2, l2 = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=123.0, v_scale=9.0,
                                bmm1_scale_tensor=b1, bmm2_scale_tensor=b2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_ext_stages_equal_the_whole_call(gpu_lib):
    w = make_workload(seqlens=[1200, 7, 0, 2500], num_heads_q=128, seed=61)
    q, kv, bt, sl = to_gpu(w)
    md, ns = mla.mla_get_metadata(sl, 128, 1, num_parts=24)
    sinks = torch.linspace(-1.0, 2.0, 128, device="cuda")
    o1, l1 = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, sinks=sinks)
    ws = torch.empty((mla.mla_workspace_bytes(w.batch, 1, 128, 1, DV, 24),), dtype=torch.uint8, device="cuda")
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, sinks=sinks, out=o2, lse=l2, workspace=ws, stage="splits")
    mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, sinks=sinks, out=o2, lse=l2, workspace=ws, stage="combine")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
