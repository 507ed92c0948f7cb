"""GPU parity of the fp8-side inputs of mla_decode_fwd_ext: an e4m3 query whose
q_scale is folded into bmm1 and the base-2 device scale (FlashInfer MLA page,
note on fused scales and its device-scale form), and per-head qkDescale /
pvDescale (Ascend ATB MLA page, parameter table), each against the oracle."""
import numpy as np
import pytest
import torch

import mla_paged_kv_metadata_amd as mla
from oracle import fused_fp8_scales
from oracle import mla_decode as oracle_decode
from workloads import fp8_query, make_config, make_workload

from gpu_util import DV, compare, scales, to_gpu

pytestmark = pytest.mark.gpu

LOG2E = np.float32(1.4426950408889634)


def _meta(w, sl, parts):
    return mla.mla_get_metadata(sl, w.heads_per_head_k, w.num_heads_k, num_parts=parts)


def _fp8_q(w, seed):
    codes, q_scale = fp8_query(w, seed)
    qt = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).cuda()
    return codes, q_scale, qt


@pytest.mark.parametrize("parts", [1, 32])
@pytest.mark.parametrize("causal,s_q,H", [(False, 1, 128), (True, 2, 64), (False, 1, 16)])
def test_fp8_query_with_fp8_cache_matches_oracle(gpu_lib, parts, causal, s_q, H):
    w = make_workload(seqlens=[0, 1, 65, 700, 2000, 130], s_q=s_q, num_heads_q=H, causal=causal,
                      kv_dtype="fp8_e4m3fn", seed=61 + H)
    codes, q_scale, qt = _fp8_q(w, 62 + H)
    _, kv, bt, sl = to_gpu(w)
    s1, s2 = fused_fp8_scales(q_scale=q_scale, k_scale=w.k_scale, v_scale=w.v_scale, head_dim_qk=w.head_dim)
    s1 = float(np.float32(s1))
    md, ns = _meta(w, sl, parts)
    out, lse = mla.mla_decode_fwd(qt, kv, bt, sl, DV, md, ns, softmax_scale=s1, causal=causal, v_scale=s2)
    torch.cuda.synchronize()
    ref = oracle_decode(codes, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, s1, causal, s2,
                        q_format="fp8_e4m3fn")
    compare(w, out, lse, ref, label=f"fp8 q causal={causal} s_q={s_q} H={H} parts={parts}")


def test_fp8_query_full_size_sampled(gpu_lib):
    """The B=128 L=8192 fp8-cache decode with an e4m3 query, default launch
    configuration, checked on three whole sequences."""
    w = make_config(5)
    codes, q_scale, qt = _fp8_q(w, 71)
    _, kv, bt, sl = to_gpu(w)
    s1, s2 = fused_fp8_scales(q_scale=q_scale, k_scale=w.k_scale, v_scale=w.v_scale, head_dim_qk=w.head_dim)
    s1 = float(np.float32(s1))
    md, ns = _meta(w, sl, None)
    out, lse = mla.mla_decode_fwd(qt, kv, bt, sl, DV, md, ns, softmax_scale=s1, v_scale=s2)
    torch.cuda.synchronize()
    bs = [0, 64, 127]
    ref = oracle_decode(codes, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, s1, False, s2,
                        batches=bs, q_format="fp8_e4m3fn")
    compare(w, out, lse, ref, batches=bs, label="c5 fp8 q")


def test_fp8_query_with_bf16_cache_is_refused(gpu_lib):
    w = make_workload(seqlens=[100, 3], num_heads_q=16, seed=73)
    _, kv, bt, sl = to_gpu(w)
    _, _, qt = _fp8_q(w, 74)
    md, ns = _meta(w, sl, 4)
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_fwd(qt, kv, bt, sl, DV, md, ns)
    assert e.value.status == mla.MLA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("parts", [1, 32])
@pytest.mark.parametrize("which", ["qk", "pv", "both"])
def test_per_head_descales_match_oracle(gpu_lib, kv_dtype, parts, which):
    """Per-head factors on the scores and on the output; parts=1 keeps each
    sequence in one split (decode epilogue), 32 splits the long ones
    (combine)."""
    H = 128
    w = make_workload(seqlens=[500, 1, 2000, 64, 0, 1300], num_heads_q=H, kv_dtype=kv_dtype, seed=79)
    q, kv, bt, sl = to_gpu(w)
    s1, s2 = scales(w)
    rng = np.random.default_rng(80)
    qk = rng.uniform(0.25, 2.5, H).astype(np.float32) if which in ("qk", "both") else None
    pv = rng.uniform(0.1, 3.0, H).astype(np.float32) if which in ("pv", "both") else None
    if qk is not None:
        qk[5] = 0.0                                    # a head with flat attention
    md, ns = _meta(w, sl, parts)
    kw = {}
    if qk is not None:
        kw["qk_descale"] = torch.from_numpy(qk).cuda()
    if pv is not None:
        kw["pv_descale"] = torch.from_numpy(pv).cuda()
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=s1, v_scale=s2, **kw)
    torch.cuda.synchronize()
    ref = oracle_decode(w.q_bits, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, s1, False, s2,
                        qk_descale=None if qk is None else qk.astype(np.float64),
                        pv_descale=None if pv is None else pv.astype(np.float64))
    compare(w, out, lse, ref, label=f"descale {which} {kv_dtype} parts={parts}")


def test_descales_with_fp8_query_and_sinks_match_oracle(gpu_lib):
    H = 64
    w = make_workload(seqlens=[900, 17, 0, 2500], s_q=2, num_heads_q=H, causal=True, kv_dtype="fp8_e4m3fn",
                      seed=83)
    codes, q_scale, qt = _fp8_q(w, 84)
    _, kv, bt, sl = to_gpu(w)
    s1, s2 = fused_fp8_scales(q_scale=q_scale, k_scale=w.k_scale, v_scale=w.v_scale, head_dim_qk=w.head_dim)
    s1 = float(np.float32(s1))
    rng = np.random.default_rng(85)
    qk = rng.uniform(0.5, 2.0, H).astype(np.float32)
    pv = rng.uniform(0.5, 2.0, H).astype(np.float32)
    sinks = np.linspace(-1.0, 4.0, H).astype(np.float32)
    for parts in (1, 16):
        md, ns = _meta(w, sl, parts)
        out, lse = mla.mla_decode_fwd(qt, kv, bt, sl, DV, md, ns, softmax_scale=s1, causal=True, v_scale=s2,
                                      qk_descale=torch.from_numpy(qk).cuda(), pv_descale=torch.from_numpy(pv).cuda(),
                                      sinks=torch.from_numpy(sinks).cuda())
        torch.cuda.synchronize()
        ref = oracle_decode(codes, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, s1, True, s2,
                            sinks=sinks.astype(np.float64), q_format="fp8_e4m3fn",
                            qk_descale=qk.astype(np.float64), pv_descale=pv.astype(np.float64))
        compare(w, out, lse, ref, label=f"fp8 q + descales + sinks parts={parts}")


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
@pytest.mark.parametrize("parts", [1, 32])
def test_log2_scale_tensor_is_bitwise_the_bmm1_tensor(gpu_lib, kv_dtype, parts):
    """bmm1_scale_log2 = fp32(bmm1 * log2 e) gives the same bits as the plain
    device bmm1 (whose log2 form the kernel forms by the same fp32 product),
    and both match the oracle."""
    w = make_workload(seqlens=[500, 1, 2000, 64], num_heads_q=128, kv_dtype=kv_dtype, seed=89)
    q, kv, bt, sl = to_gpu(w)
    s1, s2 = scales(w)
    s1 = np.float32(s1 * 1.3)
    md, ns = _meta(w, sl, parts)
    b1 = torch.tensor([s1], dtype=torch.float32, device="cuda")
    b1l = torch.tensor([np.float32(s1 * LOG2E)], dtype=torch.float32, device="cuda")
    o1, l1 = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=7.0, v_scale=s2, bmm1_scale_tensor=b1)
    o2, l2 = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=7.0, v_scale=s2,
                                bmm1_scale_log2_tensor=b1l, bmm1_scale_tensor=torch.full_like(b1, 11.0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref = oracle_decode(w.q_bits, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, float(s1), False, s2)
    compare(w, o2, l2, ref, label=f"log2 scale {kv_dtype} parts={parts}")


@pytest.mark.parametrize("bad", [float("nan"), -1.0, float("inf")])
@pytest.mark.parametrize("parts", [1, 16])
def test_invalid_qk_descale_makes_its_head_nan(gpu_lib, bad, parts):
    """A qkDescale entry that is NaN, negative or infinite turns that head's
    out and lse into NaN; the other heads are bitwise those of a valid call."""
    H = 32
    w = make_workload(seqlens=[300, 5, 1200, 0], num_heads_q=H, seed=97)
    q, kv, bt, sl = to_gpu(w)
    md, ns = _meta(w, sl, parts)
    good = torch.ones(H, dtype=torch.float32, device="cuda")
    badv = good.clone()
    badv[7] = bad
    o1, l1 = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, qk_descale=good)
    o2, l2 = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, qk_descale=badv)
    torch.cuda.synchronize()
    nonempty = (sl > 0).cpu()
    assert torch.isnan(o2[nonempty][:, :, 7].float()).all() and torch.isnan(l2[nonempty][:, 7]).all()
    keep = [h for h in range(H) if h != 7]
    assert torch.equal(o1[:, :, keep], o2[:, :, keep]) and torch.equal(l1[:, keep], l2[:, keep])


@pytest.mark.parametrize("bad", [float("nan"), -1.0, float("inf")])
def test_invalid_log2_scale_gives_nan(gpu_lib, bad):
    w = make_workload(seqlens=[300, 5, 1200], num_heads_q=64, seed=101)
    q, kv, bt, sl = to_gpu(w)
    md, ns = _meta(w, sl, 8)
    b = torch.tensor([bad], dtype=torch.float32, device="cuda")
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, bmm1_scale_log2_tensor=b)
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()


def test_fp8_query_with_split_cache_is_bitwise_the_joined_cache(gpu_lib):
    w = make_workload(seqlens=[1, 64, 65, 777, 0, 300], num_heads_q=64, kv_dtype="fp8_e4m3fn", seed=109)
    _, _, qt = _fp8_q(w, 110)
    _, kv, bt, sl = to_gpu(w)
    s1, s2 = scales(w)
    md, ns = _meta(w, sl, 8)
    o1, l1 = mla.mla_decode_fwd(qt, kv, bt, sl, DV, md, ns, softmax_scale=s1, v_scale=s2)
    o2, l2 = mla.mla_decode_fwd(qt, kv[..., :DV].contiguous(), bt, sl, DV, md, ns, softmax_scale=s1, v_scale=s2,
                                kv_rope=kv[..., DV:].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("parts", [1, 16])
@pytest.mark.parametrize("s_q,causal", [(1, False), (2, True)])
def test_all_optional_scales_with_two_waves_per_page(gpu_lib, parts, s_q, causal):
    """16 heads (at most 32 rows: two waves per page, merged per split) with
    per-head descales, sinks and device-held bmm1 / bmm2 against the oracle."""
    H = 16
    w = make_workload(seqlens=[700, 1, 33, 2500, 0, 90], s_q=s_q, num_heads_q=H, causal=causal, seed=113)
    q, kv, bt, sl = to_gpu(w)
    s1, s2 = scales(w)
    s1, s2 = float(np.float32(s1 * 1.2)), float(np.float32(0.8))
    rng = np.random.default_rng(114)
    qk = rng.uniform(0.5, 2.0, H).astype(np.float32)
    pv = rng.uniform(0.5, 2.0, H).astype(np.float32)
    sinks = np.linspace(-1.0, 3.0, H).astype(np.float32)
    md, ns = _meta(w, sl, parts)
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=5.0, v_scale=7.0, causal=causal,
                                  bmm1_scale_tensor=torch.tensor([s1], dtype=torch.float32, device="cuda"),
                                  bmm2_scale_tensor=torch.tensor([s2], dtype=torch.float32, device="cuda"),
                                  qk_descale=torch.from_numpy(qk).cuda(), pv_descale=torch.from_numpy(pv).cuda(),
                                  sinks=torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    ref = oracle_decode(w.q_bits, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, s1, causal, s2,
                        sinks=sinks.astype(np.float64), qk_descale=qk.astype(np.float64),
                        pv_descale=pv.astype(np.float64))
    compare(w, out, lse, ref, label=f"two waves per page, all scales, s_q={s_q} parts={parts}")
