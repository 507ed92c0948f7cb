"""The no-allocation entry point (mla_decode_fwd_noalloc) through the C ABI:
the same results as mla_decode_fwd with a caller workspace, on two calls in a
row on one GPU (the second with a smaller problem, so that the static scratch
still holds the first call's partials)."""
import ctypes

import numpy as np
import pytest
import torch

import mla_paged_kv_metadata_amd as mla
from workloads import make_workload

from gpu_util import DV, compare, run_oracle, scales, to_gpu

pytestmark = pytest.mark.gpu


def _noalloc_c(w, t, md, ns, out, lse):
    """One call of the C entry point with raw device pointers."""
    lib = mla.load_library()
    q, kv, bt, sl = t
    s1, s2 = scales(w)
    code = mla.KV_BF16 if w.kv_dtype == "bf16" else mla.KV_FP8_E4M3FN
    P = ctypes.c_void_p
    stream = P(torch.cuda.current_stream().cuda_stream)
    return lib.mla_decode_fwd_noalloc(
        P(q.data_ptr()), w.batch, w.s_q, w.num_heads_q, 576, P(kv.data_ptr()), code, kv.shape[0], kv.shape[1],
        w.num_heads_k, P(bt.data_ptr()), bt.shape[1], P(sl.data_ptr()), DV, s1, s2, int(w.causal),
        P(md.data_ptr()), md.shape[0], P(ns.data_ptr()), P(out.data_ptr()), P(lse.data_ptr()), stream)


def _both(w, parts=None):
    t = to_gpu(w)
    q, kv, bt, sl = t
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, w.num_heads_k, num_parts=parts)
    s1, s2 = scales(w)
    ref_o, ref_l = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=s1, v_scale=s2, causal=w.causal)
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    assert _noalloc_c(w, t, md, ns, out, lse) == 0
    torch.cuda.synchronize()
    return out, lse, ref_o, ref_l


def test_noalloc_equals_the_workspace_entry_point_twice(gpu_lib):
    # First call: a large split problem; second: a smaller one on the same scratch.
    big = make_workload(seqlens=[3000, 65, 1, 1800, 640, 4096, 0, 900], num_heads_q=128, seed=71)
    small = make_workload(seqlens=[700, 5, 130], num_heads_q=64, s_q=2, causal=True, seed=72)
    for w, parts in ((big, None), (small, 48)):
        out, lse, ref_o, ref_l = _both(w, parts)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"B={w.batch}: differs from mla_decode_fwd"
        compare(w, out, lse, run_oracle(w), label=f"noalloc B={w.batch}")


def test_noalloc_fp8_after_bf16(gpu_lib):
    w = make_workload(seqlens=[1500, 33, 800], num_heads_q=128, kv_dtype="fp8_e4m3fn", seed=73)
    out, lse, ref_o, ref_l = _both(w, 40)
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    compare(w, out, lse, run_oracle(w), label="noalloc fp8")


def test_noalloc_rejects_a_problem_larger_than_the_scratch(gpu_lib):
    lib = mla.load_library()
    P = ctypes.c_void_p
    # 8192 sequences x 1024 rows of partials exceed the 128 MiB scratch.
    rc = lib.mla_decode_fwd_noalloc(P(1), 8192, 8, 128, 576, P(1), 0, 8, 64, 1, P(1), 1, P(1), DV, 0.04, 1.0, 0,
                                    P(1), 256, P(1), P(1), P(1), P(0))
    assert rc == 3
    assert b"scratch" in lib.mla_status_str(rc)
