"""GPU parity for caches whose blocks hold other than 64 tokens (the FlashMLA
interface page takes page_block_size as the cache's second dimension; the
FlashInfer MLA page and the Ascend ATB MLA page take any page / block size).
The kernels still walk 64-token pages; each 16-token slice of a page comes
from its own block.  Rows past a sequence's end hold NaN here, so any use of
them would show."""
import numpy as np
import pytest
import torch

import mla_paged_kv_metadata_amd as mla
from workloads import make_config, make_workload, repage

from gpu_util import DV, compare, run_oracle, scales, to_gpu

pytestmark = pytest.mark.gpu

SEQLENS = [0, 1, 15, 16, 17, 63, 64, 65, 700, 2000, 130, 1000]


def _run(w, t, parts=None, **kw):
    q, kv, bt, sl = t
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, w.num_heads_k, num_parts=parts)
    s1, s2 = scales(w)
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=s1, causal=w.causal, v_scale=s2, **kw)
    torch.cuda.synchronize()
    return out, lse


# 1 part: every sequence in one split; 48 parts: splits start inside
# sequences, so a split's first page can fall in the middle of a block.
@pytest.mark.parametrize("parts", [1, 48])
@pytest.mark.parametrize("P", [16, 32, 48, 128, 256])
@pytest.mark.parametrize("kv_dtype,causal,s_q,H", [("bf16", False, 1, 64), ("bf16", True, 2, 16),
                                                   ("fp8_e4m3fn", False, 1, 128)])
def test_block_sizes_match_oracle(gpu_lib, parts, P, kv_dtype, causal, s_q, H):
    w = repage(make_workload(seqlens=SEQLENS, s_q=s_q, num_heads_q=H, causal=causal, kv_dtype=kv_dtype,
                             seed=61 + P), P, seed=P, pad="oob")
    print(f"case: P={P} {kv_dtype} causal={causal} s_q={s_q} H={H} parts={parts}", flush=True)
    out, lse = _run(w, to_gpu(w), parts)
    compare(w, out, lse, run_oracle(w), label=f"P={P} {kv_dtype} parts={parts}")


@pytest.mark.parametrize("P", [16, 32, 128])
def test_block_size_is_bitwise_invisible_at_full_size(gpu_lib, P):
    """The standard B=64 H=128 decode in its default launch configuration: the
    same rows in blocks of P tokens give bitwise the 64-token-block result."""
    w = make_config(2)
    print(f"case: c2 P={P}", flush=True)
    o1, l1 = _run(w, to_gpu(w))
    r = repage(w, P, seed=3)
    o2, l2 = _run(r, to_gpu(r))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8_e4m3fn"])
def test_split_cache_with_small_blocks_is_bitwise_the_joined_layout(gpu_lib, kv_dtype):
    w = repage(make_workload(seqlens=SEQLENS, num_heads_q=64, kv_dtype=kv_dtype, seed=67), 32, seed=1)
    q, kv, bt, sl = to_gpu(w)
    print(f"case: split cache P=32 {kv_dtype}", flush=True)
    o1, l1 = _run(w, (q, kv, bt, sl), 16)
    o2, l2 = _run(w, (q, kv[..., :DV].contiguous(), bt, sl), 16, kv_rope=kv[..., DV:].contiguous())
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_block_size_sampled_rows_against_oracle(gpu_lib):
    """Full-size causal two-token decode (B=128 H=128, L in [2048, 8192]) in
    16-token blocks, checked on sampled sequences."""
    w = repage(make_config(3), 16, seed=2)
    print("case: c3 P=16 sampled", flush=True)
    out, lse = _run(w, to_gpu(w))
    bs = [0, 77, 127]
    compare(w, out, lse, run_oracle(w, batches=bs), batches=bs, label="c3 P=16")
