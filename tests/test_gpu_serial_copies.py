"""Race check: the library built with every page copy issued only after the
workgroup is done with the page before it (MLA_SERIAL_COPIES) gives the same
out and lse, bit for bit, as the default build, whose copies overlap the
previous page's reads.  Same inputs, same table."""
import pytest
import torch

import mla_paged_kv_metadata_amd as mla
from workloads import make_workload, repage

from gpu_util import DV, scales, to_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # name, workload kwargs, block size, parts, split layout
    ("bf16 128 heads", dict(seqlens=[1, 64, 65, 700, 2000, 130, 0, 4000], num_heads_q=128), 64, 32, False),
    ("bf16 causal s_q=2", dict(seqlens=[3, 90, 1500, 640], s_q=2, num_heads_q=128, causal=True), 64, 16, False),
    ("bf16 16 heads, two waves per page", dict(seqlens=[1, 33, 700, 4000, 97], num_heads_q=16), 64, 24, False),
    ("bf16 grouped KV heads", dict(seqlens=[400, 90, 5, 1200], num_heads_q=64, num_heads_k=2), 64, 12, False),
    ("bf16 16-token blocks", dict(seqlens=[100, 1000, 63], num_heads_q=128), 16, 10, False),
    ("bf16 split cache", dict(seqlens=[100, 1000, 63], num_heads_q=64), 64, 10, True),
    ("fp8", dict(seqlens=[1, 64, 65, 700, 2000, 130, 0, 4000], num_heads_q=128, kv_dtype="fp8_e4m3fn"), 64, 32, False),
    ("fp8 causal 64 heads", dict(seqlens=[3, 90, 1500], s_q=2, num_heads_q=64, causal=True, kv_dtype="fp8_e4m3fn"),
     32, 9, False),
]


def _run(w, t, parts, split):
    q, kv, bt, sl = t
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, w.num_heads_k, num_parts=parts)
    s1, s2 = scales(w)
    kw = {}
    if split:
        kw = {"kv_rope": kv[..., DV:].contiguous(), "q_rope": q[..., DV:].contiguous()}
        q, kv = q[..., :DV].contiguous(), kv[..., :DV].contiguous()
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=s1, causal=w.causal, v_scale=s2, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name,kw,bs,parts,split", CASES, ids=[c[0] for c in CASES])
def test_serial_copies_build_is_bitwise_the_default(gpu_lib, name, kw, bs, parts, split):
    w = make_workload(seed=131, **kw)
    if bs != w.page_block_size:
        w = repage(w, bs, seed=3)
    t = to_gpu(w)
    o1, l1 = _run(w, t, parts, split)
    with mla.library_variant(mla.SERIAL_LIB_PATH):
        o2, l2 = _run(w, t, parts, split)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), name
    assert torch.equal(l1, l2), name
