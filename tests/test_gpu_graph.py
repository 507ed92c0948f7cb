"""The whole decode step (scheduler, split kernel, combine) captured in a HIP
graph and replayed: every replay must reproduce the eager result bit for bit
(the kernels are deterministic and record no memset nodes).  Replays are
interleaved with unrelated eager work and host synchronisations, and the
inputs' sequence lengths change between replays through the captured device
buffer, as a serving loop would."""
import numpy as np
import pytest
import torch

import mla_paged_kv_metadata_amd as mla
from workloads import make_workload

from gpu_util import DV, compare, run_oracle, scales, to_gpu

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(gpu_lib):
    w = make_workload(seqlens=[700, 64, 1, 2000, 129], num_heads_q=128, seed=77)
    q, kv, bt, sl = to_gpu(w)
    dev = q.device
    P = 24
    s1, s2 = scales(w)
    md = torch.empty((P, 8), dtype=torch.int32, device=dev)
    ns = torch.empty((w.batch + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, 1, w.num_heads_q, DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.num_heads_q, 1), dtype=torch.float32, device=dev)
    ws = torch.empty((mla.mla_workspace_bytes(w.batch, 1, w.num_heads_q, 1, DV, P),), dtype=torch.uint8,
                     device=dev)

    def step():
        mla.mla_get_metadata(sl, w.heads_per_head_k, 1, num_parts=P, tile_md=md, num_splits=ns)
        mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=s1, v_scale=s2, out=out, lse=lse,
                           workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    compare(w, out, lse, run_oracle(w), label="eager")

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        out.fill_(0)
        lse.fill_(0)
        junk = torch.randn(1 << 20, device=dev).sum()          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: out differs from eager"
        assert torch.equal(lse, ref_lse), f"replay {rep}: lse differs from eager"
        del junk

    # New lengths written into the captured cache_seqlens buffer are picked up
    # by the replay (the scheduler runs inside the graph).
    L2 = [300, 1000, 65, 1, 2000]
    w2 = make_workload(seqlens=L2, num_heads_q=128, seed=77)
    w2.q_bits[...] = w.q_bits
    w2.kv = w.kv
    w2.block_table = w.block_table
    sl.copy_(torch.tensor(L2, dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    compare(w2, out, lse, run_oracle(w2), label="replay with new lengths")


def test_graph_replays_with_ext_inputs(gpu_lib):
    """fp8 split cache and split query, sinks and device scales inside the graph:
    replays match eager bit for bit, and a new bmm1 scale written into its
    device buffer between replays is picked up (the eager call with that scale
    as a host value gives the same bits)."""
    w = make_workload(seqlens=[900, 3, 0, 1500, 65], num_heads_q=64, s_q=2, causal=True, kv_dtype="fp8_e4m3fn",
                      seed=79)
    q, kv, bt, sl = to_gpu(w)
    dev = q.device
    P = 16
    s1, s2 = scales(w)
    kv_nope, kv_rope = kv[..., :DV].contiguous(), kv[..., DV:].contiguous()
    q_nope, q_rope = q[..., :DV].contiguous(), q[..., DV:].contiguous()
    sinks = torch.linspace(-1.0, 2.0, 64, device=dev)
    b1 = torch.tensor([s1], dtype=torch.float32, device=dev)
    b2 = torch.tensor([s2], dtype=torch.float32, device=dev)
    md = torch.empty((P, 8), dtype=torch.int32, device=dev)
    ns = torch.empty((w.batch + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, 2, 64, DV), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, 64, 2), dtype=torch.float32, device=dev)
    ws = torch.empty((mla.mla_workspace_bytes(w.batch, 2, 64, 1, DV, P),), dtype=torch.uint8, device=dev)
    ext = dict(sinks=sinks, bmm1_scale_tensor=b1, bmm2_scale_tensor=b2, kv_rope=kv_rope, q_rope=q_rope)

    def step():
        mla.mla_get_metadata(sl, w.heads_per_head_k, 1, num_parts=P, tile_md=md, num_splits=ns)
        mla.mla_decode_fwd(q_nope, kv_nope, bt, sl, DV, md, ns, causal=True, out=out, lse=lse, workspace=ws, **ext)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(0)
        lse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {rep} differs from eager"
    b1.fill_(s1 * 0.5)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    o2, l2 = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=float(b1.item()), v_scale=s2, causal=True,
                                sinks=sinks)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
