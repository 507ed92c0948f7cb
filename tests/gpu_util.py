"""Shared helpers of the GPU parity tests: move a seeded workload to the GPU,
run the library through its C ABI, run the oracle on the same bytes, and
compare at the stated tolerances."""
import numpy as np
import torch

import mla_paged_kv_metadata_amd as mla
from oracle import fused_fp8_scales
from oracle import mla_decode as oracle_decode

DV = 512
# Tolerances: bf16 cache -> out max|d| <= 1e-2*max|out_ref| + 1e-3, lse max|d| <= 2e-3;
# fp8 cache -> out coefficient 5e-2 (same form), lse 1e-2: the fp8 matrix core takes q as
# two e4m3 terms and P as one e4m3 term per 32-token block.
TOL = {"bf16": (1e-2, 2e-3), "fp8_e4m3fn": (5e-2, 1e-2)}


def to_gpu(w, dev="cuda:0"):
    q = torch.from_numpy(np.ascontiguousarray(w.q_bits).view(np.int16)).view(torch.bfloat16).to(dev)
    if w.kv_dtype == "bf16":
        kv = torch.from_numpy(np.ascontiguousarray(w.kv).view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        kv = torch.from_numpy(np.ascontiguousarray(w.kv)).view(torch.float8_e4m3fn).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(w.cache_seqlens)).to(dev)
    return q, kv, bt, sl


def scales(w):
    """(bmm1, bmm2) for the workload: 1/sqrt(576) and 1 for a bf16 cache; the
    oracle's fused fp8 scales (FlashInfer MLA page) for an e4m3fn cache."""
    if w.kv_dtype == "bf16":
        return w.head_dim ** -0.5, 1.0
    return fused_fp8_scales(k_scale=w.k_scale, v_scale=w.v_scale, head_dim_qk=w.head_dim)


def run_gpu(w, num_parts=None, fixed_cost=None, tensors=None):
    q, kv, bt, sl = tensors if tensors is not None else to_gpu(w)
    md, ns = mla.mla_get_metadata(sl, w.heads_per_head_k, w.num_heads_k, num_parts=num_parts,
                                  fixed_cost=fixed_cost)
    s1, s2 = scales(w)
    out, lse = mla.mla_decode_fwd(q, kv, bt, sl, DV, md, ns, softmax_scale=s1, causal=w.causal, v_scale=s2)
    torch.cuda.synchronize()
    return out, lse, md, ns


def run_oracle(w, batches=None):
    s1, s2 = scales(w)
    return oracle_decode(w.q_bits, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, DV, s1, w.causal, s2,
                         batches=batches)


def compare(w, out, lse, ref, batches=None, label=""):
    """Element-wise comparison on the chosen batches; returns (max|dout|, tol, max|dlse|)."""
    ro, rl = ref
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    bs = list(range(w.batch)) if batches is None else list(batches)
    ro, rl, o, l = ro[bs], rl[bs], o[bs], l[bs]
    coef, ltol = TOL[w.kv_dtype]
    tol = coef * np.abs(ro).max() + 1e-3
    assert np.isfinite(o).all(), f"{label}: non-finite out"
    do = np.abs(o - ro).max()
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(l)), f"{label}: lse finiteness differs"
    assert (l[~fin] == -np.inf).all(), f"{label}: empty rows must have lse = -inf"
    dl = np.abs(l[fin] - rl[fin]).max() if fin.any() else 0.0
    print(f"{label}: max|dout|={do:.3e} tol={tol:.3e}  max|dlse|={dl:.3e} tol={ltol:.1e}", flush=True)
    assert do <= tol, f"{label}: out error {do} > {tol}"
    assert dl <= ltol, f"{label}: lse error {dl} > {ltol}"
    return do, tol, dl
