#!/usr/bin/env python3
"""Benchmark of MLA decode over a paged KV cache on one MI355X.

One step = the whole decode path over one synthetic batch: the split-KV
scheduler (mla_get_metadata), the split attention kernel and the
log-sum-exp combine.  Workload: B=64 sequences, 1 query token, 128 query
heads sharing one 576-wide latent KV head (V = first 512 columns), 64-token
pages, lengths uniform in [1024, 4096], bf16, seed 2.

Prints ONE JSON line on stdout.  value = algorithmic TFLOP/s of the whole
step; the decode kernel's own duration (HIP events on its stream) gives the
HBM roofline fraction.  The KV pool is replicated and rotated so that every
step streams its cache from HBM rather than the 256 MB last-level cache.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode TFLOP/s + effective KV GB/s (% roofline), B=64 H=128 ctx~4K"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_counts(w):
    """Algorithmic FLOPs and bytes of one decode over workload w."""
    L = w.cache_seqlens.astype(np.int64)
    if w.causal:
        n = sum(max(0, min(int(l), int(l) - w.s_q + 1 + i)) for l in L for i in range(w.s_q))
    else:
        n = int(L.sum()) * w.s_q
    H = w.num_heads_q
    flops = 2 * H * (w.head_dim + w.head_dim_v) * n
    e_kv = 1 if w.kv_dtype == "fp8_e4m3fn" else 2
    kv_bytes = int(L.sum()) * w.num_heads_k * w.head_dim * e_kv
    io_bytes = w.batch * w.s_q * H * (w.head_dim * 2 + w.head_dim_v * 2 + 4)
    return flops, kv_bytes, kv_bytes + io_bytes


def cpu_baseline(w, budget_s=20.0):
    """The fp64 oracle on the host cores over as many whole sequences as fit the budget."""
    from oracle import mla_decode as oracle_decode
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    scale = w.head_dim ** -0.5
    done, t_total, flops = [], 0.0, 0
    L = w.cache_seqlens.astype(np.int64)
    for b in range(w.batch):
        t0 = time.perf_counter()
        oracle_decode(w.q_bits, w.kv, w.kv_dtype, w.block_table, w.cache_seqlens, w.head_dim_v, scale,
                      w.causal, 1.0, batches=[b])
        t_total += time.perf_counter() - t0
        done.append(b)
        flops += 2 * w.num_heads_q * (w.head_dim + w.head_dim_v) * int(L[b]) * w.s_q
        if t_total >= budget_s:
            break
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(done)} of {w.batch} sequences ({int(L[done].sum())} keys), fp64 NumPy, "
                      f"{t_total:.2f} s"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=4, help="KV pool replicas rotated across steps")
    ap.add_argument("--num-parts", type=int, default=None, help="override the scheduler's balancing target")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this decode path is built and "
              "measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mla_paged_kv_metadata_amd as mla
    from workloads import make_config

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 3 times")
        return
    mla.load_library()
    dev = torch.device("cuda:0")
    w = make_config(2)
    flops, kv_bytes, alg_bytes = work_counts(w)
    log(f"workload: B={w.batch} H={w.num_heads_q} keys={int(w.cache_seqlens.sum())} pages={w.num_blocks} "
        f"kv={kv_bytes / 1e6:.1f} MB alg={alg_bytes / 1e6:.1f} MB flops={flops / 1e9:.2f} G")

    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    kv_host = torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16)
    kvs = [kv_host.to(dev) for _ in range(max(1, args.copies))]
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.cache_seqlens).to(dev)
    hpk = w.heads_per_head_k
    P = args.num_parts or mla.mla_num_parts(w.batch, hpk, w.num_heads_k)
    md = torch.empty((P, 8), dtype=torch.int32, device=dev)
    ns = torch.empty((w.batch + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((w.batch, w.s_q, w.num_heads_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, w.num_heads_q, w.s_q), dtype=torch.float32, device=dev)
    ws = torch.empty((mla.mla_workspace_bytes(w.batch, w.s_q, w.num_heads_q, w.num_heads_k, 512, P),),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    K, W = args.steps, args.warmup
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]

    def step(i, events=None):
        kv = kvs[i % len(kvs)]
        if events:
            events[0].record(stream)
        mla.mla_get_metadata(sl, hpk, w.num_heads_k, num_parts=P, tile_md=md, num_splits=ns)
        if events:
            events[1].record(stream)
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, causal=False, out=out, lse=lse, workspace=ws,
                           stage="splits")
        if events:
            events[2].record(stream)
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, causal=False, out=out, lse=lse, workspace=ws,
                           stage="combine")
        if events:
            events[3].record(stream)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(W + i, ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    t_meta = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(K)])
    t_dec = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(K)])
    t_cmb = np.array([ev[i][2].elapsed_time(ev[i][3]) for i in range(K)])
    dec_s = float(t_dec.mean()) * 1e-3
    log(f"step {ms_step * 1e3:.1f} us | metadata {t_meta.mean() * 1e3:.1f} us | decode {t_dec.mean() * 1e3:.1f} us "
        f"(min {t_dec.min() * 1e3:.1f}) | combine {t_cmb.mean() * 1e3:.1f} us")

    # correctness of the last step against the oracle on a few sequences
    check = {}
    try:
        from oracle import mla_decode as oracle_decode
        bs = [0, 17, 63]
        ro, rl = oracle_decode(w.q_bits, w.kv, "bf16", w.block_table, w.cache_seqlens, 512, 576 ** -0.5,
                               batches=bs)
        o = out.float().cpu().numpy()[bs]
        l = lse.cpu().numpy()[bs]
        check = {"batches": bs, "max_abs_dout": float(np.abs(o - ro[bs]).max()),
                 "tol_out": float(1e-2 * np.abs(ro[bs]).max() + 1e-3),
                 "max_abs_dlse": float(np.abs(l - rl[bs]).max()), "tol_lse": 2e-3}
    except Exception as e:  # the bench line must still print
        check = {"error": repr(e)}

    step_tflops = flops / (ms_step * 1e-3) / 1e12
    dec_gbs = alg_bytes / dec_s / 1e9
    rec = {
        "metric": METRIC,
        "value": round(step_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "standard MLA decode: B=64 s_q=1 H_q=128 H_k=1 D=576 Dv=512 page=64 "
                               "L~U[1024,4096] seed 2, bf16 q/kv ~N(0,1), scale 1/24",
                   "batch": w.batch, "seq_len_q": w.s_q, "num_heads_q": w.num_heads_q,
                   "total_keys": int(w.cache_seqlens.sum()), "num_parts": P, "kv_copies": len(kvs)},
        "kv_gbps_step": round(kv_bytes / (ms_step * 1e-3) / 1e9, 1),
        "kernels_us": {"metadata": round(float(t_meta.mean()) * 1e3, 2),
                       "decode": round(float(t_dec.mean()) * 1e3, 2),
                       "combine": round(float(t_cmb.mean()) * 1e3, 2)},
        "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "mla_decode_kernel<bf16>", "alg_bytes_per_launch": alg_bytes,
                     "kernel_tflops": round(flops / dec_s / 1e12, 1),
                     "mfma_frac": round(flops / dec_s / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "check": check,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
