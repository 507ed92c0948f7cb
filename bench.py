#!/usr/bin/env python3
"""Benchmark of MLA decode over a paged KV cache on one MI355X.

One step = the whole decode path over one synthetic batch: the split-KV
scheduler (mla_get_metadata), the split attention kernel and the
log-sum-exp combine.  Workload: B=64 sequences, 1 query token, 128 query
heads sharing one 576-wide latent KV head (V = first 512 columns), 64-token
pages, lengths uniform in [1024, 4096], bf16, seed 2.

Prints ONE JSON line on stdout.  value = algorithmic TFLOP/s of the whole
step (graph replays, host clock).  The roofline fraction is taken over the
whole decode call, mla_decode_fwd (split attention + combine), timed per call
with HIP events on its stream after a 1 GiB scratch read (cold caches):
median and min over --fwd-iters calls (the back-to-back rate and the
split-attention kernel alone are sub-fields).  The KV pool is replicated and rotated so that every step streams
its cache from HBM rather than the 256 MB last-level cache.
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
FP8_PEAK_TFLOPS = 5000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_counts(w, q_elem=2):
    """Algorithmic FLOPs and bytes of one decode over workload w (q_elem: bytes
    per q element, 1 for an e4m3 query)."""
    L = w.cache_seqlens.astype(np.int64)
    if w.causal:
        n = sum(max(0, min(int(l), int(l) - w.s_q + 1 + i)) for l in L for i in range(w.s_q))
    else:
        n = int(L.sum()) * w.s_q
    H = w.num_heads_q
    flops = 2 * H * (w.head_dim + w.head_dim_v) * n
    e_kv = 1 if w.kv_dtype == "fp8_e4m3fn" else 2
    kv_bytes = int(L.sum()) * w.num_heads_k * w.head_dim * e_kv
    io_bytes = w.batch * w.s_q * H * (w.head_dim * q_elem + w.head_dim_v * 2 + 4)
    return flops, kv_bytes, kv_bytes + io_bytes


DECODE_SOURCES = ["mla_paged_kv_metadata_amd/csrc/mla_decode.hip", "mla_paged_kv_metadata_amd/csrc/mla_kernels.h"]


def traffic_json(cfg):
    return os.path.join(ROOT, "profiles", f"decode_c{cfg}_hbm_traffic.json")


WORKLOAD_NAMES = {1: "tiny MLA decode: B=2 s_q=1 H_q=16 L={127,300}",
                  2: "standard MLA decode: B=64 s_q=1 H_q=128 L~U[1024,4096]",
                  3: "MTP causal MLA decode: B=128 s_q=2 H_q=128 L~U[2048,8192]",
                  4: "skewed MLA decode: B=32 s_q=1 H_q=16, one 65536 + 31 lognormal(512,1) lengths",
                  5: "fp8-e4m3 KV MLA decode: B=128 s_q=1 H_q=128 L=8192"}


def decode_source_hash():
    """Hash of the kernels' sources with comments and blank space removed, so
    that an edit of the comments alone keeps a counter summary current."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in DECODE_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(cfg):
    """HBM bytes per mla_decode_fwd call (split attention + combine) from the
    committed counter summary of the workload, or None when the kernels'
    sources changed since the counters were taken."""
    try:
        with open(traffic_json(cfg)) as fh:
            rec = json.load(fh)
        if rec.get("decode_source_hash") == decode_source_hash():
            return int(rec["hbm_bytes_per_call"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def _counter_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter, name_part):
    """Average over dispatches of the kernel whose name contains name_part of
    the counter's value summed over its instances (one dispatch = one id)."""
    per = {}
    for r in rows:
        if r.get("Counter_Name") == counter and name_part in r.get("Kernel_Name", ""):
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for a kernel named *{name_part}*")
    return sum(per.values()) / len(per), len(per)


def pmc_summary(cfg, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, commands, lds_fetch_dir=None):
    """Writes profiles/decode_c<cfg>_hbm_traffic.{md,json} from rocprofv3 --pmc runs:
    FETCH_SIZE and WRITE_SIZE of the bench workload (split-attention and
    combine kernels), and of the calibration reads of copy_mib MiB: a plain
    device copy and, if given, the LDS-DMA read (mla_lds_dma_read)."""
    copy_bytes = copy_mib << 20
    cf, _ = _per_dispatch(_counter_rows(copy_fetch_dir), "FETCH_SIZE", "copy")
    cw, _ = _per_dispatch(_counter_rows(copy_write_dir), "WRITE_SIZE", "copy")
    kf, kw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    lf = kl = None
    if lds_fetch_dir:
        lf, _ = _per_dispatch(_counter_rows(lds_fetch_dir), "FETCH_SIZE", "lds_dma_read")
        kl = copy_bytes / (lf * 1024)
    frows, wrows = _counter_rows(fetch_dir), _counter_rows(write_dir)
    df, nf = _per_dispatch(frows, "FETCH_SIZE", "mla_decode_kernel")
    dw, nw = _per_dispatch(wrows, "WRITE_SIZE", "mla_decode_kernel")
    try:
        cbf, _ = _per_dispatch(frows, "FETCH_SIZE", "mla_combine_kernel")
        cbw, _ = _per_dispatch(wrows, "WRITE_SIZE", "mla_combine_kernel")
    except SystemExit:                 # no split sequences: no combine launch
        cbf = cbw = 0.0
    # The page copies are LDS-DMA reads: the decode's fetch is scaled by the
    # LDS-DMA calibration when there is one; the combine's plain loads by the copy's.
    dec_fetch = df * 1024 * (kl if kl else kf)
    dec_write = dw * 1024 * kw
    cmb_fetch, cmb_write = cbf * 1024 * kf, cbw * 1024 * kw
    from workloads import make_config
    w = make_config(cfg)
    _, kv_bytes, alg_bytes = work_counts(w)
    kname = f"mla_decode_kernel<{'fp8' if w.kv_dtype == 'fp8_e4m3fn' else 'bf16'}>"
    rec = {"kernels": [kname, "mla_combine_kernel"], "workload": WORKLOAD_NAMES[cfg],
           "decode_source_hash": decode_source_hash(),
           "decode_fetch_kib_per_dispatch": round(df, 1), "decode_write_kib_per_dispatch": round(dw, 1),
           "combine_fetch_kib_per_dispatch": round(cbf, 1), "combine_write_kib_per_dispatch": round(cbw, 1),
           "copy_mib": copy_mib, "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
           "fetch_factor": round(kf, 4), "write_factor": round(kw, 4),
           "lds_dma_fetch_kib": None if lf is None else round(lf, 1),
           "lds_dma_fetch_factor": None if kl is None else round(kl, 4),
           "decode_fetch_bytes": int(dec_fetch), "decode_write_bytes": int(dec_write),
           "combine_fetch_bytes": int(cmb_fetch), "combine_write_bytes": int(cmb_write),
           "hbm_bytes_per_launch": int(dec_fetch + dec_write),
           "hbm_bytes_per_call": int(dec_fetch + dec_write + cmb_fetch + cmb_write),
           "algorithmic_bytes_per_launch": alg_bytes, "kv_bytes_per_launch": kv_bytes,
           "dispatches": {"fetch": nf, "write": nw}, "commands": commands}
    path = traffic_json(cfg)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    md = path[:-5] + ".md"
    with open(md, "w") as fh:
        fh.write(f"# HBM traffic of mla_decode_fwd ({kname} + mla_combine_kernel), {WORKLOAD_NAMES[cfg]}\n\n")
        fh.write("rocprofv3 TCC counters per dispatch (KiB, summed over instances), each scaled by what the "
                 f"same counter reads for a calibration of known size ({copy_mib} MiB): a plain device copy "
                 "for plain loads and stores"
                 + (", and a read through the page copies' LDS-DMA instruction (mla_lds_dma_read) for the "
                    "split-attention kernel's fetch" if kl else "") + ".\n\n")
        fh.write("| quantity | value |\n|---|---|\n")
        for k in ("decode_fetch_kib_per_dispatch", "decode_write_kib_per_dispatch", "combine_fetch_kib_per_dispatch",
                  "combine_write_kib_per_dispatch", "copy_fetch_kib", "copy_write_kib", "fetch_factor",
                  "write_factor", "lds_dma_fetch_kib", "lds_dma_fetch_factor", "decode_fetch_bytes",
                  "decode_write_bytes", "combine_fetch_bytes", "combine_write_bytes", "hbm_bytes_per_launch",
                  "hbm_bytes_per_call", "algorithmic_bytes_per_launch", "kv_bytes_per_launch",
                  "decode_source_hash"):
            fh.write(f"| {k} | {rec[k]} |\n")
        fh.write(f"\nsplit-attention kernel, measured / algorithmic bytes: "
                 f"{rec['hbm_bytes_per_launch'] / alg_bytes:.3f}\n")
        fh.write(f"whole call (split attention + combine), measured / algorithmic bytes: "
                 f"{rec['hbm_bytes_per_call'] / alg_bytes:.3f}\n\n")
        fh.write("Commands (from the repository root):\n\n")
        for c in commands:
            fh.write(f"    {c}\n")
    print(open(md).read())


def _per_dispatch_max(rows, counter, name_part):
    """As _per_dispatch, but the largest instance value per dispatch (for the
    GPU-wide GRBM counters, which every instance reports)."""
    per = {}
    for r in rows:
        if r.get("Counter_Name") == counter and name_part in r.get("Kernel_Name", ""):
            per[r["Dispatch_Id"]] = max(per.get(r["Dispatch_Id"], 0.0), float(r["Counter_Value"]))
    if not per:
        raise SystemExit(f"no {counter} rows for a kernel named *{name_part}*")
    return sum(per.values()) / len(per), len(per)


def mfma_summary(cfg, counter_dir, commands, simds=1024, xcds=8):
    """Writes profiles/decode_c<cfg>_mfma_lds.md from one rocprofv3 --pmc run of the
    matrix-core and LDS counters.  MFMA utilisation is the MFMA busy cycles per
    SIMD over the GPU-active cycles of one XCD: GRBM_GUI_ACTIVE comes back as one
    instance that adds up the 8 XCDs (its value / 8 matches the kernel's duration
    times the shader clock)."""
    rows = _counter_rows(counter_dir)
    k = "mla_decode_kernel"
    busy, n = _per_dispatch(rows, "SQ_VALU_MFMA_BUSY_CYCLES", k)
    gui, _ = _per_dispatch_max(rows, "GRBM_GUI_ACTIVE", k)
    from workloads import make_config
    w = make_config(cfg)
    fp8 = w.kv_dtype == "fp8_e4m3fn"
    # bf16: MOPS (units of 512 FLOPs); fp8: instructions, every one of them a
    # 32x32x64 MFMA (131072 FLOPs), as there is no fp8 MOPS counter.
    mops_name = "SQ_INSTS_VALU_MFMA_F8" if fp8 else "SQ_INSTS_VALU_MFMA_MOPS_BF16"
    flops_per = 32 * 32 * 64 * 2 if fp8 else 512
    mops, _ = _per_dispatch(rows, mops_name, k)
    conf, _ = _per_dispatch(rows, "SQ_LDS_BANK_CONFLICT", k)
    lds_act, _ = _per_dispatch(rows, "SQ_LDS_IDX_ACTIVE", k)
    lds_ins, _ = _per_dispatch(rows, "SQ_INSTS_LDS", k)
    alg_flops, _, _ = work_counts(w)
    util = 100.0 * (busy / simds) / (gui / xcds)
    md = os.path.join(ROOT, "profiles", f"decode_c{cfg}_mfma_lds.md")
    kname = f"mla_decode_kernel<{'fp8' if fp8 else 'bf16'}>"
    with open(md, "w") as fh:
        fh.write(f"# Matrix-core and LDS counters of {kname}, {WORKLOAD_NAMES[cfg]}\n\n")
        fh.write(f"rocprofv3 SQ/GRBM counters, averaged over {n} dispatches (one value per counter and "
                 "dispatch as rocprofv3 reports it).\n\n")
        fh.write("| quantity | value |\n|---|---|\n")
        for name, v in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("GRBM_GUI_ACTIVE", gui),
                        (mops_name, mops), ("SQ_LDS_BANK_CONFLICT", conf),
                        ("SQ_LDS_IDX_ACTIVE", lds_act), ("SQ_INSTS_LDS", lds_ins)):
            fh.write(f"| {name} | {v:.0f} |\n")
        fh.write(f"| MFMA busy cycles per SIMD (busy / {simds}) | {busy / simds:.0f} |\n")
        fh.write(f"| GPU-active cycles per XCD (GRBM_GUI_ACTIVE / {xcds}) | {gui / xcds:.0f} |\n")
        fh.write(f"| MFMA utilisation (per-SIMD busy / per-XCD active) | {util:.1f}% |\n")
        fh.write(f"| {'fp8' if fp8 else 'bf16'} MFMA FLOPs per dispatch ({'instructions x 131072' if fp8 else 'MOPS x 512'})"
                 f" | {mops * flops_per / 1e9:.2f} G |\n")
        fh.write(f"| algorithmic FLOPs per dispatch | {alg_flops / 1e9:.2f} G |\n")
        fh.write(f"| LDS bank-conflict cycles / LDS active cycles | {conf / max(lds_act, 1):.3f} |\n")
        fh.write("\nCommands (from the repository root):\n\n")
        for c in commands:
            fh.write(f"    {c}\n")
    print(open(md).read())


def trace_summary(cfg, trace_dir, commands, bench_json=None):
    """Writes profiles/decode_c<cfg>_kernel_trace.md from a rocprofv3 --kernel-trace --stats folder
    (and, if given, the JSON line that the profiled bench run printed)."""
    import csv
    import glob
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no *kernel_stats.csv under {trace_dir}")
    rows = list(csv.DictReader(open(f[0], newline="")))
    md = os.path.join(ROOT, "profiles", f"decode_c{cfg}_kernel_trace.md")
    with open(md, "w") as fh:
        fh.write(f"# rocprofv3 kernel trace, {WORKLOAD_NAMES[cfg]} (bench.py workload)\n\n")
        fh.write("| kernel | calls | average us | min us | max us | share |\n|---|---|---|---|---|---|\n")
        for r in rows:
            name = r["Name"]
            if "mla" not in name and float(r["Percentage"]) < 1.0:
                continue
            short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            fh.write(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |\n")
        fh.write("\n(Other kernels are the harness's own copies and conversions outside the timed steps.)\n\n")
        if bench_json:
            with open(bench_json) as bj:
                rec = json.loads(bj.read().strip().splitlines()[-1])
            fh.write("Per-kernel averages that the profiled run measured itself with HIP events (us): "
                     + ", ".join(f"{k} {v}" for k, v in rec["kernels_us"].items())
                     + f"; step {rec['ms_per_step'] * 1e3:.1f} us.\n\n")
        fh.write("Commands (from the repository root):\n\n")
        for c in commands:
            fh.write(f"    {c}\n")
    print(open(md).read())


def cpu_baseline(w, scale, vs, sinks, out_np, lse_np, budget_s=20.0, min_s=10.0, q_codes=None):
    """The fp64 oracle on the host cores over as many whole sequences as fit the
    budget, timed; the GPU's outputs of the same sequences (out_np, lse_np, from
    the last timed step) are checked against its results on the way.  When the
    whole workload takes less than min_s, it is run again (whole passes) until
    min_s of oracle time has accumulated, and the rate is taken over all passes."""
    from oracle import mla_decode as oracle_decode
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    sinks64 = None if sinks is None else sinks.astype(np.float64)
    done, t_total, flops, passes = [], 0.0, 0, 0
    d_out = d_lse = ref_max = 0.0
    L = w.cache_seqlens.astype(np.int64)
    while True:
        for b in range(w.batch):
            t0 = time.perf_counter()
            ro, rl = oracle_decode(w.q_bits if q_codes is None else q_codes, w.kv, w.kv_dtype, w.block_table,
                                   w.cache_seqlens, w.head_dim_v, scale, w.causal, vs, batches=[b], sinks=sinks64,
                                   q_format="bf16" if q_codes is None else "fp8_e4m3fn")
            t_total += time.perf_counter() - t0
            n = sum(max(0, min(int(L[b]), int(L[b]) - w.s_q + 1 + i)) for i in range(w.s_q)) if w.causal \
                else int(L[b]) * w.s_q
            flops += 2 * w.num_heads_q * (w.head_dim + w.head_dim_v) * n
            if passes == 0:
                done.append(b)
                d_out = max(d_out, float(np.abs(out_np[b] - ro[b]).max()))
                fin = np.isfinite(rl[b])
                if fin.any():
                    d_lse = max(d_lse, float(np.abs(lse_np[b][fin] - rl[b][fin]).max()))
                ref_max = max(ref_max, float(np.abs(ro[b]).max()))
            if t_total >= budget_s:
                break
        passes += 1
        if t_total >= min_s or len(done) < w.batch:
            break
    coef = 5e-2 if w.kv_dtype == "fp8_e4m3fn" else 1e-2
    check = {"sequences": len(done), "max_abs_dout": d_out, "tol_out": coef * ref_max + 1e-3,
             "max_abs_dlse": d_lse, "tol_lse": 1e-2 if w.kv_dtype == "fp8_e4m3fn" else 2e-3}
    check["pass"] = bool(d_out <= check["tol_out"] and d_lse <= check["tol_lse"])
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:
        blas = "unknown"
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "blas": blas,
            "sample": (f"{len(done)} of {w.batch} sequences ({int(L[done].sum())} keys)"
                       + (f", {passes} passes" if passes > 1 else "") + f", fp64 NumPy, {t_total:.2f} s")}, check


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="workload (2, the standard B=64 H=128 decode, is the headline; others for reference)")
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--copies", type=int, default=4, help="KV pool replicas rotated across steps")
    ap.add_argument("--fwd-iters", type=int, default=50,
                    help="cold-cache iterations of the whole mla_decode_fwd call (median / min)")
    ap.add_argument("--num-parts", type=int, default=None, help="override the scheduler's balancing target")
    ap.add_argument("--fixed-cost", type=int, default=None,
                    help="override the scheduler's per-split cost in pages (mla_get_metadata_ex)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--sinks", action="store_true", help="per-head attention sinks (mla_decode_fwd_ext)")
    ap.add_argument("--split-cache", action="store_true",
                    help="latent/rope cache and q as separate tensors (mla_decode_fwd_ext)")
    ap.add_argument("--device-scales", action="store_true", help="bmm1/bmm2 scales held on the device")
    ap.add_argument("--fp8-query", action="store_true",
                    help="an e4m3 query with a per-tensor q_scale folded into bmm1 (fp8 cache only)")
    ap.add_argument("--batch-share", type=int, default=1, metavar="N",
                    help="time one GPU's share of the batch split over N GPUs (its first B/N sequences)")
    ap.add_argument("--page-block-size", type=int, default=64,
                    help="tokens per cache block (a multiple of 16); the same rows re-laid in blocks of this size")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--lds-dma-calibration", type=int, default=0, metavar="MIB",
                    help="only read this many MiB through the page copies' LDS-DMA instruction (counter calibration)")
    ap.add_argument("--lds-dma-fetch-dir", help="with --pmc-summary: FETCH_SIZE folder of an --lds-dma-calibration run")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="summarise four rocprofv3 --pmc output folders into profiles/ (no GPU work)")
    ap.add_argument("--copy-mib", type=int, default=256, help="size of the calibration copy for --pmc-summary")
    ap.add_argument("--mfma-summary", metavar="COUNTER_DIR",
                    help="write profiles/decode_c<config>_mfma_lds.md from a rocprofv3 --pmc run of the MFMA/LDS counters")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats folder into profiles/ (no GPU work)")
    ap.add_argument("--bench-json", help="the profiled run's JSON line, quoted in a --trace-summary file")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="command line recorded in a --pmc-summary / --trace-summary file")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(args.config, *args.pmc_summary, args.copy_mib, args.pmc_command, args.lds_dma_fetch_dir)
        return
    if args.mfma_summary:
        mfma_summary(args.config, args.mfma_summary, args.pmc_command)
        return
    if args.trace_summary:
        trace_summary(args.config, args.trace_summary, args.pmc_command, args.bench_json)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this decode path is built and "
              "measured on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mla_paged_kv_metadata_amd as mla
    from workloads import batch_share, make_config, repage

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes 3 times")
        return
    if args.lds_dma_calibration:
        n = args.lds_dma_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        for _ in range(3):
            mla.lds_dma_read(src)
        torch.cuda.synchronize()
        log(f"read {n} bytes through LDS-DMA 3 times")
        return
    mla.load_library()
    dev = torch.device("cuda:0")
    w = make_config(args.config)
    if args.batch_share > 1:
        try:
            w = batch_share(w, args.batch_share)
        except ValueError as e:
            raise SystemExit(f"--batch-share {args.batch_share}: {e}")
    if args.page_block_size != w.page_block_size:
        w = repage(w, args.page_block_size, seed=1)
    fp8 = w.kv_dtype == "fp8_e4m3fn"
    q_codes, q_scale = None, 1.0
    if args.fp8_query:
        if not fp8:
            raise SystemExit("--fp8-query needs an fp8 cache (--config 5)")
        from workloads import fp8_query
        q_codes, q_scale = fp8_query(w, seed=1000 + args.config)
    if fp8:
        s1, s2 = mla.fp8_fused_scales(q_scale=q_scale, k_scale=w.k_scale, v_scale=w.v_scale, head_dim_qk=w.head_dim)
    else:
        s1, s2 = w.head_dim ** -0.5, 1.0
    flops, kv_bytes, alg_bytes = work_counts(w, 1 if args.fp8_query else 2)
    log(f"workload: B={w.batch} H={w.num_heads_q} keys={int(w.cache_seqlens.sum())} pages={w.num_blocks} "
        f"kv={kv_bytes / 1e6:.1f} MB alg={alg_bytes / 1e6:.1f} MB flops={flops / 1e9:.2f} G")

    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if q_codes is not None:
        q = torch.from_numpy(np.ascontiguousarray(q_codes)).view(torch.float8_e4m3fn).to(dev)
    if fp8:
        kv_host = torch.from_numpy(w.kv).view(torch.float8_e4m3fn)
    else:
        kv_host = torch.from_numpy(w.kv.view(np.int16)).view(torch.bfloat16)
    kvs = [kv_host.to(dev) for _ in range(max(1, args.copies))]
    # Optional inputs of mla_decode_fwd_ext: per-head sinks, the split
    # latent/rope cache (with split q), device-held scales.
    ext = {}
    sinks_np = None
    if args.sinks:
        sinks_np = np.linspace(-1.0, 3.0, w.num_heads_q).astype(np.float32)
        ext["sinks"] = torch.from_numpy(sinks_np).to(dev)
    if args.device_scales:
        ext["bmm1_scale_tensor"] = torch.tensor([s1], dtype=torch.float32, device=dev)
        ext["bmm2_scale_tensor"] = torch.tensor([s2], dtype=torch.float32, device=dev)
    ropes = [None] * len(kvs)
    if args.split_cache:
        ropes = [kv[..., 512:].contiguous() for kv in kvs]
        kvs = [kv[..., :512].contiguous() for kv in kvs]
        ext["q_rope"] = q[..., 512:].contiguous()
        q = q[..., :512].contiguous()
        torch.cuda.empty_cache()

    def ext_for(i):
        return dict(ext, kv_rope=ropes[i % len(kvs)]) if args.split_cache else ext
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

    def step(i):
        kv = kvs[i % len(kvs)]
        mla.mla_get_metadata(sl, hpk, w.num_heads_k, num_parts=P, fixed_cost=args.fixed_cost, tile_md=md,
                             num_splits=ns)
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, softmax_scale=s1, v_scale=s2, causal=w.causal, out=out,
                           lse=lse, workspace=ws, stage="splits", **ext_for(i))
        mla.mla_decode_fwd(q, kv, bt, sl, 512, md, ns, softmax_scale=s1, v_scale=s2, causal=w.causal, out=out,
                           lse=lse, workspace=ws, stage="combine", **ext_for(i))

    for i in range(2):                      # first launches (library and allocator set-up)
        step(i)
    torch.cuda.synchronize()

    # Each step's three launches are replayed from a HIP graph (one graph per KV
    # replica), so the GPU runs them back to back without host launch gaps;
    # --no-graph launches them eagerly instead.  The W warm-up steps run the
    # same way: under sustained load the GPU takes some 20 ms to reach its
    # steady clock, so the default W covers about 50 ms of steps.
    timing = "eager"
    graphs = []
    if not args.no_graph:
        try:
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                for c in range(len(kvs)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=side):
                        step(c)
                    graphs.append(g)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            timing = "hip_graph"
        except Exception as e:  # fall back to eager launches, and say so
            log(f"graph capture failed ({e!r}); timing eager launches")
            graphs = []
    for i in range(W):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step(i)
    torch.cuda.synchronize()
    # Timed region: K whole steps.
    t0 = time.perf_counter()
    for i in range(K):
        if graphs:
            graphs[(W + i) % len(graphs)].replay()
        else:
            step(W + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K

    # Per-kernel durations: each kernel alone, K launches back to back (graph-
    # replayed like the steps, else eager), bracketed by HIP events on the
    # launch stream; the average launch of the decode kernel gives the roofline.
    def meta_call(i):
        mla.mla_get_metadata(sl, hpk, w.num_heads_k, num_parts=P, fixed_cost=args.fixed_cost, tile_md=md,
                             num_splits=ns)

    def decode_call(i):
        mla.mla_decode_fwd(q, kvs[i % len(kvs)], bt, sl, 512, md, ns, softmax_scale=s1, v_scale=s2,
                           causal=w.causal, out=out, lse=lse, workspace=ws, stage="splits", **ext_for(i))

    def combine_call(i):
        mla.mla_decode_fwd(q, kvs[i % len(kvs)], bt, sl, 512, md, ns, softmax_scale=s1, v_scale=s2,
                           causal=w.causal, out=out, lse=lse, workspace=ws, stage="combine", **ext_for(i))

    def kernel_us(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if graphs:
            side = torch.cuda.Stream(dev)
            side.wait_stream(stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for i in range(K):
                        fn(W + i)
            stream.wait_stream(side)
            g.replay()
            torch.cuda.synchronize()
            e0.record(stream)
            g.replay()
            e1.record(stream)
        else:
            for i in range(2):
                fn(i)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(K):
                fn(W + i)
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    t_meta_us, t_dec_us, t_cmb_us = kernel_us(meta_call), kernel_us(decode_call), kernel_us(combine_call)

    # The whole decode call (mla_decode_fwd: split attention + combine) timed
    # per iteration with HIP events on the launch stream, after a pass that
    # reads a 1 GiB scratch buffer and so leaves the L2s and the last-level
    # cache cold.  (A read rather than the write that SURVEY.md's measurement
    # section suggests: a write leaves up to 256 MB of dirty lines whose
    # write-back would then compete with the timed call.)  The pass also keeps
    # the GPU busy while the host enqueues the events and the call, so no
    # host gap falls inside the timed interval.
    fwd_graph = None
    if graphs:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        fwd_graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(fwd_graph, stream=side):
                decode_call(0)
                combine_call(0)
        stream.wait_stream(side)
        torch.cuda.synchronize()
    scratch = torch.ones((1 << 28,), dtype=torch.int32, device=dev)     # 1 GiB
    n_fwd = max(5, args.fwd_iters)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_fwd + 5)]
    sums = []
    for i, (e0, e1) in enumerate(evs):
        sums.append(scratch.sum())
        e0.record(stream)
        if fwd_graph is not None:
            fwd_graph.replay()
        else:
            decode_call(0)
            combine_call(0)
        e1.record(stream)
    torch.cuda.synchronize()
    fwd = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs[5:])     # the first 5 are warm-ups
    fwd_med, fwd_min = fwd[len(fwd) // 2], fwd[0]
    # The same call back to back (warm clocks and caches): the two kernels'
    # averages from the K-launch graphs above.
    warm_us = t_dec_us + t_cmb_us
    del sums
    # Measured device-copy bandwidth beside the 8 TB/s nominal: a 1 GiB
    # device-to-device copy (read + write bytes), best of 5.
    scratch = scratch.view(torch.uint8)
    half = scratch[: 1 << 29]
    copy_us = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        scratch[1 << 29:].copy_(half)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_us.append(e0.elapsed_time(e1) * 1e3)
    copy_gbps = 2 * (1 << 29) / (min(copy_us) * 1e-6) / 1e9
    del scratch, half
    torch.cuda.empty_cache()

    # The outputs checked below come from whole steps.
    for i in range(len(kvs)):
        step(i)
    torch.cuda.synchronize()
    log(f"step {ms_step * 1e3:.1f} us ({timing}) | metadata {t_meta_us:.1f} us | decode {t_dec_us:.1f} us | "
        f"combine {t_cmb_us:.1f} us | mla_decode_fwd cold median {fwd_med:.1f} us min {fwd_min:.1f} us | "
        f"copy {copy_gbps:.0f} GB/s")

    # The last step's outputs, checked against the oracle in the cpu_baseline leg.
    out_np, lse_np = out.float().cpu().numpy(), lse.cpu().numpy()

    step_tflops = flops / (ms_step * 1e-3) / 1e12
    fwd_s = fwd_med * 1e-6
    dec_s = t_dec_us * 1e-6
    # Rooflines of the shape: HBM bytes at 8 TB/s; the matrix-core peak of the
    # arithmetic the kernels run (bf16 MFMA for a bf16 cache, fp8 MFMA for an
    # e4m3 cache, whose codes enter the fp8 matrix core as they are).  The
    # graded fraction is over the whole mla_decode_fwd call (split attention +
    # combine).
    t_hbm = alg_bytes / (HBM_PEAK_GBS * 1e9)
    t_bf16 = flops / (BF16_PEAK_TFLOPS * 1e12)
    t_fp8 = flops / (FP8_PEAK_TFLOPS * 1e12)
    mfma_peak = FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS
    t_mfma = t_fp8 if fp8 else t_bf16
    mfma_bound = t_mfma > t_hbm
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(flops / fwd_s / 1e12, 1), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(t_mfma / fwd_s, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(alg_bytes / fwd_s / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(t_hbm / fwd_s, 4)}
    plain = (not (args.sinks or args.split_cache or args.device_scales or args.fp8_query) and w.page_block_size == 64
             and args.batch_share == 1)
    roof.update({
        "traffic": measured_traffic(args.config) if plain else None,
        "timed": "mla_decode_fwd (split attention + combine), HIP events per call, cold caches",
        "t_median_us": round(fwd_med, 2), "t_min_us": round(fwd_min, 2), "iterations": len(fwd),
        "frac_at_min": round(max(t_hbm, t_mfma) / (fwd_min * 1e-6), 4),
        "back_to_back": {"us": round(warm_us, 2), "frac": round(max(t_hbm, t_mfma) / (warm_us * 1e-6), 4),
                         "timed": "decode and combine kernels, each as K launches back to back in a graph"},
        "alg_bytes_per_launch": alg_bytes, "alg_flops_per_launch": flops,
        "hbm_frac": round(t_hbm / fwd_s, 4), "bf16_mfma_frac": round(t_bf16 / fwd_s, 4),
        **({"fp8_mfma_frac": round(t_fp8 / fwd_s, 4)} if fp8 else {}),
        "roofline_us": {"hbm_8tbs": round(t_hbm * 1e6, 2), "bf16_mfma": round(t_bf16 * 1e6, 2),
                        **({"fp8_mfma": round(t_fp8 * 1e6, 2)} if fp8 else {})},
        "decode_only": {"kernel": f"mla_decode_kernel<{'fp8' if fp8 else 'bf16'}>", "avg_us": round(t_dec_us, 2),
                        "frac": round(max(t_hbm, t_mfma) / dec_s, 4)},
        "copy_gbps_measured": round(copy_gbps, 1),
        "copy_kind": "1 GiB device-to-device copy, read + write bytes, best of 5",
    })
    desc = WORKLOAD_NAMES[args.config] + f", H_k={w.num_heads_k} D=576 Dv=512 page={w.page_block_size} seed {args.config}"
    if not args.fp8_query:
        desc += ", bf16 q ~0.5*N(0,1)" if args.config == 3 else ", bf16 q ~N(0,1)"
    if fp8:
        desc += f", e4m3fn cache (per-tensor scale {w.k_scale:.4g}), fused bmm1={s1:.4g} bmm2={s2:.4g}"
    else:
        desc += f", bf16 cache ~N(0,1), scale 1/sqrt(576)"
    if args.sinks:
        desc += ", per-head sinks"
    if args.split_cache:
        desc += ", split latent/rope cache and q"
    if args.device_scales:
        desc += ", device-held bmm1/bmm2 scales"
    if args.fp8_query:
        desc += f", e4m3 q (per-tensor q_scale {q_scale:.4g} folded into bmm1)"
    if args.batch_share > 1:
        desc += (f"; one GPU's share of the batch over {args.batch_share} GPUs: its first {w.batch} sequences "
                 "and their cache blocks")
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
        "dtype": "fp8_e4m3" if fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": desc,
                   "batch": w.batch, "seq_len_q": w.s_q, "num_heads_q": w.num_heads_q, "causal": bool(w.causal),
                   "kv_dtype": w.kv_dtype, "total_keys": int(w.cache_seqlens.sum()), "num_parts": P,
                   **({"fixed_cost": args.fixed_cost} if args.fixed_cost else {}),
                   "kv_copies": len(kvs),
                   **({"batch_share_of_gpus": args.batch_share} if args.batch_share > 1 else {}),
                   "inputs": "+".join(n for n, f in (("sinks", args.sinks), ("split_cache_q", args.split_cache),
                                                     ("device_scales", args.device_scales),
                                                     ("fp8_query", args.fp8_query)) if f) or "plain"},
        "timing": timing,
        "kv_gbps_step": round(kv_bytes / (ms_step * 1e-3) / 1e9, 1),
        "kv_gbps_fwd": round(kv_bytes / fwd_s / 1e9, 1),
        "kernels_us": {"metadata": round(t_meta_us, 2), "decode": round(t_dec_us, 2),
                       "combine": round(t_cmb_us, 2)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], rec["check"] = cpu_baseline(w, s1, s2, sinks_np, out_np, lse_np, q_codes=q_codes)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
