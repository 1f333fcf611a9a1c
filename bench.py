#!/usr/bin/env python3
"""Benchmark: one step = the whole hot path (indexer scores -> Top-K -> sparse
MLA) over one batch of synthetic input, on one GPU.

Default workload: decode, batch 64, context 32768 per sequence, indexer 64 heads
x 128 fp8, Top-K 2048, MLA 128 heads x (512 + 64) bf16, paged cache with 64-token
pages and shuffled block tables.  Inputs are resident in HBM before timing; the
timed loop rotates over `--copies` distinct device copies of them so that no
step is served from the previous step's Infinity Cache contents.

Prints one JSON line (see the keys below).  `--gpus N` with N > 1 is refused:
this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query tokens/s for index+TopK+sparse-MLA; decode µs/step; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
# published fp32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2 (FMA) x 2 (packed fp32) x 2.4 GHz
FP32_VALU_PEAK_TFLOPS = 157.3


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "quant_decode", "quant_decode_tile128", "long_prefill", "cp_chunk_prefill",
                            "tiny_prefill", "mx_decode", "bf16_decode"])
    p.add_argument("--copies", type=int, default=3, help="distinct device copies of the inputs (decode)")
    p.add_argument("--order", type=int, default=0, choices=[0, 1, 2],
                   help="selection: Top-K positions score-sorted (0) or by position (1), or whole pages (2)")
    p.add_argument("--sweep-context", default=None, metavar="C1,C2,...",
                   help="no headline line: decode step time against context length (decode workloads), one JSON "
                        "line per context with per-position and page-aligned selection")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="budget for the CPU oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-breakdown", action="store_true")
    p.add_argument("--copy-probe", action="store_true",
                   help="after the run, launch a plain copy kernel of known size (HBM counter calibration)")
    p.add_argument("--traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no benchmark: turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                        "`bench.py --copy-probe` into profiles/<workload>_traffic.json")
    return p.parse_args()


# HBM traffic of the dominant kernels, from FETCH_SIZE / WRITE_SIZE counters
COPY_PROBE_BYTES = 1 << 30          # the calibration copy reads and writes this many bytes
TRAFFIC_KERNELS = {                 # roofline kernel -> (kernel-name substrings, sources it is built from)
    "sparse_mla": (("k_sparse_mla_mfma", "k_mla_combine"),
                   ("sparse_mla.hip", "sia_common.hpp", "sia_internal.hpp")),
    "index_scores": (("k_index_scores_fp8",),
                     ("indexer.hip", "index_core.hpp", "block_prims.hpp", "sia_common.hpp", "sia_internal.hpp")),
    # the fused call's steps 1 + 2: the on-chip method (ranges + candidate Top-K) or
    # the score-matrix method (scores + Top-K); count with --no-breakdown
    "index_topk": (("k_index_topk_ranges", "k_index_scores_fp8", "k_topk"),
                   ("index_topk.hip", "indexer.hip", "topk.hip", "index_core.hpp", "block_prims.hpp",
                    "sia_common.hpp", "sia_internal.hpp")),
}


def sources_digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_index_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(workload):
    return os.path.join(ROOT, "profiles", f"{workload}_traffic.json")


def write_traffic(workload, fetch_csv, write_csv):
    """Per-launch HBM bytes of each roofline kernel: counter KiB x (known copy
    bytes / the copy kernel's counter KiB), averaged over the kernel's launches."""
    import csv
    import collections

    def per_dispatch(path):
        rows = collections.defaultdict(float)
        names = {}
        for r in csv.DictReader(open(path)):
            d = r["Dispatch_Id"]
            rows[d] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
        return rows, names

    out = {"workload": workload, "copy_probe_bytes": COPY_PROBE_BYTES, "kernels": {}}
    for label, path in (("fetch", fetch_csv), ("write", write_csv)):
        vals, names = per_dispatch(path)
        copies = [vals[d] for d in vals if "elementwise" in names[d] and "MulFunctor" in names[d]]
        if not copies:
            raise SystemExit(f"no calibration copy kernel in {path}")
        factor = COPY_PROBE_BYTES / (1024.0 * sorted(copies)[len(copies) // 2])
        out[f"{label}_factor"] = factor
        for k, (subs, _) in TRAFFIC_KERNELS.items():
            # one launch of `k` = one call of its entry point.  The first of its
            # kernels that ran runs once per call; the others add every dispatch
            # they make (the split merge runs only when rows are split, and the
            # Top-K launches once per row-length class of a call with many rows)
            per = [sorted((d for d in vals if s in names[d]), key=int) for s in subs]
            per = [x for x in per if x]
            if not per:
                continue
            n = len(per[0])
            kib = sum(vals[d] for x in per for d in x) / n
            out["kernels"].setdefault(k, {})[f"{label}_bytes"] = kib * 1024.0 * factor
            out["kernels"][k]["launches"] = n
    for k, v in out["kernels"].items():
        v["traffic_bytes"] = v.get("fetch_bytes", 0.0) + v.get("write_bytes", 0.0)
        v["sources_sha256_16"] = sources_digest(TRAFFIC_KERNELS[k][1])
    os.makedirs(os.path.dirname(traffic_path(workload)), exist_ok=True)
    with open(traffic_path(workload), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def measured_traffic(workload, kernel):
    """Bytes per launch from the committed counter record, or None when there is
    none or the kernel's sources changed since it was taken."""
    try:
        with open(traffic_path(workload)) as fh:
            rec = json.load(fh)["kernels"][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("sources_sha256_16") != sources_digest(TRAFFIC_KERNELS[kernel][1]):
        return None
    return rec["traffic_bytes"]


def algorithmic_work(wl):
    """Bytes / flops per launch of each kernel, from the method's definition
    (inputs read once, outputs written once; the score round trip and split
    partials are not algorithmic)."""
    c = wl.cfg
    Hi, Di, H, Dc, Dr, K = c["Hi"], c["Di"], c["H"], c["Dc"], c["Dr"], c["K"]
    vis = (wl.q_pos.astype("int64") + 1)
    sel = vis.clip(max=K)
    if c["idx_dtype"] == "mxfp8":          # codes + one E8M0 byte per 32 elements
        key_b, q_b = Di + Di // 32, Hi * (Di + Di // 32) + 4 * Hi
    elif c["idx_dtype"] == "bf16":
        key_b, q_b = 2 * Di, Hi * 2 * Di + 4 * Hi
    else:
        key_b = Di + 4 if c["idx_dtype"] == "fp8" else 4 * Di
        q_b = Hi * Di * (1 if c["idx_dtype"] == "fp8" else 4) + 4 * Hi + 4
    if c["kv_dtype"] == "bf16":
        row_b = 2 * (Dc + Dr)
    elif c["kv_dtype"] == "fp8":     # codes, bf16 rope, and the row's share of its tile scales
        st, se = c["kv_scale"]
        row_b = Dc + 2 * Dr + 4.0 * (Dc // se) / st
    else:
        row_b = 4 * (Dc + Dr)
    elt = 4 if c["kv_dtype"] == "f32" else 2
    idx_bytes = float(vis.sum() * key_b + wl.Tq * q_b)
    idx_flops = float(vis.sum() * 2 * Hi * Di)
    mla_bytes = float(sel.sum() * (row_b + 4) + wl.Tq * H * ((Dc + Dr) + Dc) * elt)
    mla_flops = float(sel.sum() * 2 * H * ((Dc + Dr) + Dc))
    # Top-K over a score matrix reads each visible score once and writes K indices
    topk_bytes = float(vis.sum() * 4 + wl.Tq * K * 4)
    return {"index_scores": (idx_bytes, idx_flops), "topk": (topk_bytes, 0.0),
            "index_topk": (idx_bytes + float(wl.Tq * K * 4), idx_flops), "sparse_mla": (mla_bytes, mla_flops)}


def roofline_peak(wl, kernel):
    """(bound, peak, unit) of an entry point on this workload: decode steps are
    HBM-bound; prefill indexers run on the MFMA of their operand type, sparse
    MLA on the bf16 MFMA (fp8 latent rows are dequantized to bf16); the fp32
    path runs on the vector ALU."""
    c = wl.cfg
    if c["kind"] == "decode" or kernel == "topk":
        return "hbm", HBM_PEAK_GBS, "GB/s"
    dt = c["idx_dtype"] if kernel in ("index_scores", "index_topk") else c["kv_dtype"]
    if dt == "f32":
        return "alu", FP32_VALU_PEAK_TFLOPS, "TFLOP/s"
    if kernel in ("index_scores", "index_topk") and dt in ("fp8", "mxfp8"):
        return "mfma", FP8_PEAK_TFLOPS, "TFLOP/s"
    return "mfma", BF16_PEAK_TFLOPS, "TFLOP/s"


def cpu_baseline(wl, budget_s):
    """The oracle as it stands, on a bounded sample of the same workload."""
    import contextlib

    import numpy as np
    import oracle as O
    # the host cores this process may run on, capped by the thread limit the
    # environment sets for math libraries; BLAS is limited to that many threads
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        cores = min(cores, int(omp))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=cores)
    except Exception:
        limit = contextlib.nullcontext()
    K = wl.cfg["K"]
    rows = list(np.argsort(-wl.q_pos, kind="stable")) if wl.cfg["kind"] != "decode" else list(range(wl.Tq))
    rng = np.random.default_rng(0)
    if wl.cfg["kind"] != "decode":
        rows = list(rng.choice(wl.Tq, size=min(wl.Tq, 64), replace=False))
    done, t0 = [], time.perf_counter()
    with limit:
        for t in rows:
            O.index_select_attend(wl.oracle_indexer(), wl.q, wl.oracle_kv(), wl.oracle_seq(), K, wl.softmax_scale,
                                  rows=[int(t)])
            done.append(int(t))
            if time.perf_counter() - t0 >= budget_s and len(done) >= 2:
                break
    el = time.perf_counter() - t0
    vis_done = float(sum(int(wl.q_pos[t]) + 1 for t in done))
    vis_all = float((wl.q_pos.astype("int64") + 1).sum())
    rate = len(done) / el
    kind = "oracle"
    sample = f"{len(done)} of {wl.Tq} query tokens of the '{wl.name}' workload, whole path in float64"
    if wl.cfg["kind"] != "decode":
        # prefill rows differ in cost: scale by visible-key count
        rate = wl.Tq / (el * vis_all / vis_done)
        sample += "; rate extrapolated by visible-key count"
    return {"value": rate, "unit": "query tokens/s", "cores": int(cores), "kind": kind, "sample": sample,
            "seconds": round(el, 3)}


def dev(x):
    import numpy as np
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def upload_sets(wl, copies):
    """`copies` distinct device copies of the workload's inputs, each with its
    own workspace, output and index buffers."""
    import torch

    from sparse_index_attention_amd import sia
    c = wl.cfg
    K, H = c["K"], c["H"]
    sets = []
    base = None
    for i in range(copies):
        if base is None:
            seq = sia.SeqMap(dev(wl.q_seq), dev(wl.q_pos), dev(wl.block_table), wl.num_pages, wl.max_visible)
            if c["idx_dtype"] in ("f32", "bf16"):
                ix = sia.Indexer(dev(wl.iq), dev(wl.iw), dev(wl.ik))
            else:
                ix = sia.Indexer(dev(wl.iq), dev(wl.iw), dev(wl.ik), dev(wl.iq_scale), dev(wl.ik_scale))
            if c["kv_dtype"] == "fp8":
                kv = sia.LatentKV(dev(wl.kv), c["Dc"], c["Dr"], dev(wl.kv_scale), *c["kv_scale"])
            else:
                kv = sia.LatentKV(dev(wl.kv), c["Dc"], c["Dr"])
            q = dev(wl.q)
            base = (seq, ix, q, kv)
        else:
            seq, ix, q, kv = base
            ix = sia.Indexer(ix.q.clone(), ix.w.clone(), ix.k_pool.clone(),
                             None if ix.q_scale is None else ix.q_scale.clone(),
                             None if ix.k_scale is None else ix.k_scale.clone())
            kv = sia.LatentKV(kv.pool.clone(), kv.latent_dim, kv.rope_dim,
                              None if kv.scale is None else kv.scale.clone(), kv.scale_tokens, kv.scale_elems)
            q = q.clone()
            seq = sia.SeqMap(seq.q_seq.clone(), seq.q_pos.clone(), seq.block_table.clone(), seq.num_pages,
                             seq.max_visible)
        n_ws = sia.workspace_size(sia.OP_INDEX_SELECT_ATTEND, seq, K, H, c["Dc"])
        ws = torch.empty(n_ws, dtype=torch.uint8, device="cuda")
        out = torch.empty(wl.Tq, H, c["Dc"], dtype=q.dtype, device="cuda")
        idx = torch.empty(wl.Tq, K, dtype=torch.int32, device="cuda")
        sets.append(dict(seq=seq, ix=ix, q=q, kv=kv, ws=ws, out=out, idx=idx))
    torch.cuda.synchronize()
    return sets


def timed_calls(calls, steps, warmup, stream):
    """Average µs of each (name, fn(i)) over `steps` iterations after `warmup`,
    from HIP events recorded around every call on the launch stream."""
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    for i in range(warmup + steps):
        rec = ev[i - warmup] if i >= warmup else None
        for k, (_, fn) in enumerate(calls):
            if rec:
                rec[k].record(stream)
            fn(i)
        if rec:
            rec[-1].record(stream)
    torch.cuda.synchronize()
    return {nm: round(1e3 * sum(r[k].elapsed_time(r[k + 1]) for r in ev) / steps, 2)
            for k, (nm, _) in enumerate(calls)}


def sweep_context(args):
    """Decode step time against context length (batch and dims of the decode
    workload), for per-position Top-K and for page-aligned selection."""
    import torch

    from sparse_index_attention_amd import sia
    from sparse_index_attention_amd import workloads as W
    if W.CONFIGS[args.workload]["kind"] != "decode":
        print("--sweep-context needs a decode workload", file=sys.stderr)
        sys.exit(2)
    stream = torch.cuda.current_stream()
    for ctx in [int(x) for x in args.sweep_context.split(",")]:
        print(f"[sweep] context {ctx}: generating", file=sys.stderr, flush=True)
        wl = W.make_workload(args.workload, overrides={"ctx": ctx})
        c = wl.cfg
        K, H = c["K"], c["H"]
        copies = max(1, args.copies)
        sets = upload_sets(wl, copies)
        mws = torch.empty(max(sia.workspace_size(sia.OP_MLA_DECODE, sets[0]["seq"], K, H, c["Dc"]), 1),
                          dtype=torch.uint8, device="cuda")
        tws = [torch.empty(max(sia.workspace_size(sia.OP_INDEX_TOPK, st["seq"], K, 1, 1), 1), dtype=torch.uint8,
                           device="cuda") for st in sets]
        point = {"sweep": "decode_context", "workload": args.workload, "context": ctx,
                 "batch": int(len(wl.seq_lens)), "K": K, "input_copies": copies}
        for label, order in (("positions", 0), ("pages", sia.SELECT_PAGES)):
            def whole(i, order=order):
                st = sets[i % copies]
                sia.index_select_attend(st["ix"], st["q"], st["kv"], st["seq"], K, wl.softmax_scale, order=order,
                                        idx_out=st["idx"], out=st["out"], ws=st["ws"], stream=stream)

            def sel(i, order=order):
                st = sets[i % copies]
                sia.index_topk(st["ix"], st["seq"], K, order=order, idx=st["idx"], ws=tws[i % copies],
                               stream=stream)

            def mla(i):
                st = sets[i % copies]
                sia.sparse_mla_decode(st["q"], st["kv"], st["seq"], st["idx"], K, wl.softmax_scale, out=st["out"],
                                      ws=mws, stream=stream)

            t_step = timed_calls([("step", whole)], args.steps, args.warmup, stream)["step"]
            parts = timed_calls([("index_topk", sel), ("sparse_mla", mla)], args.steps, args.warmup, stream)
            point[label] = {"us_per_step": t_step, "query_tokens_per_s": round(wl.Tq / (t_step * 1e-6), 1),
                            **{k + "_us": v for k, v in parts.items()}}
        print(json.dumps(point), flush=True)
        del sets, mws, tws, wl
        torch.cuda.empty_cache()


def main():
    args = parse()
    if args.traffic:
        write_traffic(args.workload, *args.traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU path is a design note, "
              "not part of this build.", file=sys.stderr)
        sys.exit(2)
    if args.sweep_context:
        import torch
        if not torch.cuda.is_available():
            print("bench.py needs a GPU", file=sys.stderr)
            sys.exit(1)
        sweep_context(args)
        return

    import numpy as np
    import torch

    from sparse_index_attention_amd import sia
    from sparse_index_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sia.lib()
    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    t_gen = time.perf_counter()
    wl = W.make_workload(args.workload)
    c = wl.cfg
    K, H = c["K"], c["H"]
    print(f"[bench] generated in {time.perf_counter() - t_gen:.1f}s; uploading", file=sys.stderr, flush=True)

    decode = c["kind"] == "decode"
    copies = max(1, args.copies) if decode else 1
    sets = upload_sets(wl, copies)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(i):
        s = sets[i % copies]
        sia.index_select_attend(s["ix"], s["q"], s["kv"], s["seq"], K, wl.softmax_scale, order=args.order,
                                idx_out=s["idx"], out=s["out"], ws=s["ws"], stream=stream)

    print("[bench] warmup", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print("[bench] timing", file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / args.steps
    value = wl.Tq / (ms_per_step / 1e3)

    # per-kernel breakdown, measured live with events on the launch stream
    work = algorithmic_work(wl)
    breakdown = {}
    if not args.no_breakdown:
        ld = (wl.max_visible + 63) // 64 * 64
        scores = [torch.empty(wl.Tq, ld, dtype=torch.float32, device="cuda") for _ in range(copies)]
        nmla = sia.workspace_size(sia.OP_MLA_DECODE, sets[0]["seq"], K, H, c["Dc"]) if c["kv_dtype"] != "f32" else 0
        mws = torch.empty(max(nmla, 1), dtype=torch.uint8, device="cuda")
        mla_fn = sia.sparse_mla_decode if sia.workspace_size(sia.OP_MLA_DECODE, sets[0]["seq"], K, H, c["Dc"]) > 0 \
            else sia.sparse_mla_prefill
        tws = [torch.empty(max(sia.workspace_size(sia.OP_INDEX_TOPK, st["seq"], K, 1, 1), 1), dtype=torch.uint8,
                           device="cuda") for st in sets]

        def timed(calls):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
            for i in range(args.warmup + args.steps):
                rec = ev[i - args.warmup] if i >= args.warmup else None
                for k, (_, fn) in enumerate(calls):
                    if rec:
                        rec[k].record(stream)
                    fn(i)
                if rec:
                    rec[-1].record(stream)
            torch.cuda.synchronize()
            for k, (nm, _) in enumerate(calls):
                breakdown[nm] = round(1e3 * sum(r[k].elapsed_time(r[k + 1]) for r in ev) / args.steps, 2)

        def sel(i):   # steps 1 + 2 as the fused call runs them (method chosen by the library)
            st = sets[i % copies]
            sia.index_topk(st["ix"], st["seq"], K, order=args.order, idx=st["idx"], ws=tws[i % copies], stream=stream)

        def mla(i):
            st = sets[i % copies]
            mla_fn(st["q"], st["kv"], st["seq"], st["idx"], K, wl.softmax_scale, out=st["out"], ws=mws, stream=stream)

        def scr(i):   # the indexer kernel alone, then Top-K over its score matrix
            st = sets[i % copies]
            sia.index_scores(st["ix"], st["seq"], scores[i % copies], stream=stream)

        pws = [torch.empty(max(sia.workspace_size(sia.OP_TOPK_PAGES, st["seq"], K, 1, 1), 1), dtype=torch.uint8,
                           device="cuda") for st in sets] if args.order == sia.SELECT_PAGES else None

        def tk(i):
            st = sets[i % copies]
            if args.order == sia.SELECT_PAGES:
                sia.topk_pages(scores[i % copies], st["seq"], K, idx=st["idx"], ws=pws[i % copies], stream=stream)
            else:
                sia.topk(scores[i % copies], st["seq"], K, order=args.order, idx=st["idx"], stream=stream)

        timed([("index_topk", sel), ("sparse_mla", mla)])
        timed([("index_scores", scr), ("topk", tk)])
        breakdown["index_topk_method"] = sia.index_topk_method(sets[0]["ix"], sets[0]["seq"])
        del scores

    roofline = None
    if breakdown:
        # the dominant one of the kernels the timed step runs: steps 1 + 2 are
        # one fused pair on chip (ranges + candidate Top-K), or two kernels
        # through the score matrix (scores, then Top-K)
        if breakdown["index_topk_method"] == "scores":
            candidates = ("index_scores", "topk", "sparse_mla")
        else:
            candidates = ("index_topk", "sparse_mla")
        dom = max(candidates, key=lambda n: breakdown[n])
        by, fl = work[dom]
        us = breakdown[dom]
        bound, peak, unit = roofline_peak(wl, dom)
        if bound == "hbm":
            achieved = by / (us * 1e-6) / 1e9
            roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                        "frac": round(achieved / peak, 4), "traffic": measured_traffic(args.workload, dom),
                        "algorithmic_bytes": by, "avg_us": us}
        else:
            achieved = fl / (us * 1e-6) / 1e12
            roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                        "frac": round(achieved / peak, 4), "traffic": measured_traffic(args.workload, dom),
                        "algorithmic_flops": fl, "avg_us": us}
        if dom in ("index_topk", "index_scores", "topk"):
            roofline["index_topk_method"] = breakdown.get("index_topk_method")

    if args.copy_probe:
        # calibration for the HBM byte counters: one elementwise copy of known size
        src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, args.cpu_seconds)

    cfg = {"workload": args.workload, "queries": wl.Tq, "K": K, "indexer": f"{c['Hi']}x{c['Di']} {c['idx_dtype']}",
           "mla": f"{H} heads, {c['Dc']}+{c['Dr']} {c['kv_dtype']}", "page_size": 64, "topk_order": args.order,
           "input_copies": copies}
    if decode:
        cfg.update(batch=int(len(wl.seq_lens)), context=int(wl.seq_lens.max()))
    else:
        cfg.update(max_visible=wl.max_visible)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2), "wall_s": round(wall, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"fp8": "fp8+bf16", "mxfp8": "mxfp8+bf16", "bf16": "bf16"}.get(c["idx_dtype"], "f32"), "data": "synthetic",
        "config": cfg, "breakdown_us": breakdown, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
