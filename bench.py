#!/usr/bin/env python3
"""Benchmark of the lightning-indexer hot path on one MI355X.

One step = one fused prefill indexer + top-k over a single L=32768 sequence
(H=64 index heads, D=128, k=2048, fp8 e4m3 q/k with per-token scales, bf16
head weights, 1% planted heavy keys) followed by one decode indexer + top-k
over a batch of 32 sequences with 131072-token fp8 key caches.  Inputs are
seeded synthetic data generated on the device before timing; the timed region
holds only the two library calls.

Prints one JSON line.  ``value`` is the prefill throughput in algorithmic
TFLOP/s (2*H*D multiply-adds per causal (query, key) pair); the decode rate
in algorithmic GB/s is reported beside it.  Other workloads
(``--workload tiny|prefill_196k|prefill_32k_chunked|prefill_ragged|prefill_32k_h128|
prefill_32k_bf16|decode_128k_paged|decode_128k_ragged|decode_128k_h128|fs_47|fs_decode_47|
mli_decode_47``)
print their own line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer prefill TFLOP/s (%fp8 MFMA peak) + decode HBM GB/s at 128K ctx"
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def prefill_flops(L, H, D):
    return 2.0 * H * D * L * (L + 1) / 2.0


def decode_bytes(lens, H, D, topk, B):
    # cache bytes + per-token scales + queries + weights + output indices
    return float(sum(int(n) for n in lens) * (D + 4) + B * H * D * 2 + B * H * 2 + B * topk * 4)


def kernel_source_hash():
    """Hash of the kernel sources with comments and blank lines removed, so a
    counter summary stays attached to the code it was taken on."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_token_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(f.encode())
        h.update(text.encode())
    return h.hexdigest()[:16]


def load_traffic(name, per_launch_units):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def cpu_workers():
    """Host cores this process may use, at most 16 (one GPU's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _cpu_prefill_worker(job):
    """One worker of the prefill baseline: the fp64 oracle, BLAS on one
    thread, over seeded batches of query rows until its time budget is spent
    (or over the given rows).  Returns (causal pairs, rows, oracle seconds)."""
    cfg_name, seed, budget_s, fixed_rows = job
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from synth import gen
    cfg = gen.CONFIGS[cfg_name]
    L, topk = cfg["L"], cfg["topk"]
    keys = gen.prefill_inputs(cfg, rows=[0])
    rng = np.random.default_rng(seed)
    pairs = nrows = 0
    el = 0.0
    with threadpool_limits(1):
        batches = [np.asarray(fixed_rows)] if fixed_rows is not None else None
        while True:
            if batches is not None:
                if not batches:
                    break
                rows = batches.pop()
            else:
                if el >= budget_s:
                    break
                rows = np.sort(rng.choice(L, size=8, replace=False))
            inp = gen.prefill_inputs(cfg, rows=rows, with_keys=False)
            ts = time.perf_counter()
            oracle.prefill(inp["q"], inp["q_scale"], keys["k"], keys["k_scale"], inp["w"], cfg["dtype"], topk,
                           rows=rows)
            el += time.perf_counter() - ts
            pairs += int(np.sum(rows + 1))
            nrows += len(rows)
    return pairs, nrows, el


def _cpu_fs_worker(job):
    """One worker of the layer-reuse baseline: the fp64 oracle on seeded
    batches of query rows of one layer of the 47-layer workload, until its
    time budget is spent (the layer's keys are built outside the timed part).
    Returns (causal pairs, rows, oracle seconds)."""
    layer, seed, budget_s = job
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    from synth import gen
    cfg = gen.CONFIGS["fs_47"]
    L, topk = cfg["L"], cfg["topk"]
    keys = gen.fs_layer_inputs(cfg, layer, rows=[0])
    rng = np.random.default_rng(seed)
    pairs = nrows = 0
    el = 0.0
    with threadpool_limits(1):
        while el < budget_s:
            rows = np.sort(rng.choice(L, size=8, replace=False))
            inp = gen.fs_layer_inputs(cfg, layer, rows=rows, with_keys=False)
            ts = time.perf_counter()
            oracle.prefill(inp["q"], inp["q_scale"], keys["k"], keys["k_scale"], inp["w"], cfg["dtype"], topk,
                           rows=rows)
            el += time.perf_counter() - ts
            pairs += int(np.sum(rows + 1))
            nrows += len(rows)
    return pairs, nrows, el


def _cpu_decode_worker(job):
    """One worker of the decode baseline: the fp64 oracle over the given
    sequences, one at a time (inputs generated outside the timed part).
    Returns (algorithmic bytes, sequences, oracle seconds)."""
    cfg_name, seqs = job
    from threadpoolctl import threadpool_limits
    import oracle
    from synth import gen
    cfg = gen.CONFIGS[cfg_name]
    H, D, topk = cfg["H"], cfg["D"], cfg["topk"]
    nbytes = 0.0
    el = 0.0
    with threadpool_limits(1):
        for b in seqs:
            inp = gen.decode_inputs(cfg, seqs=[b])
            ts = time.perf_counter()
            oracle.decode(inp["q"], inp["w"], inp["cache"], inp["k_scale"], inp["lens"], topk)
            el += time.perf_counter() - ts
            nbytes += decode_bytes(inp["lens"], H, D, topk, 1)
    return nbytes, len(seqs), el


def cpu_baseline_workload(name, budget_s=12.0):
    """The fp64 oracle on a seeded row sample of a secondary prefill workload,
    on the host cores in worker processes: L=196608 (rows of the one
    sequence) or the 47-layer workload (rows of every third layer, one layer
    per worker).  None for the other workloads."""
    import multiprocessing as mp
    from synth import gen
    nw = cpu_workers()
    ctx = mp.get_context("spawn")
    if name == "prefill_196k":
        jobs, worker, layers = [("prefill_196k", 100 + i, budget_s, None) for i in range(nw)], _cpu_prefill_worker, 1
        cfg = gen.CONFIGS["prefill_196k"]
    elif name == "fs_47":
        cfg = gen.CONFIGS["fs_47"]
        jobs, worker, layers = [((3 * i) % cfg["N"], 100 + i, budget_s) for i in range(nw)], _cpu_fs_worker, cfg["N"]
    else:
        return None
    with ctx.Pool(nw) as pool:
        t0 = time.perf_counter()
        res = pool.map(worker, jobs)
        wall = time.perf_counter() - t0
    pairs = sum(r[0] for r in res)
    nrows = sum(r[1] for r in res)
    busy = max(r[2] for r in res)
    L, H, D = cfg["L"], cfg["H"], cfg["D"]
    what = f"L={L}" if layers == 1 else f"{layers}-layer L={L}"
    return {"value": round(pairs * 2.0 * H * D / busy / 1e12, 6), "unit": "TFLOP/s", "cores": nw, "kind": "oracle",
            "sample": f"{nrows} seeded query rows of the {what} prefill ({pairs} causal pairs) on {nw} worker "
                      f"processes, {busy:.1f} s of oracle time each (fp64, one BLAS thread per worker)",
            "rows_per_s": round(nrows / busy, 2),
            "full_workload_s_extrapolated": round(layers * L * (L + 1) / 2 / (pairs / busy), 1),
            "wall_s": round(wall, 1)}


def cpu_baseline(budget_s=12.0):
    """The fp64 oracle as it stands, on the host cores in parallel worker
    processes (one BLAS thread each), started before anything touches the
    GPU.  Headline: a seeded row sample of the L=32768 prefill (each worker
    runs rows for `budget_s` seconds); beside it the whole small prefill
    (L=2048) and the whole B=32 x 131072 decode."""
    import multiprocessing as mp
    import numpy as np
    from synth import gen
    nw = cpu_workers()
    ctx = mp.get_context("spawn")
    out = {}
    with ctx.Pool(nw) as pool:
        t0 = time.perf_counter()
        res = pool.map(_cpu_prefill_worker, [("prefill_32k", 100 + i, budget_s, None) for i in range(nw)])
        wall = time.perf_counter() - t0
        pairs = sum(r[0] for r in res)
        nrows = sum(r[1] for r in res)
        busy = max(r[2] for r in res)
        cfg = gen.CONFIGS["prefill_32k"]
        L, H, D = cfg["L"], cfg["H"], cfg["D"]
        tflops = pairs * 2.0 * H * D / busy / 1e12
        out = {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": nw, "kind": "oracle",
               "sample": f"{nrows} seeded query rows of the L={L} prefill ({pairs} causal pairs) on {nw} worker "
                         f"processes, {busy:.1f} s of oracle time each (fp64, one BLAS thread per worker)",
               "rows_per_s": round(nrows / busy, 2),
               "full_workload_s_extrapolated": round(L * (L + 1) / 2 / (pairs / busy), 1),
               "wall_s": round(wall, 1)}
        tcfg = gen.CONFIGS["tiny"]
        chunks = np.array_split(np.arange(tcfg["L"]), nw)
        t0 = time.perf_counter()
        res = pool.map(_cpu_prefill_worker, [("tiny", 0, 0.0, c) for c in chunks if len(c)])
        wall = time.perf_counter() - t0
        pairs = sum(r[0] for r in res)
        tfl = 2.0 * tcfg["H"] * tcfg["D"] * pairs / wall / 1e12
        out["tiny_full"] = {"value": round(tfl, 6), "unit": "TFLOP/s", "wall_s": round(wall, 2),
                            "sample": f"the whole L={tcfg['L']} H={tcfg['H']} D={tcfg['D']} bf16 prefill "
                                      f"(every row), wall time on {nw} workers"}
        dcfg = gen.CONFIGS["decode_128k"]
        parts = np.array_split(np.arange(dcfg["B"]), nw)
        t0 = time.perf_counter()
        res = pool.map(_cpu_decode_worker, [("decode_128k", [int(b) for b in c]) for c in parts if len(c)])
        wall = time.perf_counter() - t0
        nbytes = sum(r[0] for r in res)
        busy = max(r[2] for r in res)
        out["decode_128k_full"] = {"value": round(nbytes / busy / 1e9, 4), "unit": "GB/s",
                                   "us_per_call": round(busy * 1e6, 0),
                                   "sample": f"the whole B={dcfg['B']} x {dcfg['Lmax']} decode, sequences split "
                                             f"over {nw} workers; time = the busiest worker's oracle seconds"}
    return out


def measure_peaks(dev):
    """Measured device peaks on this machine: MFMA-only kernels (fp8, bf16) and
    HBM read and copy kernels over 2 GiB (libdsa_peak.so)."""
    import torch
    from sparse_attention_token_02_amd import peak
    f8, clk8 = peak.mfma("fp8", iters=5)
    b16, clk16 = peak.mfma("bf16", iters=5)
    buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    rd = peak.hbm_read(buf, iters=5)
    cp = peak.hbm_copy(buf[: 1 << 30], dst, iters=5)
    del buf, dst
    torch.cuda.empty_cache()
    return {"mfma_fp8_tflops": round(f8, 1), "mfma_fp8_clock_mhz": round(clk8, 0),
            "mfma_bf16_tflops": round(b16, 1), "mfma_bf16_clock_mhz": round(clk16, 0),
            "hbm_read_gbps": round(rd, 1), "hbm_copy_gbps": round(cp, 1)}


def run_main(args):
    import torch
    import sparse_attention_token_02_amd as dsa
    from synth import gen
    from synth.gpu import DeviceGen

    dev = torch.device("cuda:0")
    g = DeviceGen(dev)
    pcfg = gen.CONFIGS["prefill_32k"]
    dcfg = gen.CONFIGS["decode_128k"]
    L, H, D, topk = pcfg["L"], pcfg["H"], pcfg["D"], pcfg["topk"]
    log("generating prefill inputs")
    p = g.prefill_inputs(pcfg)
    out_idx = torch.empty((L, topk), dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.dsa_indexer_topk_prefill_workspace(L, H, D, topk, "fp8"), dtype=torch.uint8, device=dev)
    log("generating decode inputs (two cache copies, each larger than the 256 MB MALL)")
    dd = [g.decode_inputs(dcfg)]
    dd.append({k: (v.clone() if hasattr(v, "clone") else v) for k, v in dd[0].items()})
    B, Lmax = dcfg["B"], dcfg["Lmax"]
    d_idx = torch.empty((B, topk), dtype=torch.int32, device=dev)
    dws = torch.empty(dsa.dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def prefill():
        dsa.dsa_indexer_topk_prefill(p["q"], p["q_scale"], p["k"], p["k_scale"], p["w"], topk, "fp8",
                                     out_idx=out_idx, workspace=ws, stream=stream)

    turn = [0]

    def decode():
        d = dd[turn[0] & 1]
        turn[0] += 1
        dsa.dsa_indexer_topk_decode(d["q"], d["w"], d["cache"], d["k_scale"], d["lens"], topk,
                                    out_idx=d_idx, workspace=dws, stream=stream)

    log("warmup + timed steps")
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()
    ev = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        prefill()
        e[1].record(stream)
        decode()
        e[2].record(stream)
        ev.append(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    # decode on its own (outside the timed steps): back to back, alternating
    # the two cache copies, with no prefill writing back its lines in between
    alone = time_calls(decode, max(5, args.steps), 2, stream)
    pf_ms = sorted(a.elapsed_time(b) for a, b, _ in ev)
    dc_ms = sorted(b.elapsed_time(c) for _, b, c in ev)
    med = lambda xs: xs[len(xs) // 2]
    pf_avg = sum(pf_ms) / len(pf_ms)
    dc_avg = sum(dc_ms) / len(dc_ms)
    flops = prefill_flops(L, H, D)
    lens = gen.decode_lens(dcfg)
    dbytes = decode_bytes(lens, H, D, topk, B)
    pf_tflops = flops / (pf_avg * 1e-3) / 1e12
    dc_gbps = dbytes / (dc_avg * 1e-3) / 1e9
    ms_per_step = wall * 1e3 / args.steps
    res = {
        "metric": METRIC,
        "value": round(pf_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate); decode e4m3 keys x bf16 query as two e4m3 limbs",
        "data": "synthetic (seeded, generated on device)",
        "config": {"workload": "prefill L=32768 H=64 D=128 k=2048 fp8 + decode B=32 x 131072 fp8 cache k=2048",
                   "prefill_L": L, "heads": H, "head_dim": D, "topk": topk, "decode_batch": B,
                   "decode_ctx": Lmax},
        "prefill_ms": round(pf_avg, 4), "prefill_ms_median": round(med(pf_ms), 4),
        "prefill_rows_per_s": round(L / (pf_avg * 1e-3), 1),
        "decode_us": round(dc_avg * 1e3, 2), "decode_us_median": round(med(dc_ms) * 1e3, 2),
        "decode_alone_us": round(sum(alone) / len(alone) * 1e3, 2),
        "decode_GBps": round(dc_gbps, 1),
        "decode_rows_per_s": round(B / (dc_avg * 1e-3), 1),
        "roofline": {"bound": "mfma", "achieved": round(pf_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(pf_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": load_traffic("prefill_32k", 1)},
        "roofline_decode": {"bound": "hbm", "achieved": round(dc_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": round(dc_gbps / PEAK_HBM_GBPS, 4), "traffic": load_traffic("decode_128k", 1)},
        "kernel_source_hash": kernel_source_hash(),
    }
    log("measured peaks")
    pk = measure_peaks(dev)
    res["peaks_measured"] = pk
    res["roofline"]["peak_measured"] = pk["mfma_fp8_tflops"]
    res["roofline"]["frac_measured"] = round(pf_tflops / pk["mfma_fp8_tflops"], 4)
    res["roofline_decode"]["peak_measured"] = pk["hbm_read_gbps"]
    res["roofline_decode"]["frac_measured"] = round(dc_gbps / pk["hbm_read_gbps"], 4)
    res["cpu_baseline"] = args.cpu_result
    return res


def run_workload(args):
    import torch
    import sparse_attention_token_02_amd as dsa
    from synth import gen
    from synth.gpu import DeviceGen
    dev = torch.device("cuda:0")
    g = DeviceGen(dev)
    stream = torch.cuda.current_stream(dev)
    name = args.workload
    if name in ("tiny", "prefill_196k", "prefill_32k", "prefill_32k_h128", "prefill_32k_bf16"):
        cfg = shape_config(gen, name)
        L, H, D, topk = cfg["L"], cfg["H"], cfg["D"], cfg["topk"]
        p = g.prefill_inputs(cfg)
        out = torch.empty((L, topk), dtype=torch.int32, device=dev)
        ws = torch.empty(dsa.dsa_indexer_topk_prefill_workspace(L, H, D, topk, cfg["dtype"]), dtype=torch.uint8,
                         device=dev)
        fn = lambda: dsa.dsa_indexer_topk_prefill(p["q"], p["q_scale"], p["k"], p["k_scale"], p["w"], topk,
                                                  cfg["dtype"], out_idx=out, workspace=ws, stream=stream)
        ms = time_calls(fn, args.steps, args.warmup, stream)
        avg = sum(ms) / len(ms)
        tf = prefill_flops(L, H, D) / (avg * 1e-3) / 1e12
        peak = PEAK_FP8_TFLOPS if cfg["dtype"] == "fp8" else PEAK_BF16_TFLOPS
        return {"metric": METRIC, "workload": name, "value": round(tf, 2), "unit": "TFLOP/s",
                "ms_per_call": round(avg, 4), "rows_per_s": round(L / (avg * 1e-3), 1),
                "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": peak, "unit": "TFLOP/s",
                             "frac": round(tf / peak, 4), "traffic": None},
                "config": {"workload": name, **{k: v for k, v in cfg.items() if k != "kind"}}}
    if name == "prefill_ragged":
        return run_prefill_ragged(args, g, dsa, gen, stream)
    if name == "decode_128k_paged":
        return run_decode_paged(args, g, dsa, gen, stream)
    if name == "decode_128k_ragged":
        return run_decode_ragged(args, g, dsa, gen, stream)
    if name == "decode_128k_h128":
        return run_decode_ragged(args, g, dsa, gen, stream, cfg=shape_config(gen, name), name=name)
    if name == "prefill_32k_chunked":
        return run_prefill_chunked(args, g, dsa, gen, stream)
    if name == "fs_47":
        return run_fs(args, g, dsa, gen, stream)
    if name == "fs_decode_47":
        return run_fs_decode(args, g, dsa, gen, stream)
    if name == "mli_decode_47":
        return run_mli_decode(args, g, dsa, gen, stream)
    raise SystemExit(f"unknown workload {name}")


def run_decode_paged(args, g, dsa, gen, stream):
    """The B=32 x 131072 decode with the cache in 64-token pages in a seeded
    shuffled order, against the same cache stored contiguously (both timed
    back to back on one copy of the data)."""
    import torch
    cfg = gen.CONFIGS["decode_128k"]
    B, Lmax, H, D, topk = cfg["B"], cfg["Lmax"], cfg["H"], cfg["D"], cfg["topk"]
    P = 64
    dev = g.device
    d = g.decode_inputs(cfg)
    mb = Lmax // P
    perm = torch.randperm(B * mb, generator=torch.Generator().manual_seed(1)).to(dev)
    pages = torch.empty((B * mb, P, D), dtype=torch.uint8, device=dev)
    spages = torch.empty((B * mb, P), dtype=torch.float32, device=dev)
    pages.index_copy_(0, perm, d["cache"].reshape(B * mb, P, D))
    spages.index_copy_(0, perm, d["k_scale"].reshape(B * mb, P))
    table = perm.to(torch.int32).reshape(B, mb).contiguous()
    out = torch.empty((B, topk), dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk), dtype=torch.uint8, device=dev)
    contiguous = lambda: dsa.dsa_indexer_topk_decode(d["q"], d["w"], d["cache"], d["k_scale"], d["lens"], topk,
                                                     out_idx=out, workspace=ws, stream=stream)
    paged = lambda: dsa.dsa_indexer_topk_decode_paged(d["q"], d["w"], pages, spages, table, d["lens"], topk,
                                                      out_idx=out, workspace=ws, stream=stream)
    # two interleaved passes, each warmed up, so that neither layout is timed
    # alone while the device is still settling
    t_c = t_p = 0.0
    for _ in range(2):
        t_c += sum(time_calls(contiguous, args.steps, args.warmup, stream)) / args.steps / 2
        t_p += sum(time_calls(paged, args.steps, args.warmup, stream)) / args.steps / 2
    nbytes = decode_bytes(gen.decode_lens(cfg), H, D, topk, B)
    gbps = nbytes / (t_p * 1e-3) / 1e9
    return {"metric": METRIC, "workload": "decode_128k_paged", "value": round(gbps, 1), "unit": "GB/s",
            "paged_us": round(t_p * 1e3, 2), "contiguous_us": round(t_c * 1e3, 2), "page_size": P,
            "rows_per_s": round(B / (t_p * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None},
            "config": {"workload": "decode_128k_paged", "B": B, "Lmax": Lmax, "H": H, "D": D, "topk": topk,
                       "page_size": P}}


def shape_config(gen, name):
    """The recipe of a named workload; the _h128 and _bf16 variants are the
    32K prefill and the 128K decode at 128 index heads (head weights scaled
    by 1/sqrt(128)), and the 32K prefill with bf16 queries and keys."""
    import math
    import numpy as np
    w128 = float(np.float32(math.sqrt(128.0)))
    if name == "prefill_32k_h128":
        return dict(gen.CONFIGS["prefill_32k"], H=128, w_div=w128)
    if name == "prefill_32k_bf16":
        return dict(gen.CONFIGS["prefill_32k"], dtype="bf16", qk_div=8.0)
    if name == "decode_128k_h128":
        return dict(gen.CONFIGS["decode_128k"], H=128, w_div=w128)
    return gen.CONFIGS[name]


def run_decode_ragged(args, g, dsa, gen, stream, cfg=None, name="decode_128k_ragged"):
    """The B=32 decode with sequence lengths uniform in [65536, 131072]
    (seeded), or the decode recipe `cfg`; two copies of the cache alternating
    so that reads come from HBM, as in the main benchmark."""
    import torch
    cfg = cfg or gen.ragged_decode_config()
    B, Lmax, H, D, topk = cfg["B"], cfg["Lmax"], cfg["H"], cfg["D"], cfg["topk"]
    dd = [g.decode_inputs(cfg)]
    dd.append({k: (v.clone() if hasattr(v, "clone") else v) for k, v in dd[0].items()})
    out = torch.empty((B, topk), dtype=torch.int32, device=g.device)
    ws = torch.empty(dsa.dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk), dtype=torch.uint8, device=g.device)
    turn = [0]

    def call():
        d = dd[turn[0] & 1]
        turn[0] += 1
        dsa.dsa_indexer_topk_decode(d["q"], d["w"], d["cache"], d["k_scale"], d["lens"], topk, out_idx=out,
                                    workspace=ws, stream=stream)

    ms = time_calls(call, args.steps, args.warmup, stream)
    avg = sum(ms) / len(ms)
    lens = gen.decode_lens(cfg)
    nbytes = decode_bytes(lens, H, D, topk, B)
    gbps = nbytes / (avg * 1e-3) / 1e9
    return {"metric": METRIC, "workload": name, "value": round(gbps, 1), "unit": "GB/s",
            "us_per_call": round(avg * 1e3, 2), "tokens": int(sum(int(n) for n in lens)),
            "rows_per_s": round(B / (avg * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None},
            "config": {"workload": name, "B": B, "Lmax": Lmax, "H": H, "D": D, "topk": topk,
                       "lens": "uniform in [Lmax/2, Lmax], seeded" if cfg.get("ragged") else "all Lmax"}}


def run_prefill_ragged(args, g, dsa, gen, stream):
    """A packed batch of 24 whole sequences of seeded lengths in [512, 16384]
    (fp8, H=64, D=128, k=2048): one ragged launch, against one call per
    sequence on the same data."""
    import numpy as np
    import torch
    base = gen.CONFIGS["prefill_32k"]
    H, D, topk = base["H"], base["D"], base["topk"]
    lens = gen.uniform_int(7, gen.STREAM["lens"] * 1024 + 7, np.arange(24, dtype=np.uint64), 512, 16384)
    lens = [int(x) for x in lens]
    parts = [g.prefill_inputs(dict(base, L=n, heavy_count=max(1, n // 100), seed=100 + i)) for i, n in enumerate(lens)]
    cat = lambda key: torch.cat([p[key] for p in parts])
    q, qs, k, ks, w = cat("q"), cat("q_scale"), cat("k"), cat("k_scale"), cat("w")
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=g.device)
    out = torch.empty((q.shape[0], topk), dtype=torch.int32, device=g.device)
    ws = torch.empty(dsa.dsa_indexer_topk_prefill_varlen_workspace(len(lens), q.shape[0], H, D, topk, "fp8"),
                     dtype=torch.uint8, device=g.device)
    wss = torch.empty(dsa.dsa_indexer_topk_prefill_workspace(max(lens), H, D, topk, "fp8"), dtype=torch.uint8,
                      device=g.device)
    ragged = lambda: dsa.dsa_indexer_topk_prefill_varlen(q, qs, k, ks, w, cu, cu, topk, "fp8", out_idx=out,
                                                         workspace=ws, stream=stream)

    def per_sequence():
        for i, p in enumerate(parts):
            dsa.dsa_indexer_topk_prefill(p["q"], p["q_scale"], p["k"], p["k_scale"], p["w"], topk, "fp8",
                                         out_idx=out[int(cu[i]):int(cu[i]) + lens[i]], workspace=wss, stream=stream)
    t_r = sum(time_calls(ragged, args.steps, args.warmup, stream)) / args.steps
    t_s = sum(time_calls(per_sequence, args.steps, args.warmup, stream)) / args.steps
    flops = sum(prefill_flops(n, H, D) for n in lens)
    tf = flops / (t_r * 1e-3) / 1e12
    return {"metric": METRIC, "workload": "prefill_ragged", "value": round(tf, 2), "unit": "TFLOP/s",
            "ragged_ms": round(t_r, 4), "per_sequence_calls_ms": round(t_s, 4), "lengths": lens,
            "rows_per_s": round(sum(lens) / (t_r * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": None},
            "config": {"workload": "prefill_ragged", "sequences": len(lens), "total_rows": int(sum(lens)), "H": H,
                       "D": D, "topk": topk}}


def run_prefill_chunked(args, g, dsa, gen, stream):
    """The L=32768 prefill fed as four chunks of 8192 query rows in order
    (each chunk against all keys so far), as a serving engine feeds a long
    prompt; the same causal pairs as one whole-sequence call."""
    import torch
    cfg = gen.CONFIGS["prefill_32k"]
    L, H, D, topk = cfg["L"], cfg["H"], cfg["D"], cfg["topk"]
    C = 8192
    dev = g.device
    p = g.prefill_inputs(cfg)
    out = torch.empty((L, topk), dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.dsa_indexer_topk_prefill_workspace(C, H, D, topk, "fp8"), dtype=torch.uint8, device=dev)

    def chunks():
        for q0 in range(0, L, C):
            dsa.dsa_indexer_topk_prefill_chunk(p["q"][q0:q0 + C], p["q_scale"][q0:q0 + C], p["k"][:q0 + C],
                                               p["k_scale"][:q0 + C], p["w"][q0:q0 + C], q0, topk, "fp8",
                                               out_idx=out[q0:q0 + C], workspace=ws, stream=stream)
    ms = time_calls(chunks, args.steps, args.warmup, stream)
    avg = sum(ms) / len(ms)
    tf = prefill_flops(L, H, D) / (avg * 1e-3) / 1e12
    return {"metric": METRIC, "workload": "prefill_32k_chunked", "value": round(tf, 2), "unit": "TFLOP/s",
            "ms_per_sequence": round(avg, 4), "chunk_rows": C, "rows_per_s": round(L / (avg * 1e-3), 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_FP8_TFLOPS, 4), "traffic": None},
            "config": {"workload": "prefill_32k_chunked", "L": L, "H": H, "D": D, "topk": topk, "chunk": C}}


def run_fs(args, g, dsa, gen, stream):
    """Layer-reuse schedule over 47 layers: indexer time for each pattern and
    the 47x47 overlap of the all-F run."""
    import torch
    cfg = gen.CONFIGS["fs_47"]
    L, H, D, topk, N = cfg["L"], cfg["H"], cfg["D"], cfg["topk"], cfg["N"]
    dev = g.device
    log("generating 47 layers")
    layers = [g.fs_layer_inputs(cfg, l) for l in range(N)]
    ws = torch.empty(dsa.dsa_indexer_topk_prefill_workspace(L, H, D, topk, "fp8"), dtype=torch.uint8, device=dev)
    tcache = torch.empty((L, topk), dtype=torch.int32, device=dev)
    args_l = lambda key: [layers[l][key] for l in range(N)]
    res = {"metric": METRIC, "workload": "fs_47", "config": {"workload": "fs_47", "N": N, "L": L, "H": H, "D": D,
                                                              "topk": topk}}
    times = {}
    for pname, pat in gen.FS_PATTERNS.items():
        fn = lambda: dsa.indexcache_run_layers(pat, args_l("q"), args_l("q_scale"), args_l("k"), args_l("k_scale"),
                                               args_l("w"), topk, "fp8", tcache=tcache, workspace=ws, stream=stream)
        ms = time_calls(fn, max(1, args.steps), max(0, args.warmup), stream)
        times[pname] = sum(ms) / len(ms)
    nF = {p: pat.count("F") for p, pat in gen.FS_PATTERNS.items()}
    res["indexer_ms"] = {p: round(v, 3) for p, v in times.items()}
    res["indexer_time_saved_frac"] = {p: round(1 - times[p] / times["all_F"], 4) for p in times}
    res["ideal_saved_frac"] = {p: round(1 - nF[p] / N, 4) for p in times}
    tf = nF["all_F"] * prefill_flops(L, H, D) / (times["all_F"] * 1e-3) / 1e12
    res["value"] = round(tf, 2)
    res["unit"] = "TFLOP/s"
    # overlap of the all-F run: keep every layer's indices
    keep = [torch.empty((L, topk), dtype=torch.int32, device=dev) for _ in range(N)]
    hook = lambda layer, src, tc: keep[layer].copy_(tc)
    dsa.indexcache_run_layers(gen.FS_PATTERNS["all_F"], args_l("q"), args_l("q_scale"), args_l("k"),
                              args_l("k_scale"), args_l("w"), topk, "fp8", tcache=tcache, hook=hook, workspace=ws,
                              stream=stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    counts, ratio = dsa.topk_overlap_matrix(keep, topk)
    torch.cuda.synchronize()
    res["overlap_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
    res["overlap_adjacent_mean"] = round(float(sum(ratio[i, i + 1] for i in range(N - 1)) / (N - 1)), 4)
    res["overlap_matrix"] = [[round(float(x), 4) for x in row] for row in ratio]
    for pname, pat in gen.FS_PATTERNS.items():
        src = dsa.indexcache_resolve(pat)
        s_layers = [l for l in range(N) if pat[l] == "S"]
        if s_layers:
            res.setdefault("s_layer_mean_overlap_with_source", {})[pname] = round(
                float(sum(ratio[l, src[l]] for l in s_layers) / len(s_layers)), 4)
    # greedy search at retention 1/4 with the overlap proxy as its loss: a
    # labelled baseline (the pages' search uses a calibration LM loss, which
    # needs a trained model)
    proxy = lambda p: dsa.indexcache_overlap_proxy_loss(p, ratio)
    t0 = time.perf_counter()
    pat, trace, flipped = dsa.indexcache_greedy_search(N, N - 12, proxy)
    res["proxy_greedy_1_4"] = {"loss": "overlap proxy (baseline only)", "pattern": pat,
                               "proxy_loss": round(trace[-1], 5), "search_ms": round((time.perf_counter() - t0) * 1e3, 1),
                               "proxy_loss_of": {p: round(proxy(v), 5) for p, v in gen.FS_PATTERNS.items()}}
    return res


def run_fs_decode(args, g, dsa, gen, stream):
    """One decode step (32 sequences x 131072 cached tokens) through the
    layer-reuse schedule over 47 layers, each with its own key cache: indexer
    time per step for each pattern, and the cross-layer overlap of the all-F
    selections (rows = sequences)."""
    import torch
    cfg = gen.CONFIGS["fs_decode_47"]
    N, B, Lmax, H, D, topk = cfg["N"], cfg["B"], cfg["Lmax"], cfg["H"], cfg["D"], cfg["topk"]
    dev = g.device
    log("generating 47 decode layers")
    layers = [g.fs_decode_layer_inputs(cfg, l) for l in range(N)]
    lens = layers[0]["lens"]
    ws = torch.empty(dsa.dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk), dtype=torch.uint8, device=dev)
    tcache = torch.empty((B, topk), dtype=torch.int32, device=dev)
    pick = lambda key: [layers[l][key] for l in range(N)]
    times = {}
    for pname, pat in gen.FS_PATTERNS.items():
        fn = lambda: dsa.indexcache_run_decode_layers(pat, pick("q"), pick("w"), pick("cache"), pick("k_scale"),
                                                      lens, topk, tcache=tcache, workspace=ws, stream=stream)
        ms = time_calls(fn, max(1, args.steps), max(0, args.warmup), stream)
        times[pname] = sum(ms) / len(ms)
    nF = {p: pat.count("F") for p, pat in gen.FS_PATTERNS.items()}
    per_layer = decode_bytes(gen.decode_lens(cfg), H, D, topk, B)
    gbps = nF["all_F"] * per_layer / (times["all_F"] * 1e-3) / 1e9
    res = {"metric": METRIC, "workload": "fs_decode_47", "value": round(gbps, 1), "unit": "GB/s",
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                        "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None},
           "config": {"workload": "fs_decode_47", "N": N, "B": B, "Lmax": Lmax, "H": H, "D": D, "topk": topk},
           "step_us": {p: round(v * 1e3, 1) for p, v in times.items()},
           "per_F_layer_us": round(times["all_F"] * 1e3 / N, 2),
           "indexer_time_saved_frac": {p: round(1 - times[p] / times["all_F"], 4) for p in times},
           "ideal_saved_frac": {p: round(1 - nF[p] / N, 4) for p in times}}
    keep = [torch.empty((B, topk), dtype=torch.int32, device=dev) for _ in range(N)]
    hook = lambda layer, src, tc: keep[layer].copy_(tc)
    dsa.indexcache_run_decode_layers(gen.FS_PATTERNS["all_F"], pick("q"), pick("w"), pick("cache"),
                                     pick("k_scale"), lens, topk, tcache=tcache, hook=hook, workspace=ws,
                                     stream=stream)
    torch.cuda.synchronize()
    _, ratio = dsa.topk_overlap_matrix(keep, topk, row_begin=0, row_end=B)
    res["overlap_adjacent_mean"] = round(float(sum(ratio[i, i + 1] for i in range(N - 1)) / (N - 1)), 4)
    for pname, pat in gen.FS_PATTERNS.items():
        src = dsa.indexcache_resolve(pat)
        s_layers = [l for l in range(N) if pat[l] == "S"]
        if s_layers:
            res.setdefault("s_layer_mean_overlap_with_source", {})[pname] = round(
                float(sum(ratio[l, src[l]] for l in s_layers) / len(s_layers)), 4)
    return res


def run_mli_decode(args, g, dsa, gen, stream):
    """One decode step (32 sequences x 131072 cached tokens, 47 layers) with a
    stand-in sparse attention per layer (one head over the k selected rows of
    a 576-value bf16 latent cache; four latent caches, 19.3 GB, cycled over
    the layers): per pattern, the indexers alone, IndexCache with each
    layer's attention after its indexer on one stream, and the lagged
    (multi-layer indexer) schedule with the indexers on a second stream."""
    import math
    import torch
    cfg = gen.CONFIGS["fs_decode_47"]
    N, B, Lmax, H, D, topk, seed = cfg["N"], cfg["B"], cfg["Lmax"], cfg["H"], cfg["D"], cfg["topk"], cfg["seed"]
    dev = g.device
    log("generating 47 decode layers, 4 latent caches")
    layers = [g.fs_decode_layer_inputs(cfg, l) for l in range(N)]
    lens = layers[0]["lens"]
    NLAT = 4
    lat = [g.standin_latent(seed, i, B, Lmax) for i in range(NLAT)]
    qa = [g.standin_query(seed, l, B) for l in range(N)]
    scale = 1.0 / math.sqrt(576.0)
    ws = torch.empty(dsa.dsa_indexer_topk_decode_workspace(B, Lmax, H, D, topk), dtype=torch.uint8, device=dev)
    aws = torch.empty(dsa.standin_sparse_attention_workspace(B, topk), dtype=torch.uint8, device=dev)
    aout = torch.empty((B, 512), dtype=torch.float32, device=dev)
    tcache = torch.empty((B, topk), dtype=torch.int32, device=dev)
    sel_buf = torch.empty((N, B, topk), dtype=torch.int32, device=dev)
    side = torch.cuda.Stream(device=dev)
    pick = lambda key: [layers[l][key] for l in range(N)]

    def attention(layer, sel):
        dsa.standin_sparse_attention(qa[layer], lat[layer % NLAT], sel, scale, out=aout, workspace=aws, stream=stream)

    def indexers(pat):
        dsa.indexcache_run_decode_layers(pat, pick("q"), pick("w"), pick("cache"), pick("k_scale"), lens, topk,
                                         tcache=tcache, workspace=ws, stream=stream)

    def serial(pat):
        dsa.indexcache_run_decode_layers(pat, pick("q"), pick("w"), pick("cache"), pick("k_scale"), lens, topk,
                                         tcache=tcache, hook=lambda l, s, tc: attention(l, tc), workspace=ws,
                                         stream=stream)

    def lagged(pat):
        dsa.indexcache_run_decode_layers_mli(pat, pick("q"), pick("w"), pick("cache"), pick("k_scale"), lens, topk,
                                             sel_buf=sel_buf, attn=lambda l, s, sel: attention(l, sel),
                                             workspace=ws, stream=stream, side_stream=side)

    def attention_only():
        for l in range(N):
            attention(l, tcache)

    steps, warm = max(1, args.steps), max(0, args.warmup)
    avg = lambda ms: sum(ms) / len(ms) * 1e3
    indexers(gen.FS_PATTERNS["all_F"])           # a real selection in tcache for attention_only
    att_us = avg(time_calls(attention_only, steps, warm, stream))
    res = {"metric": METRIC, "workload": "mli_decode_47",
           "config": {"workload": "mli_decode_47", "N": N, "B": B, "Lmax": Lmax, "H": H, "D": D, "topk": topk,
                      "attention": "stand-in, 1 head, 576-value bf16 latent rows"},
           "attention_us_per_layer": round(att_us / N, 2), "step_us": {}, "lagged_speedup": {}}
    for pname, pat in gen.FS_PATTERNS.items():
        t_idx = avg(time_calls(lambda: indexers(pat), steps, warm, stream))
        t_ser = avg(time_calls(lambda: serial(pat), steps, warm, stream))
        t_mli = avg(time_calls(lambda: lagged(pat), steps, warm, stream))
        res["step_us"][pname] = {"indexers_only": round(t_idx, 1), "indexcache_serial": round(t_ser, 1),
                                 "lagged_two_streams": round(t_mli, 1)}
        res["lagged_speedup"][pname] = round(t_ser / t_mli, 4)
    per_layer = decode_bytes(gen.decode_lens(cfg), H, D, topk, B)
    t_all = res["step_us"]["all_F"]["lagged_two_streams"] * 1e-6
    gbps = N * per_layer / t_all / 1e9
    res.update({"value": round(gbps, 1), "unit": "GB/s",
                "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                             "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None}})
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="main")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--reference-copy-mb", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (a plain copy of known "
                         "size, used to calibrate memory-traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"this benchmark runs on one GPU only (asked for --gpus {args.gpus}); the indexer path is measured "
              "per GPU and is not sharded across GPUs", file=sys.stderr)
        sys.exit(2)
    args.cpu_result = None
    if not args.no_cpu_baseline:
        if args.workload == "main":
            log("cpu baseline (the oracle on the host cores, before the GPU is used)")
            args.cpu_result = cpu_baseline(budget_s=args.cpu_budget)
        elif args.workload in ("prefill_196k", "fs_47"):
            log("cpu baseline of the workload (the oracle on the host cores, before the GPU is used)")
            args.cpu_result = cpu_baseline_workload(args.workload, budget_s=args.cpu_budget)
    res = run_main(args) if args.workload == "main" else run_workload(args)
    if args.workload != "main" and args.cpu_result is not None:
        res["cpu_baseline"] = args.cpu_result
    if args.reference_copy_mb > 0:
        import torch
        n = args.reference_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["reference_copy_bytes"] = n
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
