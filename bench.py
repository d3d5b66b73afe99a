#!/usr/bin/env python3
"""Benchmark of the bit-plane top-k decode path on one MI355X.

A step is one decode step over every (sequence, layer, KV head) unit of the
workload: depth allocation -> prefix-plane key scan (with the fused candidate
selection: sampled threshold, candidate scan, exact top-k among the
candidates) -> union-gather attention, on a cache resident in HBM (rows,
planes, scales).  Default workload: 36 layers x 8 KV heads x 1 sequence of
n = 1,048,576 tokens, G = 4 query heads per KV head, plane budget P = 88 (the
"92-bit" point), k = 512; KV heads 4-7 have Pareto channel variances.

The headline value is the bandwidth of the decode step's key scan: the
algorithmic bytes of one scan (the selected planes, P*n/8 bytes per unit, plus
the fp16 scales of the channels read, 2*C_read*n/64 bytes per unit) over the
scan kernel's average duration, measured with the library's stage tracing
(HIP events recorded on the stream the kernels run on, around the scan
launch).  Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def scan_bytes(depth_np, n: int) -> float:
    """Algorithmic bytes of one scan over the units whose depths are given."""
    t = depth_np.reshape(-1, depth_np.shape[-1]).astype("int64")
    nb = n // 64
    return float(t.sum()) * nb * 8.0 + float((t > 0).sum()) * nb * 2.0


SAMPLE_STRIDE, SAMPLE_GROUP = 4096, 64  # the sampled scan: the first 64 blocks of every 4096


def sampled_blocks(n: int) -> int:
    """Blocks of one unit of n tokens that the decode step's sampled scan reads."""
    nb = n // 64
    return sum(min(SAMPLE_GROUP, nb - g) for g in range(0, nb, SAMPLE_STRIDE))


TRAFFIC_SOURCES = ("bit_plane_key_amd/csrc/scan.hip", "bit_plane_key_amd/csrc/scan_common.h",
                   "bit_plane_key_amd/csrc/bpk_internal.h")


def profile_field(name: str, key: str):
    """A value from a committed counter summary under profiles/, or None when
    there is none or the scan's source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", " ", "*")):
            k, _, val = line.partition(":")
            fields[k.strip()] = val.strip()
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest():
        log(f"profiles/{name} was taken on other scan sources than these: {key} not reported")
        return None
    return fields.get(key)


def counted_traffic(config: str, budget: int):
    """HBM bytes per scan launch (FETCH_SIZE + WRITE_SIZE, scaled)."""
    v = profile_field(f"scan_cand_kernel_{config}_P{budget}_hbm_bytes.md", "traffic_bytes_per_launch")
    return None if v is None else int(v)


def counted_valu(config: str, budget: int):
    """(VALU busy %, VALU instructions per 64-token block) of the scan launch."""
    name = f"scan_cand_kernel_{config}_P{budget}_sq_counters.md"
    busy = profile_field(name, "valu_busy_percent")
    per = profile_field(name, "valu_insts_per_block")
    return (None if busy is None else float(busy)), (None if per is None else float(per))


def time_launches(fn, steps: int, before=None):
    """Median milliseconds of `steps` calls of fn, each between two HIP events
    recorded on the current stream (the stream the library's calls run on);
    `before`, if given, runs ahead of each call, outside the timed region."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        if before is not None:
            before()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(statistics.median(a.elapsed_time(b) for a, b in ev))


def _oracle_unit_step(job):
    """One unit of the oracle's decode step (allocation, scan, selection,
    attention) on a host sample; returns (seconds, scan bytes).  Runs in a
    worker process with one BLAS thread; the unit's rows come from the host
    generator (the same bits the device generator wrote)."""
    cfg_name, s, l, h, tokens, budget, topk, scale = job
    import numpy as np

    import oracle as O
    from synth import config_by_name
    from synth import workload as W
    cfg = config_by_name(cfg_name)
    rows = np.arange(tokens)
    _, k = W.key_rows(cfg, s, l, h, rows)
    _, v = W.value_rows(cfg, s, l, h, rows)
    _, q = W.query(cfg, s, l, h)
    var = cfg.chan_var(s, l, h)
    planes, scales = O.encode_unit(k)
    t0 = time.perf_counter()
    depth = O.alloc_depth(q, var, budget)
    sc, _ = O.scan_scores(q, depth, planes, scales, tokens)
    idx = O.select_topk(sc, tokens, topk)
    O.attend(q, k, v, idx, scale)
    return time.perf_counter() - t0, O.scan_bytes_unit(depth, tokens)


def cpu_baseline(cfg, budget: int, tokens: int, units, n: int, step_units: int, k: int,
                 scale: float):
    """The oracle's decode step (depth allocation, scan, top-k, attention;
    the encoding of the sample is not timed) on the host cores, over a
    bounded sample of the workload: the first ``tokens`` tokens of each of
    ``units``, one unit at a time per worker process.  Reported in the
    metric's unit: scan bytes over seconds, on all the cores used."""
    import concurrent.futures as cf
    import multiprocessing as mp
    jobs = [(cfg.name, s, l, h, tokens, budget, k, scale) for (s, l, h) in units]
    # at most 16 worker processes: the host share of one GPU, whatever the
    # machine reports
    cores = min(len(jobs), os.cpu_count() or 1, 16)
    env = {"OMP_NUM_THREADS": "1", "OPENBLAS_NUM_THREADS": "1", "MKL_NUM_THREADS": "1"}
    old = {x: os.environ.get(x) for x in env}
    os.environ.update(env)
    try:
        t0 = time.perf_counter()
        with cf.ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn")) as ex:
            res = list(ex.map(_oracle_unit_step, jobs))
        wall = time.perf_counter() - t0
    finally:
        for x, val in old.items():
            if val is None:
                os.environ.pop(x, None)
            else:
                os.environ[x] = val
    secs = sum(r[0] for r in res)
    total_bytes = sum(r[1] for r in res)
    per_unit_s = secs / len(res)
    # the cores work on units side by side: throughput = cores x one core's rate
    return {"value": round(total_bytes / secs * cores / 1e9, 4), "unit": "GB/s",
            "cores": cores, "kind": "oracle",
            "keys_per_s": round(tokens * cores / per_unit_s, 1),
            "per_unit_ms": round(per_unit_s * 1e3, 2),
            "cpu_s": round(secs, 1),
            # the sample's per-unit time scaled to every unit of the step, all n
            # tokens and the cores used: an extrapolation, not a measurement
            "step_s_extrapolated": round(per_unit_s * (n / tokens) * step_units / cores, 2),
            "sample": (f"oracle decode step (depth allocation, scan, top-k, attention; not the "
                       f"encoding) of {len(units)} units (sequence 0, layers "
                       f"{sorted({u[1] for u in units})}, all KV heads) of the same workload, "
                       f"first {tokens} tokens each, P={budget}, k={k}, one unit at a time per "
                       f"process on {cores} host cores; {secs:.1f} s of CPU work, "
                       f"{wall:.1f} s wall")}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)  # clocks ramp over the first steps
    ap.add_argument("--config", default="c4")
    ap.add_argument("--budget", type=int, default=88)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the sweep over the workload's plane budgets (profiling runs)")
    ap.add_argument("--cpu-tokens", type=int, default=1 << 18)
    ap.add_argument("--cpu-layers", type=int, default=5)
    ap.add_argument("--host-resident", action="store_true",
                    help="rows, planes and scales in pinned host memory, read over the host "
                         "link (the regime of the Fathom page's measurements)")
    ap.add_argument("--layers", type=int, default=0,
                    help="use only the workload's first LAYERS layers (0: all)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard over sequences and (layer, KV head) units with no "
              "exchange between GPUs)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import bit_plane_key_amd as bpk
    from bit_plane_key_amd import workloads
    from synth import config_by_name

    cfg = config_by_name(args.config)
    if args.layers:
        import dataclasses
        cfg = dataclasses.replace(cfg, layers=min(args.layers, cfg.layers))
    budget, k, n = args.budget, cfg.k, cfg.n
    torch.cuda.set_device(0)
    t0 = time.perf_counter()
    log(f"building {cfg.name}: {cfg.description}")
    cache = workloads.build_cache(cfg, host_resident=args.host_resident,
                                  values=not args.no_sweep)
    log(f"cache built in {time.perf_counter() - t0:.1f} s")
    q = workloads.queries(cfg)
    scale = workloads.softmax_scale(cfg)
    L = cfg.layers
    ws = torch.empty(bpk.workspace_bytes(cache, bpk.BPK_OP_DECODE, 0, L, k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((cfg.seqs, L, cfg.heads, cfg.group, 128), dtype=torch.float32,
                      device="cuda")

    appends = cfg.append_steps > 0
    if appends:
        # the workload appends one token per sequence before each decode step:
        # the rows of those tokens are written once here, outside any timing
        workloads.fill_tokens(cfg, cache, n, cfg.append_steps)
        if args.warmup + 2 * args.steps > cfg.append_steps:
            log(f"{cfg.name} holds {cfg.append_steps} appended tokens: use warmup + 2 * steps <= that")
            return 2

    def step(p=budget):
        if appends:
            for s in range(cfg.seqs):
                bpk.encode_append(cache, s, None, None, 1)
        bpk.decode_step(cache, q, 0, L, p, k, scale, out=out, ws=ws)

    def traced(steps, fn):
        """Median milliseconds of each decode-step stage over `steps` calls of
        fn (stage tracing: HIP events the library records around each stage
        on the step's stream, read back after every call)."""
        per = {name: [] for name in bpk.STAGES}
        bpk.trace_enable(True)
        try:
            for _ in range(steps):
                fn()
                ms, calls = bpk.trace_read(reset=True)
                for name, v in ms.items():
                    per[name].append(v / max(calls, 1))
        finally:
            bpk.trace_enable(False)
        return {name: float(statistics.median(v)) if v else 0.0 for name, v in per.items()}

    def bits_of(d_np):
        return float(np.mean([float(t.sum()) + 0.25 * float((t > 0).sum())
                              for t in d_np.reshape(-1, 128)]))

    def kernel_label(d_np):
        rows = int(d_np.reshape(-1, 128).sum(axis=1).max())
        if rows <= 96:
            return f"scan_fast_kernel<{cfg.group}, 2, 96>"
        if rows <= 128:
            return f"scan_fast_kernel<{cfg.group}, 2, 128>"
        return f"scan_wide_kernel<{cfg.group}, 2>"

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    ms_step = time_launches(step, args.steps)
    log(f"decode step (median): {ms_step * 1e3:.1f} us")
    stage_ms = traced(args.steps, step)
    ms_scan = stage_ms["scan"]
    log("stages, median us: " + " ".join(f"{nm} {v * 1e3:.1f}" for nm, v in stage_ms.items()))
    flagged = bpk.decode_fallback_units(cache, 0, L, k, ws)
    log(f"units redone unfused in the last step: {flagged} of {cfg.units}")

    # the same step with the caches evicted first: a 1 GiB write before each
    # call, outside the timed region (c1 and c2 fit in the L2 and the
    # Infinity Cache, so their warm figures are latencies, not HBM rates)
    evicted = None
    if not appends:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

        def flushed():
            flush.fill_(1.0)

        ms_ev = time_launches(step, args.steps, before=flushed)
        st_ev = traced(args.steps, lambda: (flushed(), step()))
        del flush
        evicted = {"decode_step_us": round(ms_ev * 1e3, 1),
                   "stage_us": {nm: round(v * 1e3, 1) for nm, v in st_ev.items()}}
        log(f"caches evicted before each step: {evicted}")

    # attention: the union of the heads' selections, fetched once per unit
    idx = torch.empty((cfg.seqs, L, cfg.heads, cfg.group, k), dtype=torch.int32, device="cuda")
    bpk.decode_step(cache, q, 0, L, budget, k, scale, out=out, idx_out=idx, ws=ws)
    srt = idx.reshape(-1, cfg.group * k).sort(dim=1).values
    uniq = (srt[:, 1:] != srt[:, :-1]).sum(dim=1) + 1
    union_rows = int(uniq.sum().item())
    row_bytes = 128 * (4 if cfg.k_dtype == "f32" else 2) + 128 * 2
    attend_bytes = union_rows * row_bytes
    log(f"union rows {union_rows} ({union_rows / cfg.units:.0f} per unit), "
        f"attention {attend_bytes / (stage_ms['attend'] * 1e-3) / 1e9:.0f} GB/s")

    # the workload's other plane budgets: does the step scale with the bits read?
    sweep = {}
    if not appends and not args.no_sweep:
        for p in cfg.budgets:
            d_p, _ = bpk.alloc_depth(cache, q, 0, L, p)
            d_np = d_p.cpu().numpy()
            for _ in range(2):
                step(p)
            ms_p = time_launches(lambda: step(p), args.steps)
            st_p = traced(args.steps, lambda: step(p))
            sweep[str(p)] = {"bits_per_token": round(bits_of(d_np), 2),
                             "decode_step_us": round(ms_p * 1e3, 1),
                             "scan_us": round(st_p["scan"] * 1e3, 1),
                             "scan_gbs": round(scan_bytes(d_np, n) / (st_p["scan"] * 1e-3) / 1e9, 2)}
            log(f"P={p}: {sweep[str(p)]}")

    # the fixed-depth scans the Fathom page compares against (§2), on the
    # same planes and through the same scan, selection and attention:
    # SparQ r = 16 and 32, Double Sparsity's static c = 32 channels, the
    # 2-bit thumbnail.  Double Sparsity's offline channel sets come from the
    # workload's own statistics (mean|q| equal on every channel, mean|k_j|
    # proportional to sigma_j).
    baselines = {}
    if not appends and not args.no_sweep:
        ds = np.zeros((L, cfg.heads, 32), dtype=np.uint8)
        for l in range(L):
            for h in range(cfg.heads):
                ds[l, h] = np.sort(np.lexsort((np.arange(128), -cfg.chan_var(0, l, h)))[:32])
        ds_t = torch.from_numpy(ds).cuda()
        rules = {"sparq_r16": (bpk.BPK_DEPTH_SPARQ, 16, None),
                 "sparq_r32": (bpk.BPK_DEPTH_SPARQ, 32, None),
                 "double_sparsity_c32": (bpk.BPK_DEPTH_CHANNELS, 32, ds_t),
                 "thumbnail_2bit": (bpk.BPK_DEPTH_UNIFORM, 2, None)}
        dq = torch.empty((cfg.seqs, L, cfg.heads, 128), dtype=torch.uint8, device="cuda")
        qbq = torch.empty((cfg.seqs, L, cfg.heads, cfg.group, 128), dtype=torch.float32,
                          device="cuda")
        for name, (rule, param, ch) in rules.items():
            # each rule's bound on the rows a unit reads: 4 r, 4 c, 128 t
            bound = 128 * param if rule == bpk.BPK_DEPTH_UNIFORM else 4 * param

            def bstep(rule=rule, param=param, ch=ch, bound=bound):
                bpk.fixed_depth(cache, q, 0, L, rule, param, channels=ch, depth=dq, q_basis=qbq)
                bpk.decode_step_depth(cache, q, qbq, dq, 0, L, k, scale, out=out, ws=ws,
                                      max_rows=bound)
            for _ in range(2):
                bstep()
            ms_b = time_launches(bstep, args.steps)
            st_b = traced(args.steps, bstep)
            d_np = dq.cpu().numpy()
            baselines[name] = {"bits_per_token": round(bits_of(d_np), 2),
                               "decode_step_us": round(ms_b * 1e3, 1),
                               "scan_us": round(st_b["scan"] * 1e3, 1),
                               "scan_gbs": round(scan_bytes(d_np, n) / (st_b["scan"] * 1e-3) / 1e9, 2),
                               "units_redone": bpk.decode_fallback_units(cache, 0, L, k, ws)}
            log(f"{name}: {baselines[name]}")

    # per-layer budget calibration (Fathom §3's optional add-on; the rule is a
    # reading): four calibration queries (decode steps 1-4) water-filled over
    # every unit of every layer, per-layer budgets keeping the total 36 * P;
    # the step then runs one decode call per layer at its budget.  Reported:
    # the budgets, the step time (per-layer calls, against the same per-layer
    # loop at the uniform budget) and the predicted squared-error proxy
    # sum_u sum_j g_uj 4^-t_uj of the held-out query (step 0) under both.
    calibration = None
    if not appends and not args.no_sweep and cfg.seqs == 1:
        from synth import workload as W
        cq = torch.stack([workloads.queries(cfg, step=s) for s in range(1, 5)])
        counts = torch.stack([bpk.pooled_planes(cache, cq[i], 0, L, budget) for i in range(4)])
        lb = bpk.layer_budgets(cache, counts, 0, L, budget).cpu().numpy()
        q_l = [q[:, l:l + 1].contiguous() for l in range(L)]
        out_l = [out[:, l:l + 1].contiguous() for l in range(L)]

        def layer_loop(budgets):
            for l in range(L):
                bpk.decode_step(cache, q_l[l], l, l + 1, int(budgets[l]), k, scale, out=out_l[l],
                                ws=ws)
        uni = np.full(L, budget)
        lb_t = torch.from_numpy(lb.astype(np.int32)).cuda()
        dl = torch.empty((cfg.seqs, L, cfg.heads, 128), dtype=torch.uint8, device="cuda")
        ql = torch.empty((cfg.seqs, L, cfg.heads, cfg.group, 128), dtype=torch.float32,
                         device="cuda")

        def one_call():  # every layer at its budget in one call
            bpk.alloc_depth_layers(cache, q, 0, L, lb_t, depth=dl, q_basis=ql)
            bpk.decode_step_depth(cache, q, ql, dl, 0, L, k, scale, out=out, ws=ws,
                                  max_rows=int(lb.max()))  # a layer's units read its budget
        for _ in range(2):
            layer_loop(lb)
            layer_loop(uni)
            one_call()
        ms_cal = time_launches(lambda: layer_loop(lb), args.steps)
        ms_uni = time_launches(lambda: layer_loop(uni), args.steps)
        ms_one = time_launches(one_call, args.steps)

        def proxy(budgets):
            tot = 0.0
            for l in range(L):
                d, _ = bpk.alloc_depth(cache, q_l[l], l, l + 1, int(budgets[l]))
                d = d.cpu().numpy().reshape(cfg.heads, 128).astype(np.float64)
                for h in range(cfg.heads):
                    qh = W.query(cfg, 0, l, h, 0)[1].astype(np.float64)
                    g = cfg.chan_var(0, l, h).astype(np.float64) * (qh * qh).sum(axis=0)
                    tot += float((g * 0.25 ** d[h]).sum())
            return tot
        calibration = {"layer_budgets": [int(x) for x in lb],
                       "decode_step_us": round(ms_one * 1e3, 1),
                       "per_layer_calls_step_us": round(ms_cal * 1e3, 1),
                       "uniform_per_layer_calls_step_us": round(ms_uni * 1e3, 1),
                       "error_proxy_ratio": round(proxy(lb) / proxy(uni), 4)}
        log(f"calibrated budgets {min(lb)}..{max(lb)}: {calibration}")

    # value-side depths (ReadKV §5.3, §5.4): the same step with every union
    # row's value read at a per-token depth from its planes, for budgets of
    # v planes per unit; against the exact-value step: the attention stage's
    # time, the value bytes read (16 per plane plus the 2-byte scale of each
    # row read at all, against 256 per bf16 row) and the output's deviation
    # (max |difference| / max |exact output| per query head)
    value_depths = {}
    if cache.v_planes is not None and not appends:
        bpk.decode_step(cache, q, 0, L, budget, k, scale, out=out, ws=ws)
        ref_out = out.clone()
        wsv = torch.empty(bpk.workspace_bytes(cache, bpk.BPK_OP_DECODE_V, 0, L, k),
                          dtype=torch.uint8, device="cuda")
        outv = torch.empty_like(out)
        vdep = torch.empty((cfg.seqs, L, cfg.heads, cfg.group * k), dtype=torch.uint8,
                           device="cuda")
        for vb in (k // 2, k, 2 * k, 4 * k, 4 * cfg.group * k):
            def vstep(vb=vb):
                bpk.decode_step_v(cache, q, 0, L, budget, k, scale, vb, out=outv,
                                  v_depth_out=vdep, ws=wsv)
            for _ in range(2):
                vstep()
            ms_v = time_launches(vstep, args.steps)
            st_v = traced(args.steps, vstep)
            dv = vdep.to(torch.int64)
            vbytes = int((16 * dv.sum() + 2 * (dv > 0).sum()).item())
            dev = ((outv - ref_out).abs().amax(dim=-1)
                   / ref_out.abs().amax(dim=-1).clamp_min(1e-30)).flatten()
            value_depths[str(vb)] = {
                "mean_depth": round(float(dv.sum().item()) / union_rows, 3),
                "decode_step_us": round(ms_v * 1e3, 1),
                "attend_us": round(st_v["attend"] * 1e3, 1),
                "value_bytes": vbytes,
                "value_bytes_bf16_rows": union_rows * 256,
                "out_deviation_median": round(float(dev.median().item()), 5),
                "out_deviation_max": round(float(dev.max().item()), 5)}
            log(f"value budget {vb}: {value_depths[str(vb)]}")
        del wsv, outv, vdep, ref_out

    # the standalone full scan (scan_scores writes every score: same reads,
    # plus 16 bytes of scores per token)
    del ws
    depth, qb = bpk.alloc_depth(cache, q, 0, L, budget)
    scores = torch.empty((cfg.seqs, L, cfg.heads, cfg.group, cfg.capacity), dtype=torch.float32,
                         device="cuda")
    bpk.scan_scores(cache, qb, depth, 0, L, scores=scores)
    torch.cuda.synchronize()
    ms_full = time_launches(lambda: bpk.scan_scores(cache, qb, depth, 0, L, scores=scores),
                            args.steps)
    del scores
    log(f"standalone full scan: {ms_full * 1e3:.1f} us")

    # streaming ceilings on this GPU: a plain copy of 2 GiB (read + write;
    # also the known-size kernel the HBM byte counters are scaled by) and a
    # plain streaming read of 4 GiB (16-byte loads, four in flight a thread)
    cx = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    cy = torch.empty_like(cx)
    torch.mul(cx, 1.0, out=cy)  # the first launch loads the kernel's code object
    ms_copy = time_launches(lambda: torch.mul(cx, 1.0, out=cy), args.steps)
    copy_gbs = 2 * cx.numel() * 4 / (ms_copy * 1e-3) / 1e9
    del cx, cy
    from synth import device as synth_device
    rx = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    acc = torch.empty(4096, dtype=torch.int32, device="cuda")
    synth_device.stream_read(rx, acc)
    ms_read = time_launches(lambda: synth_device.stream_read(rx, acc), args.steps)
    read_gbs = rx.numel() * 4 / (ms_read * 1e-3) / 1e9
    del rx, acc
    log(f"plain copy of 2 GiB: {copy_gbs:.0f} GB/s; streaming read of 4 GiB: {read_gbs:.0f} GB/s")
    link_gbs = None
    if args.host_resident:
        # the host link's read ceiling: the same probe over 1 GiB of pinned host memory
        from bit_plane_key_amd._lib import _device_pointer
        hx = torch.ones(1 << 28, dtype=torch.float32, pin_memory=True)
        acc = torch.empty(4096, dtype=torch.int32, device="cuda")
        synth_device.stream_read(hx, acc, ptr=_device_pointer(hx))
        ms_link = time_launches(lambda: synth_device.stream_read(hx, acc, ptr=_device_pointer(hx)),
                                max(3, args.steps // 4))
        link_gbs = hx.numel() * 4 / (ms_link * 1e-3) / 1e9
        del hx, acc
        log(f"streaming read of 1 GiB of pinned host memory: {link_gbs:.1f} GB/s")

    d = depth.cpu().numpy()
    sbytes = scan_bytes(d, n)
    scan_gbs = sbytes / (ms_scan * 1e-3) / 1e9
    units = cfg.units
    keys_per_s = units * n / (ms_scan * 1e-3)

    result = {
        "metric": "K-scan GB/s (% of HBM peak) + decode-step us at n=1M tokens, 92-bit budget",
        "value": round(scan_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # int8 digits of 29-bit fixed-point weights times 0/1 plane bits,
        # accumulated exactly in int32 on the matrix cores
        "dtype": "i8xbit->i32 (29-bit fixed point)",
        "data": "synthetic",
        "config": {
            "workload": (f"{cfg.name}: {cfg.seqs} seq x {cfg.layers} layers x {cfg.heads} KV "
                         f"heads, G={cfg.group}, D=128, n={n}, P={budget}, k={k}"
                         + (", rows/planes/scales in pinned host memory" if args.host_resident
                            else "")),
            "units": units, "n": n, "budget_planes": budget, "k": k,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(scan_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
            "traffic": counted_traffic(cfg.name, budget),
            "valu_busy_percent": counted_valu(cfg.name, budget)[0],
            "valu_insts_per_block": counted_valu(cfg.name, budget)[1],
            "kernel": kernel_label(d) + " (the decode step's candidate scan)",
            "bytes_per_launch": sbytes,
            "avg_launch_us": round(ms_scan * 1e3, 2),
            "timing": "median of HIP-event stage times",
        },
        "decode_step_us": round(ms_step * 1e3, 1),
        "stage_us": {name: round(v * 1e3, 1) for name, v in stage_ms.items()},
        "evicted": None if evicted is None else dict(
            evicted, scan_gbs=round(sbytes / (evicted["stage_us"]["scan"] * 1e-6) / 1e9, 2)),
        "units_redone_unfused": flagged,
        "attend": {"union_rows": union_rows, "bytes": attend_bytes,
                   "gbs": round(attend_bytes / (stage_ms["attend"] * 1e-3) / 1e9, 1)},
        # algorithmic bytes over stage time: the sampled scan reads the same
        # rows as the scan over the sampled blocks only
        "stage_gbs": {
            "sample": round(sbytes * sampled_blocks(n) / max(n // 64, 1)
                            / (stage_ms["sample"] * 1e-3) / 1e9, 1),
            "scan": round(scan_gbs, 1),
            "attend": round(attend_bytes / (stage_ms["attend"] * 1e-3) / 1e9, 1)},
        "full_scan_us": round(ms_full * 1e3, 1),
        "full_scan_gbs": round(sbytes / (ms_full * 1e-3) / 1e9, 2),
        "keys_per_s": round(keys_per_s, 0),
        "copy_gbs": round(copy_gbs, 1),
        "read_ceiling_gbs": round(read_gbs, 1),
        "host_link_read_gbs": None if link_gbs is None else round(link_gbs, 1),
        "scan_bits_per_token_mean": round(bits_of(d), 2),
        "budget_sweep": sweep,
        "baselines": baselines,
        "layer_calibration": calibration,
        "value_depths": value_depths,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a CPU sample")
        sample_units = [(0, l, h) for l in range(min(args.cpu_layers, L)) for h in range(cfg.heads)]
        result["cpu_baseline"] = cpu_baseline(cfg, budget, min(args.cpu_tokens, n),
                                              sample_units, n, cfg.units, k, scale)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
