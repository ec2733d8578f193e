"""Benchmark of one DDTree verify step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM.  The default workload is the largest single-GPU
configuration, long context with all heads: 4 requests, 64 heads,
kv_lora_rank 512 + rope 64 (bf16), prefix 131072 each, 128 tree nodes (a
wide-shallow best-first tree from seeded top-8 draft candidates, depth <= 4),
and its step is
    parents -> ancestor mask -> tree-verify MLA attention (absorbed, bf16 in,
    fp32 accumulate; split-KV kernel + merge) -> greedy acceptance + KV
    compaction + length update (one launch) on the planted target ids.
`--config 2` runs the K2-like head share (1 request, 8 heads, prefix 4096,
64 nodes), whose step also takes the argmax over 64 x 163840 fp32 target
logits (fused: two launches); `--config 3` the batched ragged workload;
`--config 5` the verify loop (100 steps with cache growth).

Prints ONE JSON line.  `value` is verify-attention TFLOP/s over the whole
step (attention FLOPs / step time); `ms_per_step` and `verify_attn_ms` are
medians of 5 timed windows of at least 50 ms each (HIP events on the launch
stream around graph replays), reported with their spread; `roofline` is
the attention launch against the bf16 MFMA peak; `hbm_stages` the HBM scans
of the end-to-end step (argmax over 2048 x 163840 fp32 target logits, draft
top-8 over 256 x 163840) against 8 TB/s; `cpu_baseline` times the fp64
oracle on the host for a sample of the same workload.  The default run
also reports the K2-like head share's step, the batched ragged step and a
short verify loop (with its last step replayed at a steady clock) as extra
keys (`config2`, `config3`, `config5_loop`).

`--traffic-probe` runs a few attention launches of the workload and one
device-to-device copy of known size, and exits: it is the program that the
HBM-traffic counter runs (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE) profile.
The per-launch traffic they measured is read back from
profiles/verify_attn_<workload>_traffic.md, and reported only while the
kernel source still has the hash recorded there.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
FLOP_PER_PAIR = 2 * (512 + 64) + 2 * 512   # QK over 576 + PV over 512
WINDOWS = 5                     # timed windows per figure (median and spread reported)
WINDOW_MS = 50.0                # at least this much device time per window


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4,
                    help="workload configuration (2, 3, 4 = the default, or 5: the verify loop)")
    ap.add_argument("--loop-steps", type=int, default=100, help="timed iterations of the verify loop (config 5)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="config 5: keep the loop's cache in pages of this many rows (0: contiguous)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the on-device MFMA / HBM peak probes")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the side measurements (paged, prefill, projections, HBM stages, configs 2 and 3, loop)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache attention timing (configs 2 and 3)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget for the oracle timing")
    ap.add_argument("--hbm-stages", action="store_true",
                    help="time only the HBM scans (target argmax, draft top-k) and print their record")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run 5 attention launches and a 256 MiB calibration copy, then exit")
    return ap.parse_args()


KERNEL_SRC = os.path.join(ROOT, "mla_tree_verify_parents_amd", "csrc", "verify_attn.hip")
CALIB_BYTES = 256 << 20   # the calibration copy reads and writes this many bytes


def kernel_sha256():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic(cfg):
    """Per-launch HBM bytes (fetch + write, calibrated) of the attention
    launch from the committed counter summary, or None when there is none or
    the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"verify_attn_config{cfg}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    vals = dict(re.findall(r"^- (\w+): (\S+)$", text, re.M))
    if vals.get("kernel_source_sha256") != kernel_sha256():
        return None
    try:
        return int(vals["fetch_bytes_per_launch"]) + int(vals["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def workload_for(cfg):
    from mla_tree_verify_parents_amd import synth
    if cfg == 2:
        w = synth.workload(2)                       # logits on: argmax is part of the step
        desc = ("K2-like head share: B=1, H=8, d_lat=512, d_rope=64, bf16, prefix 4096, "
                "64 nodes (best-first, top-4, depth<=8), target logits 64x163840 fp32")
    elif cfg == 3:
        w = synth.workload(3)
        desc = "batched ragged: B=16, H=8, 512+64 bf16, prefix U[1024,32768], 32 nodes, random trees"
    elif cfg == 4:
        w = synth.workload(4)
        desc = "long context: B=4, H=64, 512+64 bf16, prefix 131072, 128 nodes (best-first, top-8, depth<=4)"
    else:
        raise SystemExit(f"bench runs configurations 2, 3, 4 or 5, not {cfg}")
    return w, desc


def spread(xs):
    """Median, min, max and (max - min) / median of a list of window figures."""
    med = float(np.median(xs))
    return {"median": round(med, 6), "min": round(min(xs), 6), "max": round(max(xs), 6),
            "rel_spread": round((max(xs) - min(xs)) / med, 4) if med > 0 else None}


def time_windows(replay, units_per_replay, est_ms_per_unit, stream, min_units=1):
    """Time WINDOWS windows of back-to-back replays on `stream` (HIP events
    around each window, synchronised on both sides).  A window holds at
    least min_units units and at least WINDOW_MS of estimated device time.
    Returns (ms per unit of every window, units per window)."""
    import torch
    reps = max(1, math.ceil(min_units / units_per_replay),
               math.ceil(WINDOW_MS / max(est_ms_per_unit * units_per_replay, 1e-6)))
    out = []
    for _ in range(WINDOWS):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / (reps * units_per_replay))
    return out, reps * units_per_replay


def graph_of(fn, n):
    """A HIP graph of n back-to-back calls of fn (captured on torch's stream)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n):
            fn()
    return g


def estimate_ms(replay, units, stream, reps=3):
    import torch
    replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * units)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the verify path here runs on a single GPU and has no "
              f"multi-GPU part (got --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.hbm_stages:
        print(json.dumps({"hbm_stages": time_hbm_stages(dev)}), flush=True)
        return
    if args.config == 5:
        if args.traffic_probe:
            return loop_traffic_probe(dev)
        res = run_loop(args, dev, args.warmup, args.loop_steps)
        add_peaks(res, args, dev)
        print(json.dumps(res), flush=True)
        return
    res = measure_config(args.config, args, dev, headline=True)
    if res is None:
        return
    if not args.no_extras:
        res["hbm_stages"] = guarded(lambda: time_hbm_stages(dev))
        progress("HBM stages timed")
        if args.config != 2:
            res["config2"] = guarded(lambda: measure_config(2, args, dev, headline=False))
            progress("config 2 timed")
        if args.config != 3:
            res["config3"] = guarded(lambda: measure_config(3, args, dev, headline=False))
            progress("config 3 timed")
        if args.config != 2:
            res["config5_loop"] = guarded(lambda: run_loop(args, dev, 3, 20, brief=True))
            progress("verify loop timed")
    add_peaks(res, args, dev)
    print(json.dumps(res), flush=True)


def progress(msg):
    """A progress line on stderr (stdout carries only the JSON line)."""
    print(f"bench: {msg} ({time.perf_counter() - T_START:.1f} s)", file=sys.stderr, flush=True)


T_START = time.perf_counter()


def guarded(f):
    """A side measurement: its failure is reported in the JSON line instead
    of taking the headline with it."""
    try:
        return f()
    except Exception as e:  # noqa: BLE001
        return {"error": f"{type(e).__name__}: {e}"}


def measure_config(cfg, args, dev, headline):
    """Time one configuration's step and attention launch; returns the JSON
    fields (the headline line, or the sub-record of a side configuration)."""
    import torch

    from mla_tree_verify_parents_amd import ddt

    w, desc = workload_for(cfg)
    progress(f"config {cfg} inputs drawn")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    pool, q = to_dev(w.pool), to_dev(w.q)
    parents, draft = to_dev(w.parents), to_dev(w.draft_ids)
    kv_base = to_dev(w.kv_base)
    # committed lengths: every step reads these and writes the advanced
    # lengths to new_prefix, so each step verifies the same tree
    prefix0 = to_dev(w.prefix_len)
    new_prefix = torch.empty_like(prefix0)
    logits = None if w.logits is None else to_dev(w.logits)
    target = None if w.target_ids is None else to_dev(w.target_ids)
    dl = w.d_lat
    q_lat, q_pe, ckv, kpe = q[:, :dl], q[:, dl:], pool[:, :dl], pool[:, dl:]
    B, N, H = w.B, w.N, w.H
    W = (N + 63) // 64
    P_host = w.prefix_len.copy()

    # preallocated outputs and workspaces: the timed loop allocates nothing
    mask = torch.empty((B, N, W), dtype=torch.int64, device=dev)
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    terr = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((w.rows, dl), dtype=q.dtype, device=dev)
    lse = torch.empty((w.rows,), dtype=torch.float32, device=dev)
    desc_c = ddt.attn_desc(q_lat, q_pe, ckv, kpe, B=B, H=H, N=N, scale=w.scale)
    ws_bytes = ddt.verify_workspace_bytes(desc_c, P_host)
    ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
    tids = torch.empty((B * N,), dtype=torch.int32, device=dev)
    am_ws = None
    if logits is not None:
        n = ddt.argmax_workspace_bytes(B * N, logits.shape[1])
        am_ws = torch.zeros((max(n, 16),), dtype=torch.uint8, device=dev)   # zero before first use
    acc = torch.empty((B,), dtype=torch.int32, device=dev)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    tok = torch.empty((B, N), dtype=torch.int32, device=dev)

    # every call launches on torch's current stream, so the step can be
    # captured into a HIP graph and replayed without host launch overhead
    def attn():
        ddt.verify_attn(q_lat, q_pe, ckv, kpe, kv_base, P_host, mask, H=H, scale=w.scale, out=out, lse=lse,
                        workspace=ws)

    in_kernel_mask = N <= 128

    def step():
        if logits is not None:
            # two launches: the attention with the (independent) target argmax
            # on the CUs it leaves idle, then the split merge with acceptance +
            # compaction + length update beside it; trees of up to 128 nodes
            # get their ancestor bits inside the attention (no mask launch)
            if not in_kernel_mask:
                ddt.build_mask(parents, mask, depth, terr)
            ddt.verify_step(q_lat, q_pe, ckv, kpe, kv_base, P_host, None if in_kernel_mask else mask, logits,
                            draft, parents, prefix0, H=H, scale=w.scale, new_prefix_len=new_prefix, out=out,
                            lse=lse, workspace=ws, idx=tids, argmax_workspace=am_ws, accept_len=acc, path=path,
                            tokens=tok)
        else:
            ddt.build_mask(parents, mask, depth, terr)
            attn()
            ddt.accept_compact(target, draft, parents, ckv, kpe, kv_base, prefix0, acc, path, tok,
                               new_prefix_len=new_prefix)

    if args.traffic_probe and headline:
        ddt.build_mask(parents, mask, depth, terr)
        for _ in range(5):
            attn()
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": f"config{cfg}", "attn_launches": 5,
                          "calibration_copy_bytes": CALIB_BYTES}), flush=True)
        return None

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        ddt.build_mask(parents, mask, depth, terr)  # for the attention-only launches timed below
        for _ in range(max(1, min(args.warmup, 3))):
            step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    # steps captured several to a graph when they are short (a device-resident
    # loop replays several steps per launch); one-step graphs, whose every
    # replay pays the host's graph launch, are timed beside them
    g_one = graph_of(step, 1)
    est_step = estimate_ms(g_one.replay, 1, stream)
    spg = 10 if est_step < 0.5 else 1
    g_step = graph_of(step, spg) if spg > 1 else g_one
    for _ in range(-(-args.warmup // spg)):
        g_step.replay()
    step_ms, step_units = time_windows(g_step.replay, spg, est_step, stream, min_units=args.steps)
    one_ms, _ = time_windows(g_one.replay, 1, est_step, stream, min_units=args.steps) if spg > 1 else (step_ms, 0)
    ms_step = float(np.median(step_ms))

    # the dominant launch alone: back-to-back attention calls in one graph
    # (at least WINDOW_MS per window)
    g_a1 = graph_of(attn, 1)
    est_attn = estimate_ms(g_a1.replay, 1, stream)
    per_graph = max(1, min(200, int(WINDOW_MS / max(est_attn, 1e-4))))
    g_attn = graph_of(attn, per_graph)
    g_attn.replay()
    attn_ms, attn_units = time_windows(g_attn.replay, per_graph, est_attn, stream)
    ms_attn = float(np.median(attn_ms))
    del g_one, g_step, g_a1, g_attn
    progress(f"config {cfg} step and attention timed")
    small = guarded(lambda: time_small_kernels(parents, draft, target if target is not None else tids, ckv, kpe,
                                               kv_base, prefix0, new_prefix, mask, depth, terr, acc, path, tok,
                                               stream))

    pairs = w.visible_pairs()
    flops = pairs * FLOP_PER_PAIR
    keys = int(w.keys().sum())
    attn_bytes = keys * (dl + w.d_rope) * 2 + w.rows * ((dl + w.d_rope) * 2 + dl * 2 + 4)
    achieved = flops / (ms_attn * 1e-3) / 1e12

    res = {
        "metric": "verify-attn TFLOP/s + cache tokens/s; % of MFMA/HBM roofline, 1xMI355X",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents and queries, best-first draft tree, planted targets)",
        "config": {"workload": f"config{cfg} {desc}", "requests": B, "heads": H, "nodes": N,
                   "cache_tokens": keys, "visible_pairs": pairs, "attn_flop_per_step": flops},
        "cache_tokens_per_s": round(keys / (ms_step * 1e-3), 1),
        "step_timing": {"median_of": WINDOWS, "steps_per_window": step_units, "steps_per_graph": spg,
                        "ms_per_step": spread(step_ms),
                        "note": "each window: HIP events on the launch stream around back-to-back graph "
                                "replays of steps_per_window steps, synchronised on both sides; ms_per_step "
                                "is the median window"},
        "verify_attn_ms": round(ms_attn, 5),
        "verify_attn_timing": {"median_of": WINDOWS, "launches_per_window": attn_units,
                               "ms_per_launch": spread(attn_ms)},
        "verify_attn_cache_tokens_per_s": round(keys / (ms_attn * 1e-3), 1),
        "roofline": {"bound": "mfma", "kernel": "verify_split+verify_combine (ddt_verify_attn)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": recorded_traffic(cfg),
                     "algorithmic_flop_per_launch": flops, "algorithmic_bytes": attn_bytes,
                     "achieved_GBps": round(attn_bytes / (ms_attn * 1e-3) / 1e9, 1),
                     "achieved_hbm_frac": round(attn_bytes / (ms_attn * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
    }
    if spg > 1:
        res["step_timing"]["one_step_graphs_ms_per_step"] = spread(one_ms)
    res["small_kernels"] = small
    if not headline:
        for k in ("metric", "n_gpus", "steps", "warmup", "higher_is_better", "scaling", "vs_baseline", "dtype",
                  "data", "unit"):
            res.pop(k, None)
        return res
    if cfg in (2, 3) and not args.no_cold:
        ms_cold, n_copies = time_cold_attn(pool, dl, q_lat, q_pe, kv_base, P_host, mask, H, w.scale, out, lse, ws,
                                           side, stream)
        res["cold_cache"] = {"verify_attn_ms": round(ms_cold, 5), "cache_copies": n_copies,
                             "copy_bytes": pool.numel() * pool.element_size(),
                             "achieved_TFLOPs": round(flops / (ms_cold * 1e-3) / 1e12, 2),
                             "frac": round(flops / (ms_cold * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                             "note": "back-to-back launches rotating over distinct copies of the cache "
                                     f"(at least {COLD_BYTES >> 20} MiB in all), so the last-level cache "
                                     "cannot serve the keys"}
    if not args.no_extras:
        progress("side measurements (paged, prefill, projections)")
        res["paged"] = guarded(lambda: time_paged(w, dev, q_lat, q_pe, mask, ms_attn))
        res["prefill"] = guarded(lambda: time_prefill(dev))
        res["projections"] = [guarded(lambda: time_projections(B * N, H, dev))]
        if B * N < 2048:
            res["projections"].append(guarded(lambda: time_projections(2048, 8, dev)))   # the loop's 32 x 64 nodes
    del pool, q
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        progress("oracle timing on the host")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, flops)
    return res


def time_small_kernels(parents, draft, target, ckv, kpe, kv_base, prefix0, new_prefix, mask, depth, terr, acc, path,
                       tok, stream):
    """The latency-bound kernels of the step alone, at the configuration's
    shape: µs per call (median of WINDOWS windows of >= WINDOW_MS of
    back-to-back calls in graphs) of the ancestor-mask build, greedy
    acceptance, and acceptance + compaction + length update in one launch
    (the form the step uses), with the compaction's effective bandwidth:
    bytes = 2 x (accepted path lengths, root included) x row bytes."""
    import torch

    from mla_tree_verify_parents_amd import ddt

    def per_call_us(fn):
        g1 = graph_of(fn, 1)
        est = estimate_ms(g1.replay, 1, stream)
        per = max(1, min(500, int(2.0 / max(est, 1e-4))))
        g = graph_of(fn, per)
        g.replay()
        ms, units = time_windows(g.replay, per, est, stream)
        del g1, g
        return {"us": round(float(np.median(ms)) * 1e3, 3), "us_spread": spread([m * 1e3 for m in ms]),
                "calls_per_window": units}

    res = {"mask": per_call_us(lambda: ddt.build_mask(parents, mask, depth, terr)),
           "greedy_accept": per_call_us(lambda: ddt.greedy_accept(target, draft, parents, acc, path, tok))}
    res["accept_compact"] = per_call_us(lambda: ddt.accept_compact(target, draft, parents, ckv, kpe, kv_base,
                                                                   prefix0, acc, path, tok,
                                                                   new_prefix_len=new_prefix))
    torch.cuda.synchronize()
    moved = int(acc.sum().item()) + int(acc.numel())
    row_bytes = (ckv.shape[1] + kpe.shape[1]) * ckv.element_size()
    res["accept_compact"]["rows_moved"] = moved
    res["accept_compact"]["GBps"] = round(2 * moved * row_bytes / (res["accept_compact"]["us"] * 1e-6) / 1e9, 2)
    return res


def time_hbm_stages(dev):
    """The HBM scans of the end-to-end step on their own, at its shapes:
    the target argmax over 2048 x 163840 fp32 logits (ddt_argmax) and the
    draft top-8 over 256 x 163840 fp32 (ddt_draft_topk); bytes = rows x V x 4,
    against 8 TB/s."""
    import torch

    from mla_tree_verify_parents_amd import ddt

    stream = torch.cuda.current_stream()
    g = torch.Generator(device=dev)
    g.manual_seed(5005)
    V = 163840
    res = {}
    for name, rows in (("argmax", 2048), ("draft_topk", 256)):
        x = torch.randn((rows, V), generator=g, device=dev, dtype=torch.float32)
        if name == "argmax":
            idx = torch.empty((rows,), dtype=torch.int32, device=dev)
            ws = torch.zeros((max(16, ddt.argmax_workspace_bytes(rows, V)),), dtype=torch.uint8, device=dev)
            fn = lambda: ddt.argmax(x, idx, ws)   # noqa: E731
        else:
            ids = torch.empty((rows, 8), dtype=torch.int32, device=dev)
            lp = torch.empty((rows, 8), dtype=torch.float32, device=dev)
            ws = torch.empty((max(16, ddt.draft_topk_workspace_bytes(rows, V, 8)),), dtype=torch.uint8, device=dev)
            fn = lambda: ddt.draft_topk(x, 8, ids, lp, ws)   # noqa: E731
        fn()
        g1 = graph_of(fn, 1)
        est = estimate_ms(g1.replay, 1, stream)
        per = max(1, min(500, int(WINDOW_MS / max(est, 1e-4))))
        gn = graph_of(fn, per)
        gn.replay()
        ms, n = time_windows(gn.replay, per, est, stream)
        med = float(np.median(ms))
        nbytes = rows * V * 4
        gbps = nbytes / (med * 1e-3) / 1e9
        res[name] = {"rows": rows, "vocab": V, "bytes": nbytes, "us": round(med * 1e3, 3),
                     "us_spread": spread([m * 1e3 for m in ms]), "launches_per_window": n,
                     "GBps": round(gbps, 1), "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4)}
        del gn, g1, x, ws
    res["note"] = "median of 5 windows of back-to-back launches in one graph; bytes = rows x V x 4 read once"
    return res


def loop_traffic_probe(dev):
    """The verify loop's attention launch (first iteration's inputs: 32
    requests, prefixes U[2048, 65536], 64 nodes) 5 times, then the 256 MiB
    calibration copy: the program the HBM-traffic counters profile."""
    import torch

    from mla_tree_verify_parents_amd import ddt, e2e

    loop = e2e.VerifyLoop(steps=1)
    inp = loop.make_inputs()
    mask = ddt.build_mask(inp.parents_dev)[0]
    dl = loop.d_lat
    ws = loop.workspace_for(inp.prefix_len)
    for _ in range(5):
        ddt.verify_attn(inp.q[:, :dl], inp.q[:, dl:], loop.ckv(), loop.kpe(), loop.kv_base, inp.prefix_len, mask,
                        H=loop.H, scale=loop.scale, out=loop.out, lse=loop.lse, workspace=ws)
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": "config5", "attn_launches": 5, "calibration_copy_bytes": CALIB_BYTES}),
          flush=True)


def run_loop(args, dev, W, K, brief=False):
    """Configuration 5: the verify loop.  Every iteration draws its inputs
    (untimed: draft logits, node latents, queries, target logits planted on
    the tree), runs the draft stage on the device (top-8 per depth and the
    best-first trees; timed with HIP events), then the hot path (one
    ddt_verify_step call: ancestor bits, attention, argmax, acceptance,
    compaction, length update; two launches; timed with HIP events), then
    advances the loop (the bonus token is the next root; the host mirrors the
    grown lengths).  A step's time is the two stages' device time; `value` is
    the attention FLOPs of all timed iterations over their summed step time.
    brief: fewer fields (a side record of another configuration's line)."""
    import torch

    from mla_tree_verify_parents_amd import ddt, e2e, synth

    loop = e2e.VerifyLoop(steps=W + K, page_size=args.page_size)
    stream = torch.cuda.current_stream()
    t_ms, flops, keys, acc_sum = 0.0, 0, 0, 0
    host_s, plan_s, draft_ms, verify_ms = 0.0, 0.0, 0.0, 0.0
    per_iter = []
    snap = None
    for it in range(W + K):
        h0 = time.perf_counter()
        inp = loop.make_inputs()       # draws on the device; the best-first trees are built on the device
        h1 = time.perf_counter()
        if it == 0 and not brief and not args.no_cpu_baseline:  # (a warmup iteration unless W == 0)
            snap = (synth.Workload(name="config5", B=loop.B, H=loop.H, N=loop.N, d_lat=loop.d_lat,
                                   d_rope=loop.d_rope, dtype="bf16", scale=loop.scale,
                                   prefix_len=inp.prefix_len.copy(), kv_base=loop.kv_base_host.copy(),
                                   capacity=loop.capacity.copy(), pool=loop.to_logical(to_host_bits(loop.pool)),
                                   q=to_host_bits(inp.q), parents=inp.parents, draft_ids=inp.draft_ids,
                                   logits=inp.logits.cpu().numpy(), vocab=loop.vocab),
                    inp.visible_pairs(loop.H) * FLOP_PER_PAIR)
        # e0 follows the input generation on the stream (no host sync): the
        # host plans and enqueues the step while the GPU still draws inputs,
        # so e0..e1 is the step's device time
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        p0 = time.perf_counter()
        res = loop.run_step(inp)
        p1 = time.perf_counter()
        e1.record(stream)
        torch.cuda.synchronize()
        acc = loop.advance(res)
        if it >= W:
            host_s += h1 - h0
            plan_s += p1 - p0
            draft_ms += inp.draft_ms
            verify_ms += e0.elapsed_time(e1)
            t_ms += inp.draft_ms + e0.elapsed_time(e1)
            per_iter.append(inp.draft_ms + e0.elapsed_time(e1))
            flops += inp.visible_pairs(loop.H) * FLOP_PER_PAIR
            keys += int(inp.prefix_len.sum()) + loop.B * loop.N
            acc_sum += int(acc.sum())
    ms_step = t_ms / K
    # the attention launch alone on the last iteration's inputs, for the roofline
    mask = ddt.build_mask(inp.parents_dev)[0]
    dl = loop.d_lat
    ws = loop.workspace_for(inp.prefix_len)

    def attn():
        ddt.verify_attn(inp.q[:, :dl], inp.q[:, dl:], loop.ckv(), loop.kpe(), None if loop.page_size else loop.kv_base,
                        inp.prefix_len, mask, H=loop.H, scale=loop.scale, out=loop.out, lse=loop.lse, workspace=ws,
                        pages=loop.pages())

    attn()
    torch.cuda.synchronize()
    g1 = graph_of(attn, 1)
    est = estimate_ms(g1.replay, 1, stream)
    per = max(1, min(100, int(WINDOW_MS / max(est, 1e-4))))
    gn = graph_of(attn, per)
    gn.replay()
    attn_ms, attn_units = time_windows(gn.replay, per, est, stream)
    ms_attn = float(np.median(attn_ms))
    del g1, gn
    # the whole verify step on the same inputs, back to back: the loop's own
    # iterations leave the GPU idle while the host draws the next inputs, and
    # the clock is lower after such gaps, so this is the step at a steady clock
    # (committed lengths read from a copy, advanced lengths to another: every
    # replay is the same step)
    p_before = torch.from_numpy(inp.prefix_len.astype(np.int32)).to(dev)
    p_after = torch.empty_like(p_before)

    def step():
        ddt.verify_step(inp.q[:, :dl], inp.q[:, dl:], loop.ckv(), loop.kpe(),
                        None if loop.page_size else loop.kv_base, inp.prefix_len, mask if loop.N > 128 else None,
                        inp.logits, inp.draft_dev, inp.parents_dev, p_before, H=loop.H, scale=loop.scale,
                        new_prefix_len=p_after, out=loop.out, lse=loop.lse, workspace=ws, idx=loop.idx,
                        argmax_workspace=loop.am_ws, accept_len=loop.acc, path=loop.path, tokens=loop.tok,
                        pages=loop.pages())

    step()
    torch.cuda.synchronize()
    g1 = graph_of(step, 1)
    est = estimate_ms(g1.replay, 1, stream)
    per = max(1, min(100, int(WINDOW_MS / max(est, 1e-4))))
    gn = graph_of(step, per)
    gn.replay()
    step_ms, step_units = time_windows(gn.replay, per, est, stream)
    del g1, gn
    last_flops = inp.visible_pairs(loop.H) * FLOP_PER_PAIR
    achieved = last_flops / (ms_attn * 1e-3) / 1e12
    last_keys = int(inp.prefix_len.sum()) + loop.B * loop.N
    attn_bytes = last_keys * (dl + loop.d_rope) * 2 + loop.B * loop.N * loop.H * ((dl + loop.d_rope) * 2 + dl * 2 + 4)
    draft = time_draft_step(loop, stream)
    res = {
        "metric": "verify-attn TFLOP/s + cache tokens/s; % of MFMA/HBM roofline, 1xMI355X",
        "value": round(flops / (t_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) latents, queries and target logits with planted tokens; "
                "best-first trees from N(0,9) draft logits)",
        "config": {"workload": "config5 verify loop: B=32, H=8, 512+64 bf16, prefix U[2048,65536] growing, "
                               "64 nodes (best-first, top-8, depth<=8), target logits 2048x163840 fp32",
                   "requests": loop.B, "heads": loop.H, "nodes": loop.N, "iterations": K,
                   "page_size": args.page_size,
                   "cache_tokens_per_iteration": keys / K, "accepted_drafts_per_request_step": acc_sum / (K * loop.B),
                   "attn_flop_per_step": flops / K},
        "cache_tokens_per_s": round(keys / (t_ms * 1e-3), 1),
        "step_timing": {"ms_per_iteration": spread(per_iter),
                        "note": "ms_per_step is the mean over the timed iterations (the cache grows, so "
                                "iterations differ); each iteration: HIP events around its two stages"},
        "verify_attn_ms": round(ms_attn, 5),
        "verify_attn_timing": {"median_of": WINDOWS, "launches_per_window": attn_units,
                               "ms_per_launch": spread(attn_ms)},
        "roofline": {"bound": "mfma", "kernel": "verify_split+verify_combine (ddt_verify_attn), last iteration",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": recorded_traffic(5),
                     "algorithmic_flop_per_launch": last_flops, "algorithmic_bytes": attn_bytes,
                     "achieved_GBps": round(attn_bytes / (ms_attn * 1e-3) / 1e9, 1),
                     "achieved_hbm_frac": round(attn_bytes / (ms_attn * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)},
        "draft_step": draft,
        "stage_ms_per_iteration": {"draft_topk_and_trees": round(draft_ms / K, 5),
                                   "verify_step": round(verify_ms / K, 5),
                                   "note": "device time; ms_per_step is their sum"},
        "verify_step_steady": {"ms": round(float(np.median(step_ms)), 5), "ms_spread": spread(step_ms),
                               "steps_per_window": step_units,
                               "note": "ddt_verify_step on the last iteration's inputs, back-to-back graph "
                                       "replays (median of 5 windows of >= 50 ms): the step at a steady clock, "
                                       "without the idle gaps the loop's host-side input drawing leaves"},
        "host_ms_per_iteration": {"inputs_and_trees": round(host_s * 1e3 / K, 3),
                                  "plan_and_enqueue": round(plan_s * 1e3 / K, 3),
                                  "note": "host wall time: drawing the inputs and running the draft stage (with "
                                          "the host copies the input generator needs), then planning + "
                                          "enqueueing the verify step's two launches"},
    }
    if brief:
        for k in ("metric", "n_gpus", "warmup", "higher_is_better", "scaling", "vs_baseline", "dtype", "data",
                  "unit", "host_ms_per_iteration"):
            res.pop(k, None)
    del loop
    torch.cuda.empty_cache()
    if snap is not None:
        res["cpu_baseline"] = cpu_baseline(snap[0], args.cpu_seconds, snap[1])
    return res


COLD_BYTES = 2 * (256 << 20)  # twice the last-level cache


def time_cold_attn(pool, dl, q_lat, q_pe, kv_base, P_host, mask, H, scale, out, lse, ws, side, stream):
    """Attention time with the keys out of every cache: one graph of
    launches that each read a different copy of the cache pool, the copies
    together at least COLD_BYTES.  Returns (ms per launch, copies)."""
    import torch

    from mla_tree_verify_parents_amd import ddt

    nbytes = pool.numel() * pool.element_size()
    n = max(2, -(-COLD_BYTES // nbytes) + 1)
    copies = [pool.clone() for _ in range(n)]

    def run_all():
        for c in copies:
            ddt.verify_attn(q_lat, q_pe, c[:, :dl], c[:, dl:], kv_base, P_host, mask, H=H, scale=scale, out=out,
                            lse=lse, workspace=ws)

    with torch.cuda.stream(side):
        run_all()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_all()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n)
    del g, copies
    torch.cuda.empty_cache()
    return ms, n


def measure_peaks(dev):
    """What the device sustains, measured by the library's probe kernels on
    this run: a bf16 MFMA loop on random N(0,1) operands and on zeros (the
    board power limit sets the clock, and the clock depends on the
    operands), a streaming HBM read and a streaming copy."""
    import torch

    from mla_tree_verify_parents_amd import ddt

    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()

    def timed(f, reps, warm):
        for _ in range(warm):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"cus": cus}
    # two wavefronts per SIMD: the loop then issues at about 97 % of the MFMA
    # rate (four or more per SIMD measured 20 % lower)
    blocks, iters = 2 * cus, 4096
    flop = blocks * 4 * iters * ddt.PROBE_MFMA_FLOP_PER_WAVE_ITER
    g = torch.Generator(device=dev)
    g.manual_seed(1009)
    for name, ops in (("random", torch.randn(ddt.PROBE_MFMA_OPERANDS, generator=g, device=dev)),
                      ("zero", torch.zeros(ddt.PROBE_MFMA_OPERANDS, device=dev))):
        ops = ops.to(torch.bfloat16)
        sink = torch.empty(blocks * ddt.PROBE_THREADS, dtype=torch.float32, device=dev)
        clk = torch.empty((blocks, 2), dtype=torch.int64, device=dev)
        ms = timed(lambda: ddt.probe_mfma_bf16(ops, blocks, iters, sink=sink, clk=clk), 20, 10)
        c = clk.sum(dim=0).tolist()
        out[f"mfma_bf16_{name}_TFLOPs"] = round(flop / (ms * 1e-3) / 1e12, 1)
        out[f"mfma_bf16_{name}_core_GHz"] = round(0.1 * c[0] / max(c[1], 1), 3)
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    sink = torch.empty(8 * cus * ddt.PROBE_THREADS, dtype=torch.int32, device=dev)
    ms = timed(lambda: ddt.probe_read(src, 8 * cus, sink=sink), 20, 3)
    out["hbm_read_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    half = src[: nbytes // 2]
    dst = src[nbytes // 2:]
    ms = timed(lambda: ddt.probe_copy(half, dst, 8 * cus), 20, 3)
    out["hbm_copy_GBps"] = round(2 * half.numel() / (ms * 1e-3) / 1e9, 1)
    out["note"] = ("achieved rates of the probe kernels on this device and run (MFMA loop: 4 independent "
                   "32x32x16 bf16 chains per wavefront, 2 wavefronts per SIMD; HBM: 2 GiB read, 1 GiB copy)")
    del src, sink
    return out


def add_peaks(res, args, dev):
    if args.no_peaks:
        return
    pk = measure_peaks(dev)
    res["measured_peaks"] = pk
    res["roofline"]["frac_of_measured_mfma_random"] = round(res["roofline"]["achieved"] /
                                                            pk["mfma_bf16_random_TFLOPs"], 4)


def time_draft_step(loop, stream):
    """The step before the verify path, on the device, at the loop's shape:
    per-depth top-k of N(0, 3^2) draft logits (B*D rows x vocabulary) and
    the best-first trees (the loop's draft stage).  The top-k is an HBM
    scan, reported against 8 TB/s."""
    import torch

    from mla_tree_verify_parents_amd import ddt

    B, D, K, V = loop.B, loop.D, loop.K, loop.vocab
    g = torch.Generator(device=loop.device)
    g.manual_seed(loop.seed)
    x = torch.randn((B * D, V), generator=g, device=loop.device, dtype=torch.float32) * loop.sigma
    ids = torch.empty((B * D, K), dtype=torch.int32, device=loop.device)
    lp = torch.empty((B * D, K), dtype=torch.float32, device=loop.device)
    ws = torch.empty((max(16, ddt.draft_topk_workspace_bytes(B * D, V, K)),), dtype=torch.uint8, device=loop.device)
    roots = torch.from_numpy(loop.roots.copy()).to(loop.device)
    outs = [torch.empty((B, loop.N), dtype=torch.int32, device=loop.device) for _ in range(3)]

    def topk():
        ddt.draft_topk(x, K, ids, lp, ws)

    def tree():
        ddt.best_first_tree(ids.view(B, D, K), lp.view(B, D, K), roots, loop.N - 1, *outs)

    def timed(f):
        f()
        torch.cuda.synchronize()
        g1 = graph_of(f, 1)
        est = estimate_ms(g1.replay, 1, stream)
        per = max(1, min(500, int(WINDOW_MS / max(est, 1e-4))))
        gn = graph_of(f, per)
        gn.replay()
        ms, _ = time_windows(gn.replay, per, est, stream)
        return float(np.median(ms))

    ms_topk, ms_tree = timed(topk), timed(tree)
    gbps = B * D * V * 4 / (ms_topk * 1e-3) / 1e9
    return {"rows": B * D, "vocab": V, "k": K, "topk_ms": round(ms_topk, 5), "tree_ms": round(ms_tree, 5),
            "topk_GBps": round(gbps, 1), "topk_hbm_frac": round(gbps / PEAK_HBM_GBPS, 4)}


def time_projections(tokens, H, dev, reps=200, d_nope=128, d_lat=512, d_rope=64, d_v=128):
    """The per-head projections around the attention (ddt_head_proj) at
    `tokens` tree nodes x H heads: q_nope @ w_kc[h] -> the first d_lat
    columns of the q_lat|q_pe rows, and out_lat @ w_vc[h] -> o.  Each is
    a graph of `reps` back-to-back launches, timed in 5 windows of >= 50 ms
    of replays (the median reported).  Algorithmic bytes
    per launch: every input and output row once plus the weights once; at
    about 100 flop/B they are HBM-bound, reported against 8 TB/s (and
    their flops against the bf16 MFMA peak)."""
    import torch

    from mla_tree_verify_parents_amd import ddt

    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    rows = tokens * H
    q_nope = torch.randn((rows, d_nope), generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn((rows, d_lat + d_rope), generator=g, device=dev).to(torch.bfloat16)
    out_lat = torch.randn((rows, d_lat), generator=g, device=dev).to(torch.bfloat16)
    o = torch.empty((rows, d_v), dtype=torch.bfloat16, device=dev)
    w_kc = ddt.proj_pack_weight((torch.randn((H, d_nope, d_lat), generator=g, device=dev) / d_nope ** 0.5)
                                .to(torch.bfloat16))
    w_vc = ddt.proj_pack_weight((torch.randn((H, d_lat, d_v), generator=g, device=dev) / d_lat ** 0.5)
                                .to(torch.bfloat16))
    stream = torch.cuda.current_stream()
    res = {"tokens": tokens, "heads": H}
    for name, f, K, n in (("absorb_q", lambda: ddt.head_proj(q_nope, w_kc, H, y=q[:, :d_lat]), d_nope, d_lat),
                          ("absorb_out", lambda: ddt.head_proj(out_lat, w_vc, H, y=o), d_lat, d_v)):
        f()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                f()
        graph.replay()
        torch.cuda.synchronize()
        est = estimate_ms(graph.replay, reps, stream)
        win, units = time_windows(graph.replay, reps, est, stream)
        ms = float(np.median(win))
        nbytes = rows * (K + n) * 2 + H * K * n * 2
        flop = 2 * rows * K * n
        gbps = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"K": K, "n_out": n, "us": round(ms * 1e3, 3), "us_spread": spread([x * 1e3 for x in win]),
                     "launches_per_window": units, "GBps": round(gbps, 1),
                     "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
                     "TFLOPs": round(flop / (ms * 1e-3) / 1e12, 2), "bytes": nbytes}
    return res


def time_paged(w, dev, q_lat, q_pe, mask, ms_contiguous, page_size=64):
    """The same attention launch with the latent cache in pages of
    `page_size` rows of one shared pool, scattered by a random permutation
    (block table; one row lookup per 32-key tile), against the contiguous
    launch's time (both the median of WINDOWS windows of at least WINDOW_MS
    of back-to-back launches)."""
    import torch

    from mla_tree_verify_parents_amd import ddt

    rng = np.random.default_rng(page_size)
    T = w.prefix_len.astype(np.int64) + w.N
    npg = (T + page_size - 1) // page_size
    total = int(npg.sum())
    perm = rng.permutation(total).astype(np.int32)
    table = np.zeros((w.B, int(npg.max())), np.int32)
    src, dst, k = [], [], 0
    for b in range(w.B):
        table[b, : npg[b]] = perm[k: k + npg[b]]
        k += npg[b]
        t = np.arange(T[b])
        src.append(w.kv_base[b] + t)
        dst.append(table[b, t // page_size].astype(np.int64) * page_size + t % page_size)
    pool = torch.from_numpy(np.ascontiguousarray(w.pool).view(np.int16)).to(dev).view(torch.bfloat16)
    phys = torch.zeros((total * page_size, pool.shape[1]), dtype=pool.dtype, device=dev)
    phys[torch.from_numpy(np.concatenate(dst)).to(dev)] = pool[torch.from_numpy(np.concatenate(src)).to(dev)]
    del pool
    td = torch.from_numpy(table).to(dev)
    dl = w.d_lat
    out = torch.empty((w.rows, dl), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.rows,), dtype=torch.float32, device=dev)
    pages = (td, page_size)
    d = ddt.attn_desc(q_lat, q_pe, phys[:, :dl], phys[:, dl:], B=w.B, H=w.H, N=w.N, scale=w.scale, pages=pages)
    ws = torch.empty((max(1, ddt.verify_workspace_bytes(d, w.prefix_len)),), dtype=torch.uint8, device=dev)

    def f():
        ddt.verify_attn(q_lat, q_pe, phys[:, :dl], phys[:, dl:], None, w.prefix_len, mask, H=w.H, scale=w.scale,
                        out=out, lse=lse, workspace=ws, pages=pages)

    f()
    torch.cuda.synchronize()
    graph = graph_of(f, 1)
    stream = torch.cuda.current_stream()
    wins, per_window = time_windows(graph.replay, 1, ms_contiguous, stream)
    ms = float(np.median(wins))
    return {"page_size": page_size, "pages": total, "verify_attn_ms": round(ms, 5), "ms_spread": spread(wins),
            "launches_per_window": per_window, "contiguous_ms": round(ms_contiguous, 5),
            "ratio": round(ms / ms_contiguous, 4)}


def time_prefill(dev, T=8192, P0=0, H=8, chunk=1024):
    """Causal prefill of a T-token prompt through the verify attention
    (chain-tree masks, chunks of `chunk` tokens, one verify call each; the
    chunk loop captured in one graph, timed in WINDOWS windows of at least
    WINDOW_MS of replays, median window).  Visible pairs: H * sum_t (P0+t+1)."""
    import torch

    from mla_tree_verify_parents_amd import synth
    from mla_tree_verify_parents_amd.prefill import ChunkedPrefill

    rng = np.random.default_rng(8192)
    dl, dr = 512, 64
    pool, base, _ = synth.make_pool(rng, np.array([P0], np.int32), T, dl + dr, "bf16")
    q = synth.normal(rng, (T * H, dl + dr), "bf16")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    pd, qd = to(pool), to(q)
    kvb = torch.from_numpy(base).to(dev)
    pf = ChunkedPrefill(H, 1.0 / np.sqrt(dl + dr), chunk=chunk, device=dev)
    out = torch.empty((T * H, dl), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T * H,), dtype=torch.float32, device=dev)

    def run():
        pf.run(qd[:, :dl], qd[:, dl:], pd[:, :dl], pd[:, dl:], kvb, P0, out=out, lse=lse)

    run()                      # builds the chain masks and the workspace
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    stream = torch.cuda.current_stream()
    est = estimate_ms(graph.replay, 1, stream)
    wins, per_window = time_windows(graph.replay, 1, est, stream)
    ms = float(np.median(wins))
    pairs = H * (T * P0 + T * (T + 1) // 2)
    tflops = pairs * FLOP_PER_PAIR / (ms * 1e-3) / 1e12
    return {"tokens": T, "prefix": P0, "heads": H, "chunk": chunk, "chunks": len(pf.chunks(T, P0)),
            "calls": len(pf.calls(T, P0)),
            "ms": round(ms, 4), "ms_spread": spread(wins), "prompts_per_window": per_window,
            "visible_pairs": pairs, "TFLOPs": round(tflops, 1), "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1)}


def to_host_bits(t):
    """bf16 device tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def row_pairs(w):
    """Visible keys of every flat query row (prefix plus ancestors and self)."""
    per = np.empty((w.B, w.N), np.int64)
    for b in range(w.B):
        d = np.zeros(w.N, np.int64)
        for i in range(1, w.N):
            d[i] = d[w.parents[b, i]] + 1
        per[b] = int(w.prefix_len[b]) + d + 1
    return np.repeat(per.reshape(-1), w.H)


def cpu_baseline(w, budget_s, flops):
    """Time the fp64 oracle on the host for the same verify step: mask,
    attention, argmax, acceptance, compaction.  The attention runs on every
    query row when that fits the time budget, else on a seeded random sample
    of rows sized to it, and its time is scaled by visible pairs."""
    from oracle import oracle

    oracle.lib()
    pairs = row_pairs(w)
    total = int(pairs.sum())
    rng = np.random.default_rng(0)
    # rate probe on a few rows decides the sample size
    probe = np.sort(rng.choice(w.rows, min(w.rows, 16), replace=False))
    t0 = time.perf_counter()
    oracle.verify_attn(w.q_lat(), w.q_pe(), w.ckv(), w.kpe(), w.kv_base, w.prefix_len, w.parents,
                       H=w.H, scale=w.scale, rows=probe)
    rate = pairs[probe].sum() / max(time.perf_counter() - t0, 1e-6)   # pairs per second
    n = w.rows if total / rate <= 0.8 * budget_s else max(16, int(w.rows * 0.8 * budget_s * rate / total))
    rows = None if n >= w.rows else np.sort(rng.choice(w.rows, n, replace=False))
    reps, t_att, t_rest = 0, 0.0, 0.0
    while True:   # whole steps, repeated while within the budget (at most 20)
        t0 = time.perf_counter()
        oracle.build_mask(w.parents)
        oracle.verify_attn(w.q_lat(), w.q_pe(), w.ckv(), w.kpe(), w.kv_base, w.prefix_len, w.parents,
                           H=w.H, scale=w.scale, rows=rows)
        t1 = time.perf_counter()
        t = oracle.argmax(w.logits).reshape(w.B, w.N) if w.logits is not None else w.target_ids
        a, pth, _ = oracle.greedy_accept(t, w.draft_ids, w.parents)
        pool = w.pool.copy()
        oracle.compact_kv(pool[:, :w.d_lat], pool[:, w.d_lat:], w.kv_base, w.prefix_len, pth, a)
        t2 = time.perf_counter()
        reps += 1
        t_att += t1 - t0
        t_rest += t2 - t1
        if t_att + t_rest >= budget_s or reps >= 20:
            break
    sampled = total if rows is None else int(pairs[rows].sum())
    att = t_att / reps * total / sampled
    step_s = att + t_rest / reps
    what = "all query rows" if rows is None else f"{n} of {w.rows} query rows (seeded), time scaled by visible pairs"
    return {"value": round(flops / step_s / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} verify step(s) of the same workload, attention on {what}; "
                      f"{step_s * 1e3:.1f} ms/step ({att * 1e3:.1f} ms attention)"}


if __name__ == "__main__":
    main()
