#!/usr/bin/env python3
"""MLRA-4 decode-attention benchmark on one MI355X.

One step = one full decode of the workload's batch through the C ABI
(split-KV attention kernel, combine/W_UV kernel, finalize kernel), inputs resident in HBM.

    python bench.py [--steps K] [--warmup W] [--config 2] [--no-cpu-baseline]

Prints one JSON line. `value` is microseconds per step (lower is better) for the
workload the headline metric is quoted on (B=32, h=32, L=32768, MLRA-4, bf16).

Order: W untimed warm-up steps, then a settle phase of back-to-back steps (at least
--settle-min-ms, until three consecutive 20-step windows agree within 1.5 %, at most
--settle-max-ms; reported as `settle`), then the K timed steps. On MI355X the step runs
15-45 % slow for 25-45 ms after any change of load (a fresh process, an idle gap of
20 ms or more, a burst of other kernels) whatever the shader clock reads; the settle
phase waits that out without depending on W.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLRA-4 decode attn µs/step + achieved HBM TB/s (B=32, h=32, L=32K)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense
def flop_per_head_token(w):
    """QK over the latent and RoPE channels (the RoPE dot once per head) plus PV over the latent."""
    return 2 * (w.NB * w.DL + w.DR) + 2 * w.NB * w.DL


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before the settle phase")
    ap.add_argument("--settle-min-ms", type=float, default=100.0,
                    help="settle phase: back-to-back steps for at least this long before timing")
    ap.add_argument("--settle-max-ms", type=float, default=1000.0,
                    help="settle phase: stop after this long even if the windows still disagree")
    ap.add_argument("--config", type=int, default=2, help="workload number (1-7); 2 is the headline")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = one split per resident workgroup slot")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="also time steps each preceded by a write of this many MiB (cold L2 / Infinity Cache); 0 = skip")
    ap.add_argument("--copy-probe-mib", type=int, default=1024, help="size of the copy-kernel reference run")
    ap.add_argument("--record-mfma", metavar="COUNTER_CSV",
                    help="no GPU: turn a rocprofv3 --pmc counter CSV (SQ_INSTS_VALU_MFMA_MOPS_BF16, "
                         "SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) of this benchmark into the per-launch "
                         "MFMA record under profiles/")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of this "
                         "benchmark into the per-launch HBM traffic record under profiles/")
    ap.add_argument("--absorb", action="store_true",
                    help="also time the query-side absorption kernel (q_nope = W_UK q_pre) on this workload")
    ap.add_argument("--no-gqa", action="store_true",
                    help="skip the GQA comparator leg (64 query / 8 KV heads, d 128, same B and lengths)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step recorded once as a HIP graph and replayed (reported beside)")
    return ap.parse_args()


def attention_kernel_name(w):
    """The split-KV attention kernel the library launches for this workload."""
    if w.dtype == "bf16" and w.NB == 4 and w.h <= 32:
        return "decode_branch_kernel"
    if w.dtype == "bf16" and w.NB == 1 and w.DL == 128:
        return "decode_shard_kernel"
    if w.dtype == "bf16" and w.NB < 4:
        return "decode_hs_kernel"
    return "decode_kernel"


def attention_kernel_design(w):
    """One line on how the attention kernel of this workload is organised."""
    return {
        "decode_branch_kernel": "one barrier-free wave per latent head, private LDS rings, one workgroup per CU",
        "decode_shard_kernel": "one barrier-free wave per split of the one latent head, private LDS rings",
        "decode_hs_kernel": "split-head: wave pairs over 256 latent channels each, whole tiles shared, one "
                            "LDS-only barrier per tile, two workgroups per CU (not MLRA-4's design)",
        "decode_kernel": "whole tiles shared by the workgroup, one LDS-only barrier per tile",
    }[attention_kernel_name(w)]


def algorithmic_bytes(inp):
    """Bytes the method must move once per step: cache rows of every cached token,
    queries, W_UV, the output, plus the int32 metadata."""
    w = inp.w
    B, h = len(inp.seqlens), w.h
    cache = inp.cache_bytes()
    q = B * h * w.token_elems * w.elem_bytes
    meta = B * 4 + (inp.block_table.numel() * 4 if inp.block_table is not None else 0)
    wuv = w.NB * h * w.DL * w.DV * 4
    out = B * h * w.DV * 4
    return dict(attention=cache + q + meta, step=cache + q + meta + wuv + out, cache=cache)


# The files the attention kernel is compiled from: a counter record taken on other sources is void.
KERNEL_SOURCES = ("long_context_decode_mlra_amd/csrc/mlra_attention.hip",
                  "long_context_decode_mlra_amd/csrc/mlra_device.h",
                  "long_context_decode_mlra_amd/csrc/mlra_internal.h", "include/mlra.h")


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()


def traffic_record(workload_name):
    """Counter-measured HBM bytes per decode-kernel launch, valid only for the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_decode_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec


def record_traffic(fetch_csv, write_csv, args):
    """Scale the decode kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same
    counters read for the copy kernel, whose bytes are known (copy_probe_mib read + written)."""
    import csv
    from mlra_workloads import WORKLOADS, make_inputs

    def means(path):
        acc = {}
        for r in csv.DictReader(open(path)):
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in acc.items()}

    f, wr = means(fetch_csv), means(write_csv)
    pick = lambda d, key: next(v for k, v in d.items() if key in k)
    copy_bytes = args.copy_probe_mib << 20
    f_scale = copy_bytes / (pick(f, "copy_kernel") * 1024)
    w_scale = copy_bytes / (pick(wr, "copy_kernel") * 1024)
    w = WORKLOADS[args.config]
    inp = make_inputs(w, seed=args.config)
    attn = lambda d: next(v for k, v in d.items() if re.search(r"decode_(branch_|hs_|shard_)?kernel", k))
    fetch = attn(f) * 1024 * f_scale
    write = attn(wr) * 1024 * w_scale
    ab = algorithmic_bytes(inp)
    rec = {"workload": w.name, "kernel": "split-KV attention kernel", "fetch_bytes_per_launch": round(fetch),
           "write_bytes_per_launch": round(write), "hbm_bytes_per_launch": round(fetch + write),
           "algorithmic_bytes_per_launch": ab["attention"],
           "traffic_over_algorithmic": round((fetch + write) / ab["attention"], 4),
           "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
           "calibration": f"copy_kernel of {copy_bytes} bytes read and written in the same runs",
           "kernel_sources": list(KERNEL_SOURCES), "kernel_source_sha256": kernel_source_hash()}
    out = os.path.join(ROOT, "profiles", f"traffic_decode_{w.name}.json")
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec))


def settle(step, min_ms, max_ms, window=20, tol=0.015):
    """Back-to-back calls of step() in windows of `window`, each ended by a device synchronisation,
    until at least min_ms have passed and the last three window means agree within tol (relative
    to the smallest), or max_ms have passed. Returns what it saw."""
    import torch
    means = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        for _ in range(window):
            step()
        torch.cuda.synchronize()
        means.append((time.perf_counter() - t0) * 1e6 / window)
        el = (time.perf_counter() - t_start) * 1e3
        last = means[-3:]
        agreed = len(means) >= 3 and max(last) - min(last) <= tol * min(last)
        if el >= max_ms or (el >= min_ms and agreed):
            break
    return {"settle_ms": round(el, 1), "windows": len(means), "window_steps": window, "agreed": agreed,
            "first_window_us": round(means[0], 2), "last_windows_us": [round(x, 2) for x in last]}


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def mfma_record(workload_name):
    """Counter-measured MFMA work per attention-kernel launch, valid only for the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"mfma_decode_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec


def record_mfma(counter_csv, args):
    """Per-launch means of the attention kernel's MFMA counters. SQ_INSTS_VALU_MFMA_MOPS_BF16 counts
    bf16 MFMA work in units of 512 FLOP; SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of every SIMD;
    GRBM_GUI_ACTIVE comes summed over the 8 XCDs (one count per XCD), so the busy fraction is
    busy / (GRBM_GUI_ACTIVE / 8 * SIMDs), the expression rocprofv3 uses for MfmaUtil."""
    import csv
    from mlra_workloads import WORKLOADS, make_inputs
    acc, spans = {}, {}
    for r in csv.DictReader(open(counter_csv)):
        k = r["Kernel_Name"]
        if not re.search(r"decode_(branch_|hs_|shard_)?kernel", k):
            continue
        acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        spans[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
        kname = re.search(r"decode_\w*kernel(<[^>]*>)?", k).group(0)
    mean = {c: sum(v) / len(v) for c, v in acc.items()}
    w = WORKLOADS[args.config]
    inp = make_inputs(w, seed=args.config)
    us = sum(spans.values()) / len(spans)
    flops = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
    algo = flop_per_head_token(w) * w.h * inp.total_tokens
    simds = 1024
    busy_frac = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (mean["GRBM_GUI_ACTIVE"] / 8 * simds)
    rec = {"workload": w.name, "kernel": kname, "launches": len(spans),
           "mfma_bf16_flop_per_launch": round(flops), "algorithmic_flop_per_launch": algo,
           "executed_over_algorithmic": round(flops / algo, 4),
           "mfma_busy_cycles_per_launch": round(mean["SQ_VALU_MFMA_BUSY_CYCLES"]),
           "grbm_gui_active_per_launch": round(mean["GRBM_GUI_ACTIVE"]),
           "mfma_busy_frac": round(busy_frac, 4),
           "avg_launch_us_under_profiler": round(us, 2),
           "executed_TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
           "executed_frac_of_bf16_peak": round(flops / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS["bf16"], 4),
           "counters": list(MFMA_COUNTERS), "simds": simds,
           "kernel_sources": list(KERNEL_SOURCES), "kernel_source_sha256": kernel_source_hash()}
    out = os.path.join(ROOT, "profiles", f"mfma_decode_{w.name}.json")
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec))


def gqa_leg(mlra, inp, args, stream, mlra_ms, shard=False):
    """The GQA decode comparator at the pages' GQA shape (64 query heads over 8 KV heads of
    128 channels) on the same batch and lengths as the MLRA workload; inputs drawn on the GPU.
    shard: one GPU's share of it under four-way tensor parallelism over heads (16 query heads
    over 2 KV heads), to set beside the one-latent-head share of MLRA-4."""
    import torch
    from mlra_workloads import GQA_WORKLOADS, make_gqa_inputs
    g = GQA_WORKLOADS["gqa_bf16_b32_hq64_hkv8_L32k"].replace(B=len(inp.seqlens), lengths=("list", tuple(inp.seqlens.tolist())))
    if shard:
        g = g.replace(Hq=g.Hq // 4, Hkv=g.Hkv // 4)
    gi = make_gqa_inputs(g, seed=args.config, device="cuda")
    sl = gi.seqlens.to("cuda")
    dec = mlra.GqaDecoder(gi.q, gi.k_cache, gi.v_cache, seqlens=sl, sm_scale=g.sm_scale, max_seqlen=gi.max_seqlen)
    for _ in range(args.warmup):
        dec(stream)
    st = settle(lambda: dec(stream), args.settle_min_ms / 2, args.settle_max_ms)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec(stream)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / args.steps
    cb = gi.cache_bytes()
    del dec, gi
    torch.cuda.empty_cache()
    return {"workload": f"gqa_bf16_b{g.B}_hq{g.Hq}_hkv{g.Hkv}_d128 (lengths of this run"
                        + ("; one GPU's share at four-way tensor parallelism)" if shard else ")"),
            "us_per_step": round(us, 2),
            "cache_bytes": cb, "cache_GBps": round(cb / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(cb / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
            "gqa_over_mlra_step_time": round(us / (mlra_ms * 1e3), 3),
            "settle": st,
            "timing": "eager launches (attention + merge), K steps between two device synchronisations, "
                      "after its own settle phase"}


def cpu_baseline(inp, target_s):
    import numpy as np  # noqa: F401
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    B = len(inp.seqlens)
    Ls = inp.seqlens.tolist()
    t0 = time.perf_counter()
    oracle.decode_inputs(inp, batch_indices=[0])
    one = time.perf_counter() - t0
    n = max(1, min(B, int(target_s / max(one, 1e-3))))
    sel = list(range(n))
    # When the whole batch fits the time budget, repeat it until the budget is spent (up to 7 runs)
    # and take the median.
    els = []
    while True:
        t0 = time.perf_counter()
        oracle.decode_inputs(inp, batch_indices=sel)
        els.append(time.perf_counter() - t0)
        if n < B or len(els) >= 7 or sum(els) + els[-1] > target_s:
            break
    runs = len(els)
    el = sorted(els)[len(els) // 2]
    tok_sample = sum(Ls[b] for b in sel)
    per_step_s = el * (sum(Ls) / max(tok_sample, 1))
    return {"value": per_step_s * 1e6, "unit": "µs/step", "cores": threads, "kind": "oracle",
            "sample": f"fp64 NumPy oracle on sequences 0..{n - 1} of {B} ({tok_sample} of {sum(Ls)} cached "
                      f"tokens; median of {runs} run(s), {el:.1f} s each), scaled by token count to the full step"}


def dpm_clocks():
    """Clock levels from the amdgpu driver's sysfs tables (pp_dpm_sclk / _mclk / _fclk: one line
    per level, the current one starred): the current and the highest level of each, per card.
    Plain file reads, so they are safe in a process that has already touched the GPU."""
    import glob
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card[0-9]*/device")):
        card = {}
        for kind in ("sclk", "mclk", "fclk"):
            try:
                lines = [l.strip() for l in open(os.path.join(dev, f"pp_dpm_{kind}")) if l.strip()]
            except OSError:
                continue
            cur = [l.split(":", 1)[1].replace("*", "").strip() for l in lines if l.endswith("*")]
            card[kind] = {"current": cur[0] if cur else None, "max": lines[-1].split(":", 1)[1].replace("*", "").strip()}
        if card:
            out[os.path.basename(os.path.dirname(dev))] = card
    return out or None


def device_info(torch):
    pr = torch.cuda.get_device_properties(0)
    return {"name": pr.name, "arch": getattr(pr, "gcnArchName", None), "compute_units": pr.multi_processor_count,
            "memory_GiB": round(pr.total_memory / 2 ** 30, 1), "dpm_clocks_after_run": dpm_clocks()}


def main():
    args = parse()
    if args.record_traffic:
        record_traffic(*args.record_traffic, args)
        return
    if args.record_mfma:
        record_mfma(args.record_mfma, args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}). One GPU's share "
              f"of MLRA-4 split over four GPUs by latent head is --config 7; the cross-GPU sum is not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_decode_mlra_amd as mlra
    from mlra_workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.config]
    print(f"bench: generating workload {w.name} (seed {args.config})", file=sys.stderr, flush=True)
    inp = make_inputs(w, seed=args.config)
    d = inp.to(dev)
    dec = mlra.Decoder(d.q_nope, d.q_rope, d.latent, d.rope, seqlens=d.seqlens, W_UV=d.W_UV,
                       sm_scale=w.sm_scale, out_scale=w.gamma, max_seqlen=inp.max_seqlen,
                       block_table=d.block_table, page_size=w.page_size, num_splits=args.num_splits)
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    print(f"bench: {args.warmup} warmup steps, settle phase, {args.steps} timed steps, splits={dec.splits}",
          file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        dec(stream)
    torch.cuda.synchronize()
    st = settle(lambda: dec(stream), args.settle_min_ms, args.settle_max_ms)
    print(f"bench: settled after {st['settle_ms']} ms: {st['last_windows_us']} us/step", file=sys.stderr,
          flush=True)

    # Headline: K back-to-back steps through the C ABI between two device synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Per-kernel durations in the same settled state: K more steps, each with HIP events on the
    # launch stream around its attention launch and its combine launches. An event between
    # launches idles the GPU for a moment, so these read slightly high.
    evs = [[ev() for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record(stream)
        dec.splitkv(stream)
        evs[k][1].record(stream)
        dec.combine(stream)
        evs[k][2].record(stream)
    torch.cuda.synchronize()
    ev_step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dk = sorted(e[0].elapsed_time(e[1]) for e in evs)
    ck = sorted(e[1].elapsed_time(e[2]) for e in evs)
    dk_mean = sum(dk) / len(dk)
    ck_mean = sum(ck) / len(ck)

    # Cold caches: before each step an untimed write of flush_mib MiB evicts L2 and the
    # Infinity Cache, then events bracket the whole step.
    cold = None
    if args.flush_mib > 0:
        junk = torch.empty(args.flush_mib << 18, dtype=torch.float32, device=dev)
        cev = [(ev(), ev()) for _ in range(args.steps)]
        for k in range(args.steps):
            junk.fill_(float(k))
            cev[k][0].record(stream)
            dec(stream)
            cev[k][1].record(stream)
        torch.cuda.synchronize()
        cold = sorted(a.elapsed_time(b) for a, b in cev)
        del junk
    graph = None
    if args.graph:
        # The same step recorded once as a HIP graph and replayed: the way a serving loop runs it.
        g = dec.capture_graph()
        gst = settle(g.replay, args.settle_min_ms / 2, args.settle_max_ms)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        graph = {"us_per_step": round((time.perf_counter() - t0) * 1e6 / args.steps, 2), "settle": gst}
        # Eight steps recorded in one graph: the runtime's gap between graph launches is paid once
        # per eight steps, as in a serving loop that records a whole model step.
        g8 = dec.capture_graph(steps=8)
        reps = max(1, args.steps // 8)
        gst8 = settle(g8.replay, args.settle_min_ms / 2, args.settle_max_ms)
        t0 = time.perf_counter()
        for _ in range(reps):
            g8.replay()
        torch.cuda.synchronize()
        graph["us_per_step_eight_steps_per_graph"] = round((time.perf_counter() - t0) * 1e6 / (8 * reps), 2)
        graph["settle_eight_steps_per_graph"] = gst8
        del g, g8
    absorb = None
    if args.absorb:
        from mlra_workloads import make_absorption_inputs
        q_pre, W_UK = make_absorption_inputs(w, seed=args.config, B=len(inp.seqlens))
        q_pre, W_UK = q_pre.to(dev), W_UK.to(dev)
        qn = torch.empty(len(inp.seqlens), w.h, w.NB, w.DL, dtype=w.torch_dtype, device=dev)
        absorber = mlra.Absorber(q_pre, W_UK, qn)
        for _ in range(3):
            absorber(stream)
        ea = [ev() for _ in range(2)]
        ea[0].record(stream)
        for _ in range(args.steps):
            absorber(stream)
        ea[1].record(stream)
        torch.cuda.synchronize()
        a_us = ea[0].elapsed_time(ea[1]) * 1e3 / args.steps
        a_bytes = q_pre.numel() * q_pre.element_size() + W_UK.numel() * 4 + qn.numel() * qn.element_size()
        absorb = {"us_per_call": round(a_us, 2), "algorithmic_bytes": a_bytes,
                  "achieved_GBps": round(a_bytes / (a_us * 1e-6) / 1e9, 1)}
    gqa = None
    if not args.no_gqa and w.dtype == "bf16" and w.page_size == 0:
        gqa = gqa_leg(mlra, inp, args, stream, ms_per_step, shard=(w.NB == 1 and w.DL == 128))

    # Copy-kernel reference (achievable bandwidth; also the calibration kernel for byte counters),
    # last, so that its load pattern does not precede the measurements above.
    copy_gbps = read_gbps = None
    if args.copy_probe_mib > 0:
        nbytes = args.copy_probe_mib << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            mlra.copy_bandwidth_probe(src, dst)
        e0, e1 = ev(), ev()
        e0.record(stream)
        for _ in range(10):
            mlra.copy_bandwidth_probe(src, dst)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2 * nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            mlra.read_bandwidth_probe(src, sink)
        e0.record(stream)
        for _ in range(10):
            mlra.read_bandwidth_probe(src, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        read_gbps = nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst

    ab = algorithmic_bytes(inp)
    tokens = inp.total_tokens
    flops = flop_per_head_token(w) * w.h * tokens + 2 * len(inp.seqlens) * w.h * w.NB * w.DL * w.DV
    us = ms_per_step * 1e3
    achieved = ab["attention"] / (dk_mean * 1e-3) / 1e9
    trec = traffic_record(w.name)
    mrec = mfma_record(w.name)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": (trec["hbm_bytes_per_launch"] if trec else None),
                "kernel": attention_kernel_name(w) + " (split-KV attention)",
                "attention_kernel_design": attention_kernel_design(w),
                "algorithmic_bytes_per_launch": ab["attention"],
                "avg_launch_us": round(dk_mean * 1e3, 2),
                "timing": "HIP events on the launch stream around each attention launch of K settled steps"}
    result = {
        "metric": METRIC, "value": round(us, 2), "unit": "µs/step", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "B": len(inp.seqlens), "h": w.h, "latent_heads": w.NB,
                   "d_latent": w.DL, "d_rope": w.DR, "d_v": w.DV, "seq_len": inp.max_seqlen,
                   "cached_tokens": tokens, "page_size": w.page_size, "num_splits": dec.splits,
                   "parallelism": "none (one GPU)"},
        "timing": "eager launches through the C ABI, K steps between two device synchronisations, "
                  "after W warm-up steps and a settle phase",
        "settle": st,
        "achieved_hbm_TBps": round(ab["step"] / (us * 1e-6) / 1e12, 3),
        "hbm_frac_step": round(ab["step"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(len(inp.seqlens) / (us * 1e-6), 1),
        "mfma_frac": round(flops / (us * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS[w.dtype], 4),
        "mfma_counters": None if mrec is None else {
            k: mrec[k] for k in ("mfma_busy_frac", "executed_frac_of_bf16_peak", "executed_over_algorithmic",
                                 "mfma_bf16_flop_per_launch", "avg_launch_us_under_profiler")},
        "kernels_us": {"attention_kernel_mean": round(dk_mean * 1e3, 2),
                       "attention_kernel_p10": round(dk[len(dk) // 10] * 1e3, 2),
                       "attention_kernel_p90": round(dk[(9 * len(dk)) // 10] * 1e3, 2),
                       "combine_mean": round(ck_mean * 1e3, 2),
                       "combine_p10": round(ck[len(ck) // 10] * 1e3, 2),
                       "combine_p90": round(ck[(9 * len(ck)) // 10] * 1e3, 2),
                       "step_with_events": round(ev_step_ms * 1e3, 2)},
        "cold_cache_us_per_step": None if cold is None else {
            "median": round(cold[len(cold) // 2] * 1e3, 2), "p10": round(cold[len(cold) // 10] * 1e3, 2),
            "p90": round(cold[(9 * len(cold)) // 10] * 1e3, 2),
            "note": f"each step after an untimed {args.flush_mib} MiB write, events around the step"},
        "graph_replay": graph,
        "algorithmic_bytes_per_step": ab["step"],
        "copy_probe_GBps": None if copy_gbps is None else round(copy_gbps, 1),
        "read_probe_GBps": None if read_gbps is None else round(read_gbps, 1),
        "roofline": roofline,
        "absorb_query": absorb,
        "gqa_comparator": gqa,
        "cpu_baseline": None,
        "device": device_info(torch),
    }
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
