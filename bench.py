"""Benchmark: one context-parallel rank's share of exact causal attention on
one MI355X, through the C ABI.

A step is one pass of the hot path over the rank's share: every KV block, in
the seeded arrival order, folded into the (O, LSE) state by cpattn_partial
(the LSE merge runs in the kernel's epilogue). Inputs and positions are
resident in HBM before timing starts.

Default workload: 65536 tokens zig-zag split over cp = 8, rank 1 — 8192 local
queries x 32 heads, head_dim 128, bf16, against 8 KV blocks of 8192 tokens.

Prints ONE JSON line. value = causal-effective TFLOP/s = 4 * d * (visible
(query, key, head) triples) / time. roofline: the partial-attention kernel's
algorithmic FLOPs per launch over its mean launch duration (HIP events on its
stream) against MI355X's dense bf16 MFMA peak. cpu_baseline: the fp64 oracle
on a bounded sample of the same rows, timed on the host.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "causal-effective attention TFLOPS per rank share (bf16) + % of MFMA peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X published dense MFMA peaks (bf16; fp32 matrix)


KERNEL_SOURCES = ("partial_fwd.hip", "tile_io.hpp", "device_common.hpp", "kernels.hpp")
BWD_KERNEL_SOURCES = ("partial_bwd.hip", "tile_io.hpp", "device_common.hpp", "kernels_bwd.hpp")


def kernel_source_hash(sources=KERNEL_SOURCES):
    """sha256 over a kernel's sources, in a fixed order, with comments and
    blank lines removed (so that a comment edit does not orphan a profile
    taken on the same code)."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "context_long_sequence_amd", "csrc")
    for name in sources:
        with open(os.path.join(csrc, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()


def profiled_traffic(workload, sources=KERNEL_SOURCES, key="traffic_bytes_per_launch"):
    """HBM bytes per launch (or per `key`) from a committed rocprofv3 counter
    summary under profiles/, or None when no summary was taken on the current
    kernel sources for this workload."""
    import glob
    import re
    want = kernel_source_hash(sources)
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
    for path in sorted(glob.glob(os.path.join(root, "*.md"))):
        text = open(path).read()
        src = re.search(r"^kernel_sources_sha256: ([0-9a-f]{64})$", text, re.M)
        wl = re.search(r"^workload: (\S+)$", text, re.M)
        tr = re.search(r"^%s: (\d+)$" % key, text, re.M)
        if src and wl and tr and src.group(1) == want and wl.group(1) == workload:
            return int(tr.group(1))
    return None


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def visible_pairs(q_pos, k_pos_blocks, q_start=None):
    """Visible (query, key) pairs per block (per head), by counting on sorted positions."""
    out = []
    for kp in k_pos_blocks:
        hi = np.searchsorted(kp, q_pos, side="right").astype(np.int64)
        lo = 0 if q_start is None else np.searchsorted(kp, q_start, side="left").astype(np.int64)
        out.append(int(np.sum(hi - lo)))
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="zigzag64k_cp8_h32_d128", help="one of synth.WORKLOADS (default: the 64K-token zig-zag cp 8 rank share)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain elementwise copy of MIB MiB (read once, written "
                         "once) a few times: the reference kernel that scales the HBM byte counters")
    ap.add_argument("--pipeline", action="store_true",
                    help="instead of the headline line, measure the KV arrival pipeline on the workload "
                         "(communication alone, computation alone, overlapped) for pieces of 1K..8K keys "
                         "delivered from pinned host memory and from device memory; one JSON line each")
    ap.add_argument("--fused", action="store_true",
                    help="instead of the headline line, time the step as ONE cpattn_partial_multi call over all "
                         "blocks (state kept in registers between blocks); one JSON line")
    ap.add_argument("--merge", action="store_true",
                    help="instead of the headline line, time the standalone LSE merge kernel on the workload's "
                         "(O, LSE) shape against the HBM roofline; one JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the headline line, time the gradient step on the workload: D = <dO, O> "
                         "once, then the backward of every KV block in arrival order (dQ summed over blocks, "
                         "dK and dV per block); one JSON line")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's rank share only; runs on more than one GPU are not supported "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import context_long_sequence_amd as cp
    from context_long_sequence_amd.share import share_from_workload
    from synth import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    cp.load_library()  # fails loudly if the HIP library is missing
    wl = WORKLOADS[args.workload]
    if args.merge:
        merge_bench(wl, args.steps, args.warmup)
        return
    log("workload %s: %s" % (wl.name, wl.description))
    t0 = time.time()
    share = share_from_workload(wl)
    torch.cuda.synchronize()
    log("inputs resident in HBM (%.1f s)" % (time.time() - t0))
    order = [int(b) for b in wl.arrival()]

    qs = None
    if share.cu_host is not None:
        cu = share.cu_host
        qs = cu[np.searchsorted(cu, share.q_pos_host, side="right") - 1]
    pairs = visible_pairs(share.q_pos_host, share.k_pos_host, qs)
    flops_blocks = [4.0 * wl.d * wl.hq * p for p in pairs]
    step_flops = sum(flops_blocks)

    if args.pipeline:
        pipeline_sweep(wl, share, order, step_flops)
        return
    if args.fused:
        fused_step(wl, share, order, step_flops, args.steps, args.warmup)
        return
    if args.backward:
        backward_step(wl, share, order, step_flops, args.steps, args.warmup,
                      None if args.no_cpu_baseline else args.cpu_seconds)
        return

    for _ in range(args.warmup):
        share.step(order)
    torch.cuda.synchronize()

    # timed region: K steps, events only around the whole region (on the launch stream)
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    t_wall = time.perf_counter()
    for _ in range(args.steps):
        share.step(order)
    stop.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(stop)
    # the kernel's own duration for the roofline: the same K steps again, one
    # event pair around each launch (an event between launches lengthens the
    # step a little, so this pass is not the one the step time comes from)
    n_launch = args.steps * len(order)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_launch)]
    n = 0
    for _ in range(args.steps):
        for idx, b in enumerate(order):
            ev[2 * n].record(stream)
            share.call_block(b, share.o, share.lse, accumulate=idx > 0)
            ev[2 * n + 1].record(stream)
            n += 1
    torch.cuda.synchronize()
    launch_ms = np.array([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_launch)])
    evented_ms = ev[0].elapsed_time(ev[-1]) / args.steps
    ms_per_step = total_ms / args.steps
    tflops = step_flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    kernel_flops = step_flops * args.steps / n_launch
    # the kernel's mean duration for the roofline: the timed region's time per
    # launch (launches run back to back on one stream, so this includes the
    # short gaps between them and bounds the mean duration from above); the
    # per-launch event pairs of the second pass are reported beside it (each
    # pair adds its own overhead, so they are not used)
    kernel_ms = ms_per_step / len(order)
    achieved = kernel_flops / (kernel_ms * 1e-3) / 1e12
    log("%.3f ms/step (wall %.3f ms/step), %.1f TFLOP/s, %.4f ms per launch (event pairs around every launch: "
        "mean %.4f ms, %.3f ms/step)" % (ms_per_step, t_wall * 1e3 / args.steps, tflops, kernel_ms,
                                        float(launch_ms.mean()), evented_ms))

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": wl.description,
            "name": wl.name,
            "seq_len": wl.S, "cp_size": wl.cp, "rank": wl.rank, "layout": wl.layout,
            "local_queries": wl.lq, "q_heads": wl.hq, "kv_heads": wl.hkv, "head_dim": wl.d,
            "kv_blocks": wl.n_blocks, "arrival_order": order, "global_batch": 1,
            "parallelism": "one cp%d rank share on 1 GPU" % wl.cp,
            "visible_pairs_per_head": int(sum(pairs)),
            "causal_effective_flop_per_step": step_flops,
        },
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "roofline": {
            "kernel": "partial_fwd_kernel",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": profiled_traffic(wl.name),
            "flop_per_launch": kernel_flops,
            "mean_launch_ms": round(kernel_ms, 5),
            "mean_launch_ms_from": "timed region / launches (includes the gaps between launches)",
            "launches": n_launch,
            "mean_launch_ms_event_pairs": round(float(launch_ms.mean()), 5),
            "ms_per_step_with_launch_events": round(evented_ms, 4),
        },
    }
    # context beside the headline: the same step as one multi-block call (all
    # blocks already resident, so the per-launch starts, tails and O/LSE
    # round trips of the single-block calls are gone); not the headline value
    if len(order) > 1:
        fused_ms = time_fused(share, order, args.steps, max(1, args.warmup))
        fused_tflops = step_flops / (fused_ms * 1e-3) / 1e12
        log("the same step as one multi-block call: %.3f ms/step, %.1f TFLOP/s" % (fused_ms, fused_tflops))
        out["multi_block_call"] = {"ms_per_step": round(fused_ms, 4), "value": round(fused_tflops, 2),
                                   "unit": "TFLOP/s", "pct_of_peak": round(100.0 * fused_tflops / peak, 2),
                                   "entry_point": "cpattn_partial_multi", "headline": False}
        share.step(order)  # the sample check below reads the headline path's output
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, share, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def time_fused(share, order, steps, warmup):
    """ms per step of the step as ONE cpattn_partial_multi call over all
    blocks in arrival order (one event pair around the K steps)."""
    import torch
    for _ in range(warmup):
        share.step(order, "fused")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        share.step(order, "fused")
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def fused_step(wl, share, order, step_flops, steps, warmup):
    """The step as one multi-block call (the FCP page's blocks arriving
    together): prints one JSON line in the headline's unit."""
    ms = time_fused(share, order, steps, warmup)
    tflops = step_flops / (ms * 1e-3) / 1e12
    log("fused step: %.3f ms/step, %.1f TFLOP/s" % (ms, tflops))
    print(json.dumps({"metric": METRIC + ", one multi-block call per step", "value": round(tflops, 2),
                      "unit": "TFLOP/s", "ms_per_step": round(ms, 4), "steps": steps, "warmup": warmup,
                      "higher_is_better": True, "workload": wl.name, "kv_blocks": len(order),
                      "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS[wl.dtype], 2)}), flush=True)


def merge_bench(wl, steps, warmup, reps=10):
    """The standalone merge (o_acc, lse_acc) <- merge(acc, part) on the
    workload's output shape: algorithmic bytes per launch = O_acc and O_part
    read, O_acc written, two LSEs read and one written. Timed with one event
    pair around each launch on the launch stream; one JSON line with the HBM
    roofline."""
    import torch
    from context_long_sequence_amd import cpattn_merge_lse
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(7)
    shape = (wl.lq, wl.hq, wl.d)
    o_acc = torch.randn(shape, generator=g, device="cuda").to(dt)
    o_part = torch.randn(shape, generator=g, device="cuda").to(dt)
    lse_acc = torch.rand((wl.hq, wl.lq), generator=g, device="cuda") * 10
    lse_part = torch.rand((wl.hq, wl.lq), generator=g, device="cuda") * 10
    for _ in range(warmup):
        cpattn_merge_lse(o_acc, lse_acc, o_part, lse_part)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    n = steps * reps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n)]
    for i in range(n):
        ev[2 * i].record(stream)
        cpattn_merge_lse(o_acc, lse_acc, o_part, lse_part)
        ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n)]))
    esz = 2 if dt == torch.bfloat16 else 4
    rows = wl.lq * wl.hq
    nbytes = 3 * rows * wl.d * esz + 3 * rows * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    log("merge: %.4f ms per launch, %.1f GB/s (%.1f MB per launch)" % (ms, gbs, nbytes / 1e6))
    print(json.dumps({"metric": "standalone LSE merge: HBM throughput", "value": round(gbs, 1), "unit": "GB/s",
                      "higher_is_better": True, "workload": wl.name, "launches": n, "mean_launch_ms": round(ms, 5),
                      "roofline": {"kernel": "merge_kernel", "bound": "hbm", "achieved": round(gbs, 1),
                                   "peak": 8000.0, "unit": "GB/s", "frac": round(gbs / 8000.0, 4),
                                   "traffic": None, "bytes_per_launch": nbytes}}), flush=True)


def bwd_call_bytes(q_pos, k_pos, cu, hq, hkv, d, esz, accumulate):
    """Bytes one gradient call must move when each kernel reads what it uses
    once: the key kernel reads K and V of the keys some row sees, Q and dO
    (and LSE, D) of the rows that see some key, and writes dK and dV of every
    key; the query kernel reads the same Q, dO, LSE, D, K and V and writes dQ
    of the seeing rows (adding to it: reads it too), or of every row when it
    is not accumulating. (Both kernels read Q, dO, K and V: the two-kernel
    design forms S and dP in each instead of exchanging gradients through
    atomics.)"""
    q = np.asarray(q_pos, np.int64)
    k = np.asarray(k_pos, np.int64)
    lq, lk = len(q), len(k)
    if lk == 0 or lq == 0:
        rows = keys = 0
    else:
        lo_pos = np.full(lq, np.iinfo(np.int64).min) if cu is None else \
            np.asarray(cu, np.int64)[np.searchsorted(cu, q, side="right") - 1]
        lo = np.searchsorted(k, lo_pos, side="left")
        hi = np.searchsorted(k, q, side="right")
        seeing = hi > lo
        rows = int(seeing.sum())
        cover = np.zeros(lk + 1, np.int64)          # keys inside some row's visible range
        np.add.at(cover, lo[seeing], 1)
        np.add.at(cover, hi[seeing], -1)
        keys = int((np.cumsum(cover)[:lk] > 0).sum())
    qdo = 2 * rows * hq * d * esz + 2 * rows * hq * 4
    kv = 2 * keys * hkv * d * esz
    dkv = qdo + kv + 2 * lk * hkv * d * 4
    dq = qdo + kv + (2 * rows * hq * d * 4 if accumulate else lq * hq * d * 4)
    return dkv + dq


def backward_step(wl, share, order, step_flops, steps, warmup, cpu_seconds=None):
    """The gradient step of the share, timed: one cpattn_bwd_delta call, then
    one cpattn_partial_bwd call per block (its key kernel and query kernel).
    Algorithmic work is five matrix products per visible pair (S, dP, dV, dK,
    dQ: 2.5 times the forward's two); the kernels run seven (S and dP are
    formed in both kernels). The step time comes from a region with events at
    its ends only; the mean block-call duration for the roofline from a second
    pass with an event pair around every call. Prints one JSON line."""
    import torch
    from context_long_sequence_amd.share import bits_to_device
    from context_long_sequence_amd import cpattn_bwd_delta, cpattn_partial_bwd
    share.step(order)
    dout_host = wl.dout()
    dout = bits_to_device(dout_host)
    for _ in range(max(1, warmup)):   # (the first call also allocates the gradient buffers)
        share.backward(dout, order)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        share.backward(dout, order)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    n_call = steps * len(order)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_call)]
    n = 0
    for _ in range(steps):
        cpattn_bwd_delta(share.o, dout, share.delta)
        for i, b in enumerate(order):
            ev[2 * n].record(stream)
            cpattn_partial_bwd(share.q, share.k_blocks[b], share.v_blocks[b], dout, share.q_pos,
                               share.k_pos_blocks[b], share.lse, share.delta, share.dq, share.dk[b], share.dv[b],
                               causal=share.causal, accumulate_dq=i > 0, cu_seqlens=share.cu_seqlens)
            ev[2 * n + 1].record(stream)
            n += 1
    torch.cuda.synchronize()
    call_ms = float(np.mean([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(n_call)]))
    bwd_flops = 2.5 * step_flops
    esz = 2 if wl.dtype == "bf16" else 4
    call_bytes = float(np.mean([bwd_call_bytes(share.q_pos_host, share.k_pos_host[b], share.cu_host, wl.hq, wl.hkv,
                                               wl.d, esz, i > 0) for i, b in enumerate(order)]))
    traffic = profiled_traffic(wl.name, BWD_KERNEL_SOURCES, "traffic_bytes_per_block_call")
    tflops = bwd_flops / (ms * 1e-3) / 1e12
    call_flops = bwd_flops / len(order)
    achieved = call_flops / (call_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    log("backward step: %.3f ms/step, %.1f TFLOP/s algorithmic (%.1f executed), %.3f ms per block call" %
        (ms, tflops, tflops * 1.4, call_ms))
    out = {"metric": "causal-effective backward TFLOP/s of one rank share (bf16 MFMA, fp32 gradients)",
           "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms, 4), "steps": steps,
           "warmup": warmup, "higher_is_better": True, "workload": wl.name, "kv_blocks": len(order),
           "algorithmic_flop_per_step": bwd_flops, "executed_flop_per_step": 1.4 * bwd_flops,
           "mean_block_call_ms": round(call_ms, 5),
           "pct_of_peak": round(100.0 * tflops / peak, 2),
           "roofline": {
               "kernel": "one block's backward call: bwd_dkv_kernel then bwd_dq_kernel",
               "bound": "mfma",
               "achieved": round(achieved, 2),
               "peak": peak,
               "unit": "TFLOP/s",
               "frac": round(achieved / peak, 4),
               "traffic": traffic,
               "algorithmic_bytes_per_call": round(call_bytes),
               "traffic_over_algorithmic": round(traffic / call_bytes, 3) if traffic else None,
               "flop_per_call": call_flops,
               "mean_call_ms": round(call_ms, 5),
               "calls": n_call,
           }}
    # beside it: the same step with every block's gradients in one
    # cpattn_partial_bwd_multi call (dQ summed in registers, one grid of key
    # workgroups over all blocks)
    if len(order) > 1:
        for _ in range(max(1, warmup)):
            share.backward(dout, order, mode="fused")
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            share.backward(dout, order, mode="fused")
        stop.record(stream)
        torch.cuda.synchronize()
        fms = start.elapsed_time(stop) / steps
        ftf = bwd_flops / (fms * 1e-3) / 1e12
        log("the same backward step as one multi-block call: %.3f ms/step, %.1f TFLOP/s algorithmic" % (fms, ftf))
        out["multi_block_call"] = {"ms_per_step": round(fms, 4), "value": round(ftf, 2), "unit": "TFLOP/s",
                                   "pct_of_peak": round(100.0 * ftf / peak, 2),
                                   "entry_point": "cpattn_partial_bwd_multi", "headline": False}
        share.backward(dout, order)  # the sample check below reads the per-block path's dq
        torch.cuda.synchronize()
    if cpu_seconds:
        out["cpu_baseline"] = cpu_baseline_bwd(wl, share, dout_host, cpu_seconds)
    print(json.dumps(out), flush=True)


def pipeline_sweep(wl, share, order, step_flops, chunks=(1024, 2048, 4096, 8192), slots=3, reps=3):
    """The arrival pipeline of the FCP page's overlap section: KV pieces of
    `chunk` keys copied in on one stream while the kernels fold them in on
    another, one event per piece each way. Prints one JSON line per (source,
    chunk): communication alone, computation alone, overlapped (ms per step)
    and the fraction of the shorter side the overlap hid."""
    from context_long_sequence_amd.pipeline import ArrivalPipeline
    kv_bytes = sum(2 * k.numel() * k.element_size() + p.numel() * 4
                   for k, p in zip(share.k_blocks, share.k_pos_blocks))
    for source in ("host", "device"):
        for chunk in chunks:
            pipe = ArrivalPipeline(share, chunk, n_slots=slots, source=source)
            m = pipe.measure(order, reps=reps, warmup=1)
            m.update({"metric": "KV arrival pipeline: overlapped step time", "unit": "ms",
                      "higher_is_better": False, "workload": wl.name,
                      "link_GBps": kv_bytes / (m["comm_ms"] * 1e-3) / 1e9,
                      "overlapped_TFLOPs": step_flops / (m["overlapped_ms"] * 1e-3) / 1e12})
            print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in m.items()}), flush=True)
            log("pipeline %s chunk %d: comm %.3f ms, compute %.3f ms, overlapped %.3f ms, hidden %.2f" % (
                source, chunk, m["comm_ms"], m["compute_ms"], m["overlapped_ms"], m["hidden"]))
            del pipe


def calibrate_copy(mib, reps=5):
    """y = -x over MIB MiB of float32: MIB MiB read and MIB MiB written per launch.
    Profiling this with FETCH_SIZE / WRITE_SIZE gives the counters' scale factor."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4, "launches": reps}),
          flush=True)


def oracle_block_positions(orc, wl, docs):
    """Each KV block's positions from the oracle's own closed forms (rank b's
    share; the b-th contiguous chunk, i.e. the contiguous split with
    cp = n_blocks; or the whole sequence, the contiguous split with cp = 1)."""
    if wl.block_kind == "rank_shares":
        return [orc.local_positions(wl.S, wl.cp, b, wl.layout, doc_lens=docs)[0] for b in range(wl.n_blocks)]
    if wl.block_kind == "chunks":
        return [orc.local_positions(wl.S, wl.n_blocks, b, "contiguous")[0] for b in range(wl.n_blocks)]
    return [orc.local_positions(wl.S, 1, 0, "contiguous")[0]]


def oracle_threads():
    """(threads the oracle runs on, cores in this process's affinity mask).
    The threads are the cores of the affinity mask, capped at OMP_NUM_THREADS
    when that is set (a GPU host's CPU share per GPU), else at 16."""
    cores = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return max(1, min(cores, cap)), cores


def cpu_baseline(wl, share, seconds):
    """Time the fp64 oracle on a bounded sample of the same workload's rows,
    and check the GPU output on that sample."""
    import oracle
    orc = oracle.get()
    threads, affinity_cores = oracle_threads()
    docs = wl.doc_lens()
    qp, qst = orc.local_positions(wl.S, wl.cp, wl.rank, wl.layout, doc_lens=docs)
    kps = oracle_block_positions(orc, wl, docs)
    log("cpu baseline: loading inputs on the host")
    q = wl.q()
    k = np.concatenate([wl.kv_block(b, "k") for b in range(wl.n_blocks)])
    v = np.concatenate([wl.kv_block(b, "v") for b in range(wl.n_blocks)])
    kp = np.concatenate(kps)
    qstart = qst if docs is not None else None
    # calibrate: a small sample first, then scale to ~`seconds`
    n = 32
    while True:
        rows, heads = wl.sample_pairs(n)
        t = time.perf_counter()
        o_ref, lse_ref, cnt = orc.attention(q, k, v, qp, kp, qstart, True, rows=rows, heads=heads, n_threads=threads)
        dt = time.perf_counter() - t
        if dt >= 0.5 * seconds or n >= wl.lq * wl.hq:
            break
        n = int(min(wl.lq * wl.hq, max(2 * n, n * seconds / max(dt, 1e-3))))
    flops = 4.0 * wl.d * float(np.sum(cnt))
    o = share.o.float().cpu().numpy()
    lse = share.lse.cpu().numpy()
    eo = float(np.max(np.abs(o[rows, heads] - o_ref)))
    el = float(np.max(np.abs(lse[heads, rows] - lse_ref)))
    log("cpu baseline: %d (row, head) pairs in %.1f s on %d threads; GPU vs oracle max|dO| %.2e max|dLSE| %.2e"
        % (len(rows), dt, threads, eo, el))
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cores_in_affinity_mask": affinity_cores,
        "kind": "oracle",
        "sample": "%d sampled (query row, head) pairs of this workload against all its keys, fp64 two-pass "
                  "softmax attention, %.1f s" % (len(rows), dt),
        "seconds": round(dt, 3),
        "gpu_vs_oracle_max_abs_err": {"o": eo, "lse": el},
    }


def cpu_baseline_bwd(wl, share, dout_host, seconds):
    """Time the fp64 oracle's gradients on a bounded sample of the workload's
    rows (dQ of sampled (row, head) pairs against all keys: the oracle forms
    scores, O for D, dP and dQ, four products per visible pair), and check the
    GPU's dQ on that sample."""
    import oracle
    from synth import bf16_bits_to_f32
    orc = oracle.get()
    threads, affinity_cores = oracle_threads()
    docs = wl.doc_lens()
    qp, qst = orc.local_positions(wl.S, wl.cp, wl.rank, wl.layout, doc_lens=docs)
    kps = oracle_block_positions(orc, wl, docs)
    log("cpu baseline (backward): loading inputs on the host")
    q = wl.q()
    k = np.concatenate([wl.kv_block(b, "k") for b in range(wl.n_blocks)])
    v = np.concatenate([wl.kv_block(b, "v") for b in range(wl.n_blocks)])
    dout = bf16_bits_to_f32(dout_host).astype(np.float64)
    kp = np.concatenate(kps)
    qstart = qst if docs is not None else None
    n = 16
    while True:
        rows, heads = wl.sample_pairs(n)
        t = time.perf_counter()
        dq_ref, _, _, _ = orc.attention_grad(q, k, v, dout, qp, kp, qstart, True, rows=rows, heads=heads,
                                             n_threads=threads)
        dt = time.perf_counter() - t
        if dt >= 0.5 * seconds or n >= wl.lq * wl.hq:
            break
        n = int(min(wl.lq * wl.hq, max(2 * n, n * seconds / max(dt, 1e-3))))
    kp_sorted = np.sort(kp)   # (the blocks' keys, concatenated, need not ascend)
    hi = np.searchsorted(kp_sorted, qp[rows], side="right")
    lo = 0 if qstart is None else np.searchsorted(kp_sorted, qstart[rows], side="left")
    pairs = float(np.sum(hi - lo))
    flops = 8.0 * wl.d * pairs
    dq = share.dq.cpu().numpy()[rows, heads]
    rel = float(np.max(np.abs(dq - dq_ref)) / max(np.max(np.abs(dq_ref)), 1e-30))
    log("cpu baseline (backward): %d (row, head) pairs in %.1f s on %d threads; GPU vs oracle max|ddQ|/max|dQ| %.2e"
        % (len(rows), dt, threads, rel))
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cores_in_affinity_mask": affinity_cores,
        "kind": "oracle",
        "sample": "dQ of %d sampled (query row, head) pairs of this workload against all its keys, fp64, "
                  "8 d flop per visible pair (scores, O, dP, dQ), %.1f s" % (len(rows), dt),
        "seconds": round(dt, 3),
        "gpu_vs_oracle_dq_max_rel_err": rel,
    }


if __name__ == "__main__":
    main()
