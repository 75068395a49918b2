#!/usr/bin/env python3
"""Benchmark of sparse MLA decode and the split-KV LSE merge on one MI355X.

One step is one sparse_mla_decode call over the large-batch workload (T=64 tokens, H=128
heads, 2048 gathered 576-byte FP8 rows per token from a 1M-row pool), inputs resident in HBM,
rotating 8 index sets across calls so the gathered rows are not served from the caches of the
previous call.  The metric is gathered-KV bytes per second (the rows the method must move:
active columns x 576 bytes) and microseconds per call.  Beside it: the small-batch shapes (1, 5
and 12 tokens) in microseconds per call, warm and cold; lse_merge, mla_value and
paged_mla_decode at their workload shapes in GB/s; an empty-kernel launch baseline measured the
same way; and the FP64 CPU oracle's rate on the host cores.  Before the warm-up steps the device
runs the decode untimed for --settle-ms (clock and translation-cache ramp).

Prints ONE JSON line.  N > 1 GPUs is not supported (one rank's share runs on one GPU).
"""
from __future__ import annotations

import argparse
import concurrent.futures
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
ROW_BYTES = 576
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_throughput_traffic.json")
CSRC = os.path.join(ROOT, "sparse_mla_attention_amd", "csrc")
# the sources of the decode kernels: the traffic counters are valid only for these exact files
DECODE_SRCS = [os.path.join(CSRC, f) for f in
               ("smla_decode.hip", "smla_decode_g64.hip", "smla_device.h", "smla_internal.h",
                "smla_spread.h")]
COLD_POOL_BYTES = 512 << 20    # pool copies rotated across calls for the cold small-batch runs


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=1000.0,
                    help="milliseconds of untimed decode calls run before the warm-up steps, so "
                         "that the device's clocks and translation caches reach steady state")
    ap.add_argument("--replays", type=int, default=15,
                    help="timed replays of the K-step graph; the median is reported")
    ap.add_argument("--one-term", action="store_true",
                    help="make the headline the one-term E4M3-P recipe (default: two-term)")
    ap.add_argument("--splits", type=int, default=0, help="override the plan's split count")
    ap.add_argument("--tiles", type=int, default=0, help="override the plan's tiles per WG")
    ap.add_argument("--merge", type=int, default=-1,
                    help="override the plan's merge mode (0 last-arriver, 1 spread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latency", action="store_true", help="skip the small-batch timings")
    ap.add_argument("--no-merge", action="store_true", help="skip the lse_merge leg")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="wall seconds of each CPU-oracle sample (one thread, all threads)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    return ap.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    for f in DECODE_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def plan_str(plan) -> str:
    merge = "spread" if plan.merge == 1 and plan.splits > 1 else "last"
    heads = f",heads={plan.heads}" if plan.heads else ""
    return f"splits={plan.splits},tiles={plan.tiles},merge={merge}{heads}"


def kernel_name(plan) -> str:
    return "decode_g64_kernel" if plan.tiles == 2 else "decode_kernel"


def traffic_for(plan, one_term):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel source and plan; else None."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("source_sha") != source_hash():
        return None
    key = f"{plan_str(plan)},one_term={int(one_term)}"
    e = d.get("entries", {}).get(key)
    return None if e is None else e.get("hbm_bytes_per_call")


def time_calls(fn, n, stream):
    """Back-to-back launches from Python; ms per call (includes any host launch gaps)."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(n):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n  # ms per call


def settle(fn, ms):
    """Run the decode for about `ms` milliseconds before anything is timed: measured on the
    large-batch call, the first milliseconds of work on an idle device run up to 15% slower
    than the steady state (clock and translation-cache ramp).  Returns what was run."""
    import torch
    if ms <= 0:
        return {"ms": 0.0, "calls": 0}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(50):
            fn(i, s)
    torch.cuda.synchronize()
    t0, reps = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        g.replay()
        torch.cuda.synchronize()
        reps += 1
    return {"ms": round((time.perf_counter() - t0) * 1e3, 1), "calls": 50 * reps}


def graph_replays(fn, calls, replays):
    """`calls` calls captured in one HIP graph (the device runs them back to back, no host
    launch gaps), replayed once untimed, then `replays` times, each replay alone between two
    HIP events on the stream it runs on, with synchronizations around.  Returns the ms per
    call of every timed replay."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(min(calls, 3)):  # warm the code paths on the capture stream
            fn(i, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(calls):
            fn(i, s)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    out = []
    cur = torch.cuda.current_stream()
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(cur)
        g.replay()
        b.record(cur)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / calls)
    del g
    return out


def empty_kernel_baseline(replays):
    """Launch cost of a minimal kernel (torch's fill of one element) timed as the decode is:
    100 launches in one graph, median over replays, us per launch."""
    import torch
    x = torch.empty(1, device="cuda")
    t = graph_replays(lambda i, s: x.fill_(float(i)), 100, replays)
    return {"us_per_launch": round(statistics.median(t) * 1e3, 3),
            "kernel": "one-element fill (torch)", "timing": "100 launches in one HIP graph, "
            f"median of {replays} replays"}


def small_batch(smla, inputs, replays):
    """Microseconds per call of the small-batch shapes: warm (the same pools every call) and
    cold (pool copies totalling more than 512 MB rotated across calls, so the rows come from
    HBM, not from the 256 MB MALL or the L2s), 100 calls per graph, median of the replays.
    Besides the three workloads: DeepSeek-V4 under the chunk-local recipe (SMLA_P_CHUNK_LOCAL)
    and the verify-row shape on 656-byte fp8_ds_mla rows."""
    import numpy as np
    import torch
    res = {}
    shapes = [("tiny", lambda: inputs.CONFIGS["tiny"](poison=False), False),
              ("verify", lambda: inputs.CONFIGS["verify"](poison=False), False),
              ("dsv4", lambda: inputs.CONFIGS["dsv4"](poison=False), False),
              ("dsv4_chunk_local", lambda: inputs.CONFIGS["dsv4"](poison=False), True),
              ("verify_fp8_ds_mla", lambda: inputs.random_problem(
                  21, 5, 128, 320, pool_rows=65536, row_bytes=656, poison=False), False)]
    for name, make, chunk_local in shapes:
        p = make()
        d = {k: (torch.from_numpy(np.ascontiguousarray(v)).cuda() if isinstance(v, np.ndarray)
                 else v) for k, v in p.items()}
        T, H, _ = p["q"].shape
        W = p["indices"].shape[1]
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
        plan = smla.plan_for(T, H, W, p["kv_a"].shape[1],
                             smla.SMLA_P_CHUNK_LOCAL if chunk_local else 0)
        ws = smla.new_workspace(plan, T, H)
        pool_bytes = d["kv_a"].numel() + (0 if d["kv_b"] is None else d["kv_b"].numel())
        copies = max(4, -(-COLD_POOL_BYTES // pool_bytes))
        pools = [(d["kv_a"], d["kv_b"])] + [
            (d["kv_a"].clone(), None if d["kv_b"] is None else d["kv_b"].clone())
            for _ in range(copies - 1)]

        def call(i, s, pool):
            a, b = pool(i)
            smla.sparse_mla_decode(d["q"], a, d["indices"], d["lens"], p["bmm1"], p["bmm2"],
                                   out, lse, kv_b=b, split_col=p["split_col"], sinks=d["sinks"],
                                   qk_dim=p["qk_dim"], lse_log2=p["lse_log2"], plan=plan,
                                   workspace=ws, stream=s, chunk_local=chunk_local)
        warm = graph_replays(lambda i, s: call(i, s, lambda i: pools[0]), 100, replays)
        cold = graph_replays(lambda i, s: call(i, s, lambda i: pools[i % copies]), 100, replays)
        active = int(sum(((p["indices"][t, :int(np.clip(p["lens"][t], 0, W))] >= 0).sum())
                         for t in range(T)))
        gathered = active * p["kv_a"].shape[1]
        uw, uc = statistics.median(warm) * 1e3, statistics.median(cold) * 1e3
        res[name] = {"us_per_call_warm": round(uw, 3), "us_per_call_cold": round(uc, 3),
                     "cold_pool_copies": copies,
                     "cold_pool_bytes": copies * pool_bytes, "T": T, "H": H, "W": W,
                     "gathered_bytes": gathered,
                     "gathered_gbs_cold": round(gathered / (uc * 1e-6) / 1e9, 1),
                     "plan": plan_str(plan),
                     "workgroups": T * (-(-H // (plan.heads or 32 * plan.tiles))) * plan.splits}
        log(f"latency {name}: warm {uw:.2f} us, cold {uc:.2f} us ({copies} pool copies)")
        del pools
    return res


def merge_leg(smla, inputs, replays):
    """lse_merge at its workload shape (8 sources, T=32, H=128, D=512): us per call and GB/s
    on its algorithmic bytes (partials and LSEs read, output and LSE written), cold (calls
    rotate over copies of the partials totalling more than the 256 MB MALL) and warm (every
    call reads the same partials); the rate is the cold one."""
    import numpy as np
    import torch
    m = inputs.config_merge()
    S, T, H, D = m["partials"].shape
    x = torch.from_numpy(np.ascontiguousarray(m["partials"])).cuda().view(torch.bfloat16)
    l2 = torch.from_numpy(np.ascontiguousarray(m["lse"])).cuda()
    copies = max(4, -(-COLD_POOL_BYTES // (x.numel() * 2)))
    xs = [x] + [x.clone() for _ in range(copies - 1)]
    out = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    warm = graph_replays(lambda i, s: smla.lse_merge(x, l2, out, lse, stream=s), 100, replays)
    cold = graph_replays(lambda i, s: smla.lse_merge(xs[i % copies], l2, out, lse, stream=s),
                         100, replays)
    del xs
    uw, uc = statistics.median(warm) * 1e3, statistics.median(cold) * 1e3
    nbytes = S * T * H * D * 2 + S * T * H * 4 + T * H * D * 2 + T * H * 4
    gbs = nbytes / (uc * 1e-6) / 1e9
    log(f"lse_merge: cold {uc:.2f} us ({gbs:.0f} GB/s), warm {uw:.2f} us")
    return {"workload": f"S={S} sources, T={T}, H={H}, D={D}, BF16 partials, base-2 LSE, "
                        "10% empty sources", "us_per_call": round(uc, 3),
            "us_per_call_warm": round(uw, 3), "cold_copies": copies,
            "algorithmic_bytes": nbytes, "gbs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "gbs_warm": round(nbytes / (uw * 1e-6) / 1e9, 1), "kernel": "lse_merge_kernel",
            "timing": f"100 calls in one HIP graph, median of {replays} replays; cold calls "
                      f"rotate over {copies} copies of the partials"}


def value_leg(smla, inputs, replays):
    """mla_value (split merge, W_UV and the sigmoid gate) at the merge workload's shape with
    W_UV [128, 512, 128] and gates: us per call and GB/s on its algorithmic bytes, cold (calls
    rotate over copies of the partials and W_UV totalling more than the 256 MB MALL) and warm;
    the rate is the cold one."""
    import numpy as np
    import torch
    v = inputs.value_problem(900, 8, 32, 128)
    S, T, H, D = v["partials"].shape
    x = torch.from_numpy(v["partials"]).cuda().view(torch.bfloat16)
    l2 = torch.from_numpy(v["lse"]).cuda()
    wt = torch.from_numpy(v["w_uv_t"]).cuda().view(torch.bfloat16)
    g = torch.from_numpy(v["gate"]).cuda().view(torch.bfloat16)
    tot = torch.from_numpy(v["totals"]).cuda()
    out = torch.empty((T, H * 128), dtype=torch.bfloat16, device="cuda")
    copies = max(4, -(-COLD_POOL_BYTES // (x.numel() * 2 + wt.numel() * 2)))
    sets = [(x, wt)] + [(x.clone(), wt.clone()) for _ in range(copies - 1)]

    def call(i, s, k):
        xi, wi = sets[k(i)]
        smla.mla_value(xi, l2, wi.transpose(1, 2), g, out, totals=tot, stream=s)
    warm = graph_replays(lambda i, s: call(i, s, lambda i: 0), 100, replays)
    cold = graph_replays(lambda i, s: call(i, s, lambda i: i % copies), 100, replays)
    del sets
    uw, uc = statistics.median(warm) * 1e3, statistics.median(cold) * 1e3
    nbytes = (S * T * H * D * 2 + S * T * H * 4 + H * 512 * 128 * 2 + 2 * T * H * 128 * 2 +
              T * 4)
    gbs = nbytes / (uc * 1e-6) / 1e9
    flops = 2 * T * H * 512 * 128
    log(f"mla_value: cold {uc:.2f} us ({gbs:.0f} GB/s), warm {uw:.2f} us")
    return {"workload": f"S={S} sources, T={T}, H={H}: merge + W_UV [H, 512, 128] BF16 + "
                        "sigmoid gate", "us_per_call": round(uc, 3),
            "us_per_call_warm": round(uw, 3), "cold_copies": copies,
            "algorithmic_bytes": nbytes,
            "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "gbs_warm": round(nbytes / (uw * 1e-6) / 1e9, 1),
            "tflops_bf16": round(flops / (uc * 1e-6) / 1e12, 2), "kernel": "mla_value_kernel",
            "timing": f"100 calls in one HIP graph, median of {replays} replays; cold calls "
                      f"rotate over {copies} copies of the partials and W_UV"}


def paged_leg(smla, inputs, replays):
    """paged_mla_decode (dense paged MLA decode on the same skeleton): B=32 requests, one q
    row each, H=128, 4096-token contexts in 64-row pages (75.5 MB of KV gathered per call,
    as the large sparse batch); us per call and gathered GB/s, two-term P, default plan."""
    import torch
    p = inputs.paged_problem(1030, 32, 1, 128, [4096] * 32, page_size=64, poison=False)
    q, cache = torch.from_numpy(p["q"]).cuda(), torch.from_numpy(p["cache"]).cuda()
    bt, lens = torch.from_numpy(p["block_table"]).cuda(), torch.from_numpy(p["lengths"]).cuda()
    T, H = 32, 128
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    plan = smla.paged_plan_for(32, 1, H, p["block_table"].shape[1], 64)
    ws = smla.new_workspace(plan, T, H)
    t = graph_replays(lambda i, s: smla.paged_mla_decode(q, cache, bt, lens, 1, p["bmm1"],
                                                         p["bmm2"], out, lse, plan=plan,
                                                         workspace=ws, stream=s),
                      20, replays)
    us = statistics.median(t) * 1e3
    gathered = 32 * 4096 * 576
    gbs = gathered / (us * 1e-6) / 1e9
    log(f"paged decode: {us:.2f} us, {gbs:.0f} GB/s")
    return {"workload": "B=32 requests x 1 q row, H=128, 4096-token contexts, 64-row pages",
            "plan": plan_str(plan), "us_per_call": round(us, 2),
            "gathered_bytes": gathered, "gathered_gbs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "timing": f"20 calls in one HIP graph, median of {replays} replays"}


def cpu_info():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, os.cpu_count() or 1, usable


def cpu_baseline(w, idx_host, seconds):
    """The FP64 oracle (exact mode, unmodified) on (token, head) units of the same workload,
    for about `seconds` on one thread and then on every usable host thread (its C calls release
    the interpreter lock); reported as gathered-KV bytes per second at the GPU's accounting
    (each (token, head) unit stands for 1/(T*H) of a call's gathered bytes)."""
    import numpy as np
    import oracle
    q = w["q"].cpu().numpy()
    pool = w["kv_a"].cpu().numpy()
    lens = w["lens"].cpu().numpy()
    host = dict(q=q, kv_a=pool, kv_b=None, split_col=2048, qk_dim=576, indices=idx_host,
                lens=lens, sinks=None, bmm1=w["bmm1"], bmm2=w["bmm2"])
    T, H = q.shape[0], q.shape[1]
    call_bytes = T * 2048 * ROW_BYTES
    model, nproc, usable = cpu_info()

    def run(worker_seed, deadline):
        rng = np.random.default_rng(worker_seed)
        done = 0
        while time.perf_counter() < deadline:
            units = [(int(rng.integers(T)), int(rng.integers(H))) for _ in range(2)]
            oracle.decode_exact(host, units=units)
            done += len(units)
        return done

    t0 = time.perf_counter()
    one = run(0, t0 + seconds)
    el1 = time.perf_counter() - t0
    threads = usable
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        done = sum(ex.map(lambda k: run(k + 1, t0 + seconds), range(threads)))
    el = time.perf_counter() - t0
    gbs = call_bytes * (done / (T * H)) / el / 1e9
    gbs1 = call_bytes * (one / (T * H)) / el1 / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} random (token, head) units of the T=64 H=128 W=2048 workload in "
                      f"{el:.1f} s on {threads} threads (exact FP64 mode); one thread: {one} "
                      f"units in {el1:.1f} s",
            "single_thread_value": round(gbs1, 6),
            "us_per_call_equiv": round(el / done * T * H * 1e6, 1),
            "nproc": nproc, "usable_cpus": usable, "cpu_model": model}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs one rank's share on one GPU; "
                                   "--gpus must be 1"}))
        sys.exit(2)
    import torch
    import sparse_mla_attention_amd as smla
    from sparse_mla_attention_amd import inputs

    smla.library()  # fail loudly if the HIP library is not built
    torch.cuda.init()
    stream = torch.cuda.current_stream()

    if args.copy_bytes:
        n = args.copy_bytes
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        ms = time_calls(lambda i: b.copy_(a), 5, stream)
        print(json.dumps({"copy_bytes": n, "ms": ms, "gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}))
        return

    log("generating the large-batch workload")
    w = inputs.config_throughput_device("cuda", index_sets=8)
    T, H, W = 64, 128, 2048
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    plan = smla.plan_for(T, H, W, ROW_BYTES)
    if args.splits or args.tiles or args.merge >= 0:
        plan = smla.make_plan(args.splits or plan.splits, args.tiles or plan.tiles,
                              plan.merge if args.merge < 0 else args.merge)
    ws = smla.new_workspace(plan, T, H)
    sets = w["index_sets"]

    def call(i, s=stream, one_term=args.one_term):
        smla.sparse_mla_decode(w["q"], w["kv_a"], sets[i % len(sets)], w["lens"], w["bmm1"],
                               w["bmm2"], out, lse, one_term=one_term, plan=plan,
                               workspace=ws, stream=s)

    # back-to-back eager launches with prepared arguments (converted once, as a serving loop
    # holds them) are timed too, for reference
    prepared = [smla.prepare_decode(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], out,
                                    lse, one_term=args.one_term, plan=plan, workspace=ws,
                                    stream=stream) for idx in sets]

    settled = settle(call, args.settle_ms)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    log(f"timing {args.steps} calls x {args.replays} graph replays, {plan}")
    # Each timed replay runs exactly K = --steps calls from one HIP graph between two events on
    # the stream the kernels run on; the median replay is the step time, and region / K is
    # also the kernel's average launch duration (the calls run back to back).
    reps = graph_replays(call, args.steps, args.replays)
    ms = statistics.median(reps)
    ms_eager = time_calls(lambda i: prepared[i % len(prepared)](), args.steps, stream)
    other = graph_replays(lambda i, s: call(i, s, not args.one_term), args.steps, args.replays)
    ms_other = statistics.median(other)

    gathered = T * W * ROW_BYTES  # every column active: lens = W, no -1 entries
    gbs = gathered / (ms * 1e-3) / 1e9
    qbytes, outbytes = T * H * 576, T * H * 512 * 2
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(plan, args.one_term),
            "kernel": f"{kernel_name(plan)} (the split merge is fused into it)",
            "us_per_launch": round(ms * 1e3, 2),
            "algorithmic_bytes_per_call": gathered,
            "all_algorithmic_bytes_per_call": gathered + qbytes + outbytes + T * W * 4 + T * 4 +
            T * H * 4}
    result = {
        "metric": "gathered-KV HBM GB/s of a sparse MLA decode call (with us/call)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8e4m3->f32",
        "data": "synthetic (seeded; pool N(0,1) per-tensor scaled to E4M3, 8 rotating index sets)",
        "config": {"workload": "large-batch sparse MLA decode: T=64 tokens, H=128 heads, 2048 "
                               "active 576-byte E4M3 rows per token from a 1,048,576-row pool",
                   "p_terms": 1 if args.one_term else 2, "plan": plan_str(plan),
                   "us_per_call": round(ms * 1e3, 2),
                   "us_per_call_replays": [round(x * 1e3, 2) for x in reps],
                   "us_per_call_eager": round(ms_eager * 1e3, 2),
                   f"us_per_call_{'two' if args.one_term else 'one'}_term":
                       round(ms_other * 1e3, 2),
                   "timing": f"K calls captured in one HIP graph; median of {args.replays} "
                             "timed replays",
                   "settle": settled},
        "roofline": roof,
    }
    result["launch_baseline"] = empty_kernel_baseline(args.replays)
    if not args.no_latency:
        result["latency_small_batch"] = small_batch(smla, inputs, args.replays)
    if not args.no_merge:
        result["lse_merge"] = merge_leg(smla, inputs, args.replays)
        result["mla_value"] = value_leg(smla, inputs, args.replays)
        result["paged_decode"] = paged_leg(smla, inputs, args.replays)
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(w, sets[0].cpu().numpy(), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
