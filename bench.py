#!/usr/bin/env python3
"""Benchmark of sparse MLA decode on one MI355X.

One step is one sparse_mla_decode call over the large-batch workload (T=64 tokens, H=128
heads, 2048 gathered 576-byte FP8 rows per token from a 1M-row pool), inputs resident in HBM,
rotating 8 index sets across calls so the gathered rows are not served from the caches of the
previous call.  The metric is gathered-KV bytes per second (the rows the method must move:
active columns x 576 bytes) and microseconds per call; the small-batch shapes (1, 5 and 12
tokens) are timed for microseconds per call as well.

Prints ONE JSON line.  N > 1 GPUs is not supported (one rank's share runs on one GPU).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
ROW_BYTES = 576
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_throughput_traffic.json")
CSRC = os.path.join(ROOT, "sparse_mla_attention_amd", "csrc")
# the sources of the decode kernels: the traffic counters are valid only for these exact files
DECODE_SRCS = [os.path.join(CSRC, f) for f in
               ("smla_decode.hip", "smla_decode_g64.hip", "smla_device.h", "smla_internal.h")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--one-term", action="store_true", help="time the one-term E4M3-P recipe")
    ap.add_argument("--splits", type=int, default=0, help="override the plan's split count")
    ap.add_argument("--tiles", type=int, default=0, help="override the plan's tiles per WG")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-latency", action="store_true", help="skip the small-batch timings")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    return ap.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    for f in DECODE_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


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
    key = f"splits={plan.splits},tiles={plan.tiles},one_term={int(one_term)}"
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


def graph_steps(fn, steps):
    """The timed steps: `steps` calls captured in one HIP graph (so the device runs them back to
    back without host launch gaps), replayed once untimed, then once between two HIP events on
    the stream the kernels run on, bracketed by synchronizations.  Returns ms per call."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            fn(i, s)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    cur = torch.cuda.current_stream()
    a.record(cur)
    g.replay()
    b.record(cur)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def graph_time(fn, calls_per_graph, replays):
    """Device time per call: `calls_per_graph` calls captured in one HIP graph, replayed
    `replays` times; the median over replays of (elapsed / calls_per_graph), in ms."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(calls_per_graph):  # warm the code paths on the capture stream
            fn(i, s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(calls_per_graph):
            fn(i, s)
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / calls_per_graph)
    times.sort()
    return times[len(times) // 2]


def latency_configs(smla, inputs, stream, reps=200):
    """Microseconds per call of the small-batch shapes (back-to-back launches on one stream)."""
    import numpy as np
    import torch
    res = {}
    for name in ("tiny", "verify", "dsv4"):
        p = inputs.CONFIGS[name](poison=False)
        d = {k: (torch.from_numpy(np.ascontiguousarray(v)).cuda() if isinstance(v, np.ndarray)
                 else v) for k, v in p.items()}
        T, H, _ = p["q"].shape
        W = p["indices"].shape[1]
        out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
        plan = smla.plan_for(T, H, W, p["kv_a"].shape[1])
        ws = smla.new_workspace(plan, T, H)

        def call(i, s=stream):
            smla.sparse_mla_decode(d["q"], d["kv_a"], d["indices"], d["lens"], p["bmm1"],
                                   p["bmm2"], out, lse, kv_b=d["kv_b"], split_col=p["split_col"],
                                   sinks=d["sinks"], qk_dim=p["qk_dim"], lse_log2=p["lse_log2"],
                                   plan=plan, workspace=ws, stream=s)
        for i in range(20):
            call(i)
        ms_eager = time_calls(call, reps, stream)
        ms = graph_time(call, 100, 20)
        active = int(sum(((p["indices"][t, :int(np.clip(p["lens"][t], 0, W))] >= 0).sum())
                         for t in range(T)))
        res[name] = {"us_per_call": round(ms * 1e3, 3), "us_per_call_eager": round(ms_eager * 1e3, 3),
                     "T": T, "H": H, "gathered_bytes": active * p["kv_a"].shape[1],
                     "plan": f"splits={plan.splits},tiles={plan.tiles}"}
        print(f"[bench] latency {name}: {ms * 1e3:.2f} us/call (graph), {ms_eager * 1e3:.2f} "
              f"(eager)", file=sys.stderr, flush=True)
    return res


def cpu_baseline(w, idx_host, seconds):
    """The FP64 oracle (exact mode, single thread) on (token, head) units of the same workload
    until about `seconds` have passed; reported as gathered-KV bytes per second at the same
    per-unit accounting as the GPU (each (token, head) unit stands for 1/(T*H) of a call)."""
    import numpy as np
    import oracle
    q = w["q"].cpu().numpy()
    pool = w["kv_a"].cpu().numpy()
    lens = w["lens"].cpu().numpy()
    host = dict(q=q, kv_a=pool, kv_b=None, split_col=2048, qk_dim=576, indices=idx_host,
                lens=lens, sinks=None, bmm1=w["bmm1"], bmm2=w["bmm2"])
    T, H = q.shape[0], q.shape[1]
    rng = np.random.default_rng(0)
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        units = [(int(rng.integers(T)), int(rng.integers(H))) for _ in range(4)]
        oracle.decode_exact(host, units=units)
        done += len(units)
    el = time.perf_counter() - t0
    call_bytes = T * 2048 * ROW_BYTES
    gbs = call_bytes * (done / (T * H)) / el / 1e9
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} (token, head) units of the T=64 H=128 W=2048 workload in "
                      f"{el:.1f} s, exact FP64 mode, one thread",
            "us_per_call_equiv": round(el / done * T * H * 1e6, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs one rank's share on one GPU; "
                                   "--gpus must be 1"}))
        sys.exit(2)
    import numpy as np
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
        print(json.dumps({"copy_bytes": n, "ms": ms}))
        return

    print("[bench] generating the large-batch workload", file=sys.stderr, flush=True)
    w = inputs.config_throughput_device("cuda", index_sets=8)
    T, H, W = 64, 128, 2048
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    plan = smla.plan_for(T, H, W, ROW_BYTES)
    if args.splits or args.tiles:
        plan = smla.make_plan(args.splits or plan.splits, args.tiles or plan.tiles)
    ws = smla.new_workspace(plan, T, H)
    sets = w["index_sets"]

    def call(i, s=stream):
        smla.sparse_mla_decode(w["q"], w["kv_a"], sets[i % len(sets)], w["lens"], w["bmm1"],
                               w["bmm2"], out, lse, one_term=args.one_term, plan=plan,
                               workspace=ws, stream=s)

    # the timed loop launches prepared calls (arguments converted once, as a serving loop holds
    # them), one per index set
    prepared = [smla.prepare_decode(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], out,
                                    lse, one_term=args.one_term, plan=plan, workspace=ws,
                                    stream=stream) for idx in sets]

    def timed_call(i):
        prepared[i % len(prepared)]()

    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} calls, {plan}", file=sys.stderr, flush=True)
    # the timed steps run from one HIP graph: the region over the step count is both the time
    # per step and the kernel's average launch duration; back-to-back eager launches (prepared
    # arguments) are timed too, for reference (each eager dispatch adds a gap of a few us)
    ms = graph_steps(call, args.steps)
    ms_launch = ms
    ms_eager = time_calls(timed_call, args.steps, stream)

    gathered = T * W * ROW_BYTES  # every column active: lens = W, no -1 entries
    gbs = gathered / (ms * 1e-3) / 1e9
    gbs_kernel = gathered / (ms_launch * 1e-3) / 1e9
    qbytes, outbytes = T * H * 576, T * H * 512 * 2
    roof = {"bound": "hbm", "achieved": round(gbs_kernel, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(gbs_kernel / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(plan, args.one_term),
            "kernel": f"{kernel_name(plan)} (the split merge is fused into it)",
            "us_per_launch": round(ms_launch * 1e3, 2),
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
                   "p_terms": 1 if args.one_term else 2, "plan": f"splits={plan.splits},"
                   f"tiles={plan.tiles}", "us_per_call": round(ms * 1e3, 2),
                   "us_per_call_eager": round(ms_eager * 1e3, 2),
                   "timing": "K calls captured in one HIP graph, one timed replay"},
        "roofline": roof,
    }
    if not args.no_latency:
        result["latency_small_batch"] = latency_configs(smla, inputs, stream)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, sets[0].cpu().numpy(), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
