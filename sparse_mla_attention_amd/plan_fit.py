"""Measure the decode plans on this GPU and fit the planner's cost model.

    python -m sparse_mla_attention_amd.plan_fit measure OUT.jsonl [H ...]   (on the GPU)
    python -m sparse_mla_attention_amd.plan_fit fit OUT.jsonl       (anywhere)

`measure` times every plan smla_decode_plan considers on a grid of shapes (T in 1..64, H in
16, 64, 128 or the head counts given, W in 128..2048: 198 shapes for the three head counts;
576-byte rows, every column active) with rows gathered from a 604 MB pool, as graph replays of
40 back-to-back calls on one stream (median of 5 replays), rotating over 8 index sets so that
consecutive calls gather different rows.  Each line appended to OUT records the shape, the
plan, the microseconds per call, and whether the plan is the one smla_decode_plan returns.

`fit` fits one linear model per kind of plan (the features are those smla_decode_plan's
predicted_us uses) by non-negative least squares on relative error, prints the coefficient
table, and reports, over the grid's shapes, how much more time the model's choices and the
library's own choices take than the best plan measured for each shape.
"""
import json
import statistics
import sys

CUS = 256  # compute units of the device the coefficients are for (MI355X)
KINDS = ["64-head, one range", "64-head, last arriver", "64-head, spread",
         "32-head, one range", "32-head, last arriver"]


def kind(tiles, splits, merge):
    if tiles == 2:
        return 0 if splits == 1 else (2 if merge == 1 else 1)
    return 3 if splits == 1 else 4


def features(T, H, W, splits, tiles, merge, heads, cus=CUS):
    """The quantities predicted_us (the C planner) weighs, in its order."""
    gw = heads or 32 * tiles
    groups = -(-H // gw)
    nwg = T * groups * splits
    waves = -(-nwg // cus)
    cpr = -(-(-(-W // splits)) // 64)
    occ = min(nwg, cus) / cus
    hr = min(gw, H) / 64.0
    f = [1.0, waves, cpr * waves, occ * cpr * waves, hr * waves, 0.0, 0.0, 0.0, 0.0, 0.0]
    if splits > 1:
        spread = merge == 1
        moved = splits if spread else splits - 1
        f[5:9] = [splits, hr * (2 if spread else splits), T * H * moved * 4096.0 / 1e6, nwg / cus]
        if spread:
            f[9] = splits / 16.0 * occ
    return f


# The coefficients smla_decode_plan carries (predicted_us in csrc/smla_api.hip), one row per
# kind of plan in KINDS' order: the last fit of this module on the MI355X grid.
LIBRARY_COEF = [
    [1.297, 3.166, 1.583, 0.241, 0.880, 0.0, 0.0, 0.0, 0.0, 0.0],
    [0.0, 4.064, 1.581, 0.060, 0.768, 2.780, 0.0, 0.026, 3.934, 0.0],
    [0.0, 6.172, 1.621, 0.196, 0.0, 0.084, 1.709, 0.086, 0.198, 4.583],
    [0.0, 6.484, 1.125, 0.164, 1.502, 0.0, 0.0, 0.0, 0.0, 0.0],
    [1.485, 7.198, 1.207, 0.171, 0.216, 0.691, 0.291, 0.0, 2.213, 0.0],
]


def library_plan(T, H, W, cus=CUS):
    """The plan smla_decode_plan returns for E4M3 rows without flags, from this module's copy of
    its model: the first candidate, in its order, with the least predicted time."""
    best, best_us = None, float("inf")
    for s, t, m, h in candidates(T, H, W, cus):
        us = 0.0
        for c, f in zip(LIBRARY_COEF[kind(t, s, m)], features(T, H, W, s, t, m, h, cus)):
            us += c * f
        if us < best_us:
            best, best_us = (s, t, m, h), us
    return best


def candidates(T, H, W, cus=CUS):
    """Every plan smla_decode_plan considers, in its order: (splits, tiles, merge, heads)."""
    out = []
    for heads in (0, 32, 16):
        gw = heads or 64
        for s, m in [(1, 0), (2, 0)] + [(s, 1) for s in range(2, 17)]:
            if -(-W // s) > 2048:
                continue
            if m == 1 and T * (-(-H // gw)) * s > cus:
                continue
            out.append((s, 2, m, heads))
    for s in (1, 2, 4, 8):
        out.append((s, 1, 0, 0))
    return out


def _graph_us(fn, calls=40, reps=5):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):
            fn(i, s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(calls):
            fn(i, s)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e3 / calls)
    return statistics.median(ts)


def measure(out_path, heads=(128, 64, 16)):
    import torch
    import sparse_mla_attention_amd as smla
    from sparse_mla_attention_amd import inputs
    w = inputs.config_throughput_device("cuda", index_sets=8)
    shapes = [(T, H, W) for H in heads for T in (1, 2, 3, 4, 5, 6, 8, 12, 16, 32, 64)
              for W in (128, 320, 512, 640, 1024, 2048)]
    with open(out_path, "a") as f:
        for T, H, W in shapes:
            q = w["q"][:T, :H]
            idx = [s[:T, :W].contiguous() for s in w["index_sets"]]
            lens = torch.full((T,), W, dtype=torch.int32, device="cuda")
            o = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
            dp = smla.plan_for(T, H, W, 576)
            default = (dp.splits, dp.tiles, dp.merge if dp.splits > 1 else 0, dp.heads)
            for key in candidates(T, H, W):
                plan = smla.make_plan(key[0], key[1], key[2], heads=key[3])
                ws = smla.new_workspace(plan, T, H)

                def call(i, s, plan=plan, ws=ws):
                    smla.sparse_mla_decode(q, w["kv_a"], idx[i % 8], lens, w["bmm1"], w["bmm2"],
                                           o, lse, plan=plan, workspace=ws, stream=s)
                us = _graph_us(call)
                f.write(json.dumps(dict(T=T, H=H, W=W, splits=key[0], tiles=key[1], merge=key[2],
                                        heads=key[3], default=key == default,
                                        us=round(us, 3))) + "\n")
            f.flush()
            print(f"measured T={T} H={H} W={W}", flush=True)


def fit(path):
    import numpy as np
    from scipy.optimize import nnls
    rows = [json.loads(l) for l in open(path)]
    coef = {}
    for k in range(len(KINDS)):
        rs = [r for r in rows if kind(r["tiles"], r["splits"], r["merge"]) == k]
        if not rs:
            continue
        A = np.array([features(r["T"], r["H"], r["W"], r["splits"], r["tiles"], r["merge"],
                               r["heads"]) for r in rs])
        y = np.array([r["us"] for r in rs])
        c, _ = nnls(A / y[:, None], np.ones_like(y))
        coef[k] = c
        err = np.abs(A @ c - y) / y
        print(f"{{{', '.join(f'{v:.3f}' for v in c)}}},  // {KINDS[k]}: {len(rs)} timings, "
              f"relative error mean {err.mean():.3f}, max {err.max():.3f}")
    by = {}
    for r in rows:
        by.setdefault((r["T"], r["H"], r["W"]), {})[(r["splits"], r["tiles"], r["merge"],
                                                     r["heads"])] = r
    best_sum = model_sum = lib_sum = 0.0
    for (T, H, W), plans in sorted(by.items()):
        best = min(r["us"] for r in plans.values())
        pick = min(plans, key=lambda p: (float(np.dot(coef[kind(p[1], p[0], p[2])],
                                                      features(T, H, W, p[0], p[1], p[2], p[3])))))
        lib = [r["us"] for r in plans.values() if r["default"]]
        best_sum += best
        model_sum += plans[pick]["us"]
        lib_sum += lib[0] if lib else float("nan")
    print(f"{len(by)} shapes: best plans {best_sum:.1f} us in sum; this fit's choices "
          f"{model_sum:.1f} (+{100 * (model_sum / best_sum - 1):.1f}%); the library's planner "
          f"{lib_sum:.1f} (+{100 * (lib_sum / best_sum - 1):.1f}%)")


if __name__ == "__main__":
    if len(sys.argv) < 3 or sys.argv[1] not in ("measure", "fit"):
        sys.exit(__doc__)
    if sys.argv[1] == "measure":
        measure(sys.argv[2], tuple(int(h) for h in sys.argv[3:]) or (128, 64, 16))
    else:
        fit(sys.argv[2])
