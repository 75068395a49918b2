"""The default plans (smla_decode_plan's cost model) on a spread of shapes: each is accepted by
the decode and exact against the FP64 oracle, and together they exercise every kind of plan the
planner can return (one range, the last-arriver and spread merges, 16- and 32-head groups, the
32-head kernel)."""
import numpy as np
import pytest

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, EXACT_REL_L2, LSE_ABS, DeviceProblem,
                          check_empty_rows_exact, log, lse_err, rel_l2)

pytestmark = pytest.mark.gpu

# (T, H, W, extra generator options)
SHAPES = [
    (1, 128, 1500, {}),
    (1, 16, 2048, dict(sinks=True)),
    (2, 64, 900, dict(neg_frac=0.1)),
    (3, 128, 700, dict(lens=[700, 0, 333])),
    (5, 128, 320, {}),
    (3, 128, 1024, dict(neg_frac=0.05)),
    (4, 128, 128, {}),
    (2, 48, 520, dict(sinks=True, lens=[520, 77])),
    (12, 16, 640, dict(row_bytes=512, two_pools=True, split_col=128, rows_b=3000)),
    (32, 128, 512, {}),
    (64, 64, 1024, dict(lens=600)),
    (40, 128, 1024, dict(lens=700)),
]


@pytest.fixture(scope="module")
def chosen():
    return {}


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"T{s[0]}_H{s[1]}_W{s[2]}")
def test_default_plan_exact(shape, chosen):
    T, H, W, kw = shape
    kw = dict(kw)
    if "lens" in kw and not np.isscalar(kw["lens"]):
        kw["lens"] = np.array(kw["lens"])
    p = inputs.random_problem(1000 + T + H + W, T, H, W, pool_rows=4000, **kw)
    d = DeviceProblem(p)
    out, lse, plan = d.run()
    chosen[(T, H, W)] = plan
    check_empty_rows_exact(d.out, d.lse, p)
    ref, ref_lse = oracle.decode_exact(p)
    r, m, le = rel_l2(out, ref), float(np.abs(out - ref).max()), lse_err(lse, ref_lse)
    log(f"T={T} H={H} W={W} default {plan}: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
    assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS


def test_default_plans_cover_every_kind(chosen):
    """Runs after the shapes above (same module): their default plans between them take every
    kind of plan the planner returns."""
    if len(chosen) < len(SHAPES):
        pytest.skip("needs every shape of this module to have run")
    plans = list(chosen.values())
    kinds = {
        "one range": any(p.splits == 1 for p in plans),
        "64-head last arriver": any(p.tiles == 2 and p.splits == 2 and
                                    p.merge == smla.SMLA_MERGE_LAST for p in plans),
        "spread": any(p.splits > 1 and p.merge == smla.SMLA_MERGE_SPREAD for p in plans),
        "16-head groups": any(p.heads == 16 for p in plans),
        "32-head groups": any(p.heads == 32 for p in plans),
        "32-head kernel": any(p.tiles == 1 for p in plans),
    }
    log("default plans: " + ", ".join(f"{k}: {v}" for k, v in chosen.items()))
    missing = [k for k, v in kinds.items() if not v]
    assert not missing, f"no shape took {missing}"


def test_library_plan_matches_the_fitted_model():
    """smla_decode_plan picks, over a grid of shapes, the plan plan_fit's copy of its model
    picks (same features, coefficients, candidate order and tie rule), for this device's
    compute-unit count."""
    import torch
    from sparse_mla_attention_amd import plan_fit
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    diff = []
    n = 0
    for T in (1, 2, 3, 5, 7, 12, 16, 33, 64, 100):
        for H in (16, 48, 64, 128):
            for W in (1, 64, 100, 320, 640, 1000, 2048, 3000):
                p = smla.plan_for(T, H, W, 576)
                got = (p.splits, p.tiles, p.merge if p.splits > 1 else 0, p.heads)
                want = plan_fit.library_plan(T, H, W, cus)
                n += 1
                if got != want:
                    diff.append(((T, H, W), got, want))
    log(f"{n} shapes, {len(diff)} differ")
    assert not diff, diff[:5]
