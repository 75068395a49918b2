"""SMLA_P_CHUNK_LOCAL, the chunk-local recipe (the sparse_mla_cute page, "How."): one key range
per 128-column window, P = E4M3(256 x 2^(s2 - m_k)) at the window's own maximum, the windows
merged as split partials.  Parity with the oracle's chunk-local mode (same quantization points)
and with exact mode (the recipe's own distance), bit-identical results across head groupings and
merge modes, the DeepSeek-V4 workload, and the host's plan checks."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, LSE_ABS, MIMIC_MAX_ABS, MIMIC_REL_L2,
                          ONE_TERM_EXACT_REL_L2, DeviceProblem, check_empty_rows_exact, flip_stats,
                          log, lse_err, mimic_max_abs_ok, rel_l2)

pytestmark = pytest.mark.gpu

SPREAD, LAST = smla.SMLA_MERGE_SPREAD, smla.SMLA_MERGE_LAST

CASES = {
    # five windows (the last one partial), ragged and empty rows, masked columns, sinks
    "H64_ragged_empty": dict(seed=900, T=3, H=64, W=300, lens=[300, 129, 0], neg_frac=0.1,
                             sinks=True),
    # one window, a partial one-chunk row
    "H128_one_window": dict(seed=901, T=2, H=128, W=128, lens=[128, 77]),
    # 576-byte rows with a 512-byte score, a padded head group, five windows
    "H48_qk512": dict(seed=902, T=2, H=48, W=520, qk_dim=512, lens=[520, 256], sinks=True),
    # sixteen windows: the spread merge applies
    "T1_W2048": dict(seed=903, T=1, H=16, W=2048, pool_rows=8000, sinks=True),
    # per-tensor scaled rows (amax 448): large scores
    "H64_amax": dict(seed=904, T=2, H=64, W=400, kv_scale_to_amax=True),
    # 512-byte rows in two pools (the split column inside the first window)
    "H16_two_pools": dict(seed=905, T=4, H=16, W=640, row_bytes=512, two_pools=True,
                          split_col=128, rows_b=5000, sinks=True, lens=[640, 500, 129, 1]),
}


def _problem(name):
    kw = dict(CASES[name])
    seed, T, H, W = kw.pop("seed"), kw.pop("T"), kw.pop("H"), kw.pop("W")
    if "lens" in kw:
        kw["lens"] = np.array(kw["lens"])
    kw.setdefault("pool_rows", 3000)
    return inputs.random_problem(seed, T, H, W, **kw)


def _check_parity(p, out, lse, what):
    lse_log2 = bool(p.get("lse_log2", False))
    ref, ref_lse = oracle.decode_chunk_local(p, lse_log2=lse_log2)
    ex, ex_lse = oracle.decode_exact(p, lse_log2=lse_log2)
    if lse_log2:
        ref_lse, ex_lse, lse = ref_lse * np.log(2.0), ex_lse * np.log(2.0), lse * np.log(2.0)
    r, le = rel_l2(out, ref), lse_err(lse, ref_lse)
    re, me, lee = rel_l2(out, ex), float(np.abs(out - ex).max()), lse_err(lse, ex_lse)
    log(f"{what}: vs recipe rel_l2={r:.3e} ({flip_stats(out, ref, MIMIC_MAX_ABS)}) lse={le:.3e}; "
        f"vs exact rel_l2={re:.3e} max_abs={me:.3e} lse={lee:.3e}")
    assert r <= MIMIC_REL_L2 and le <= LSE_ABS
    assert mimic_max_abs_ok(out, ref, MIMIC_MAX_ABS, EXACT_MAX_ABS)
    assert re <= ONE_TERM_EXACT_REL_L2 and me <= EXACT_MAX_ABS and lee <= LSE_ABS


def _plans(T, H, W):
    """The default chunk-local plan and the other head groupings and merges of its split
    count."""
    s = -(-W // 128)
    plans = [smla.plan_for(T, H, W, 576, smla.SMLA_P_CHUNK_LOCAL)]
    for heads in (0, 16, 32):
        plans.append(smla.make_plan(s, 2, LAST, heads=heads))
        if 2 <= s <= 16 and T * -(-H // (heads or 64)) * s <= 256:
            plans.append(smla.make_plan(s, 2, SPREAD, heads=heads))
    return plans


@pytest.mark.parametrize("name", list(CASES))
def test_chunk_local_parity_and_plan_invariance(name):
    p = _problem(name)
    d = DeviceProblem(p)
    T, H, _ = p["q"].shape
    W = p["indices"].shape[1]
    ref_bits = None
    for plan in _plans(T, H, W):
        out, lse, use = d.run(plan=plan, chunk_local=True)
        check_empty_rows_exact(d.out, d.lse, p)
        bits = (d.out.view(torch.int16).cpu().clone(), d.lse.view(torch.int32).cpu().clone())
        if ref_bits is None:
            _check_parity(p, out, lse, f"{name} {use}")
            ref_bits = bits
        else:
            # every grouping and merge sums the same windows in the same order
            assert torch.equal(bits[0], ref_bits[0]), f"{use}: output differs from the default"
            assert torch.equal(bits[1], ref_bits[1]), f"{use}: LSE differs from the default"


def test_chunk_local_dsv4_workload():
    """The DeepSeek-V4 workload (12 tokens, 16 heads, 640 columns in two pools, sinks) under the
    chunk-local recipe: five windows, as the page's five CTAs per token."""
    p = inputs.CONFIGS["dsv4"]()
    d = DeviceProblem(p)
    out, lse, plan = d.run(chunk_local=True)
    assert plan.splits == 5 and plan.tiles == 2
    check_empty_rows_exact(d.out, d.lse, p)
    _check_parity(p, out, lse, f"dsv4 {plan}")


def test_chunk_local_many_windows_under_the_last_arriver_merge():
    """More than 16 windows (3,000 columns: 24 ranges) take the last-arriver merge."""
    p = inputs.random_problem(906, 2, 16, 3000, pool_rows=8000, lens=np.array([3000, 1900]),
                              sinks=True, neg_frac=0.05)
    d = DeviceProblem(p)
    out, lse, plan = d.run(chunk_local=True)
    assert plan.splits == 24 and plan.merge == LAST
    check_empty_rows_exact(d.out, d.lse, p)
    _check_parity(p, out, lse, f"W=3000 {plan}")


def test_chunk_local_is_deterministic():
    p = _problem("T1_W2048")
    d = DeviceProblem(p)
    d.run(chunk_local=True)
    first = d.out.view(torch.int16).cpu().clone()
    for _ in range(3):
        d.run(chunk_local=True)
        assert torch.equal(d.out.view(torch.int16).cpu(), first)


def test_chunk_local_plan_and_flags_are_checked():
    p = _problem("H64_ragged_empty")
    d = DeviceProblem(p)
    for plan in (smla.make_plan(3, 1), smla.make_plan(2, 2), smla.make_plan(4, 2, SPREAD)):
        with pytest.raises(smla.SmlaError) as e:
            d.run(plan=plan, chunk_local=True)
        assert e.value.status == smla.SMLA_EUNSUPPORTED
    plan = smla.plan_for(3, 64, 300, 576, smla.SMLA_P_CHUNK_LOCAL)
    assert plan.splits == 3 and plan.tiles == 2
    # the flag implies one term: passing SMLA_P_ONE_TERM as well changes nothing
    d.run(plan=plan, chunk_local=True)
    a = d.out.view(torch.int16).cpu().clone()
    d.run(plan=plan, chunk_local=True, one_term=True)
    assert torch.equal(d.out.view(torch.int16).cpu(), a)
