"""Parity on the five workload shapes (full outputs where the oracle finishes in seconds,
sampled (token, head) units at the large-batch size) and of lse_merge."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, EXACT_REL_L2, LSE_ABS, MIMIC_MAX_ABS, MIMIC_REL_L2,
                          DeviceProblem, bf16_to_f64, check_empty_rows_exact, dev, flip_stats,
                          log, lse_err, mimic_max_abs_ok, rel_l2)

pytestmark = pytest.mark.gpu

LN2 = np.log(2.0)


@pytest.mark.parametrize("name", ["tiny", "verify", "dsv4"])
def test_config_exact_parity(name):
    p = inputs.CONFIGS[name]()  # pools poisoned: unused rows are E4M3 NaN
    log(f"config {p['name']}")
    d = DeviceProblem(p)
    out, lse, plan = d.run()
    check_empty_rows_exact(d.out, d.lse, p)
    ref, ref_lse = oracle.decode_exact(p, lse_log2=p["lse_log2"])
    if p["lse_log2"]:
        ref_lse, lse = ref_lse * LN2, lse * LN2
    r, m, le = rel_l2(out, ref), float(np.abs(out - ref).max()), lse_err(lse, ref_lse)
    log(f"  {plan}: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
    assert np.all(np.isfinite(out))
    assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS


@pytest.mark.parametrize("name", ["tiny", "verify", "dsv4"])
def test_config_one_term_matches_recipe_and_exact_gate(name):
    """The one-term path (the attn_sparse page's E4M3-P recipe) against mimic mode of the same
    plan, and against the exact formula at the gate the method is held to on these workloads:
    max-abs <= 3e-2 and LSE within 2e-3 (its relative L2 is the recipe's own, ~2e-2)."""
    p = inputs.CONFIGS[name]()
    d = DeviceProblem(p)
    out, lse, plan = d.run(one_term=True)
    check_empty_rows_exact(d.out, d.lse, p)
    ref, ref_lse = oracle.decode_mimic(p, plan.splits, plan.chunk, terms=1,
                                       lse_log2=p["lse_log2"])
    ex, ex_lse = oracle.decode_exact(p, lse_log2=p["lse_log2"])
    if p["lse_log2"]:
        ref_lse, ex_lse, lse = ref_lse * LN2, ex_lse * LN2, lse * LN2
    r, m, le = rel_l2(out, ref), float(np.abs(out - ref).max()), lse_err(lse, ref_lse)
    re, me, lee = rel_l2(out, ex), float(np.abs(out - ex).max()), lse_err(lse, ex_lse)
    log(f"  {p['name']} one-term {plan}: vs recipe rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e} "
        f"({flip_stats(out, ref, MIMIC_MAX_ABS)}); vs exact rel_l2={re:.3e} max_abs={me:.3e} "
        f"lse={lee:.3e}")
    assert r <= MIMIC_REL_L2 and le <= LSE_ABS
    assert mimic_max_abs_ok(out, ref, MIMIC_MAX_ABS, EXACT_MAX_ABS)
    assert me <= EXACT_MAX_ABS and lee <= LSE_ABS


def _throughput_units(T=64, H=128, count=48, seed=7):
    rng = np.random.default_rng(seed)
    units = {(0, 0), (T - 1, H - 1), (0, H - 1), (T - 1, 0), (31, 64), (32, 63)}
    while len(units) < count:
        units.add((int(rng.integers(T)), int(rng.integers(H))))
    return sorted(units)


def test_throughput_config_sampled_parity():
    """T=64, H=128, 2048 columns per token over a 1M-row pool, in the launch configuration the
    benchmark times (its default plan), checked on sampled (token, head) units."""
    log("generating the throughput workload on the device")
    w = inputs.config_throughput_device("cuda", index_sets=1)
    T, H, W = 64, 128, 2048
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    plan = smla.plan_for(T, H, W, 576)
    ws = smla.new_workspace(plan, T, H)
    idx = w["index_sets"][0]
    for one_term in (False, True):
        smla.sparse_mla_decode(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], out, lse,
                               one_term=one_term, plan=plan, workspace=ws)
        torch.cuda.synchronize()
        units = _throughput_units()
        host = dict(q=w["q"].cpu().numpy(), kv_a=w["kv_a"].cpu().numpy(), kv_b=None,
                    split_col=W, qk_dim=576, indices=idx.cpu().numpy(),
                    lens=w["lens"].cpu().numpy(), sinks=None, bmm1=w["bmm1"], bmm2=w["bmm2"])
        got = np.stack([bf16_to_f64(out[t, h]) for t, h in units])
        got_lse = np.array([float(lse[t, h]) for t, h in units])
        ex, ex_lse = oracle.decode_exact(host, units=units)
        re, me, lee = rel_l2(got, ex), float(np.abs(got - ex).max()), lse_err(got_lse, ex_lse)
        assert np.all(np.isfinite(bf16_to_f64(out)))
        if one_term:
            ref, ref_lse = oracle.decode_mimic(host, plan.splits, plan.chunk, terms=1,
                                               units=units)
            r, m, le = rel_l2(got, ref), float(np.abs(got - ref).max()), lse_err(got_lse, ref_lse)
            log(f"  throughput {plan} one-term: vs recipe rel_l2={r:.3e} max_abs={m:.3e} "
                f"lse={le:.3e} ({flip_stats(got, ref, MIMIC_MAX_ABS)}); vs exact "
                f"rel_l2={re:.3e} max_abs={me:.3e} lse={lee:.3e} over {len(units)} units")
            assert r <= MIMIC_REL_L2 and le <= LSE_ABS
            assert mimic_max_abs_ok(got, ref, MIMIC_MAX_ABS, EXACT_MAX_ABS)
            assert me <= EXACT_MAX_ABS and lee <= LSE_ABS
        else:
            log(f"  throughput {plan}: vs exact rel_l2={re:.3e} max_abs={me:.3e} "
                f"lse={lee:.3e} over {len(units)} units")
            assert re <= EXACT_REL_L2 and me <= EXACT_MAX_ABS and lee <= LSE_ABS
        del host


def test_throughput_config_full_parity():
    """Every (token, head) of the large-batch launch the benchmark times (default plan,
    two-term P) against the exact oracle: 8192 units of 2048 columns, computed by the C oracle
    on host threads (its calls release the GIL), under the gate the method is held to."""
    import concurrent.futures
    import os
    log("generating the throughput workload on the device")
    w = inputs.config_throughput_device("cuda", index_sets=1)
    T, H, W = 64, 128, 2048
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    plan = smla.plan_for(T, H, W, 576)
    idx = w["index_sets"][0]
    smla.sparse_mla_decode(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], out, lse,
                           plan=plan, workspace=smla.new_workspace(plan, T, H))
    torch.cuda.synchronize()
    host = dict(q=w["q"].cpu().numpy(), kv_a=w["kv_a"].cpu().numpy(), kv_b=None,
                split_col=W, qk_dim=576, indices=idx.cpu().numpy(),
                lens=w["lens"].cpu().numpy(), sinks=None, bmm1=w["bmm1"], bmm2=w["bmm2"])
    units = [(t, h) for t in range(T) for h in range(H)]
    workers = max(1, min(16, os.cpu_count() or 1))
    parts = [units[i::workers] for i in range(workers)]
    log(f"  exact oracle over {len(units)} units on {workers} host threads")
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda u: oracle.decode_exact(host, units=u), parts))
    ref = np.empty((T * H, 512))
    ref_lse = np.empty(T * H)
    for i, (o, l) in enumerate(res):
        ref[i::workers] = o
        ref_lse[i::workers] = l
    got = bf16_to_f64(out).reshape(T * H, 512)
    got_lse = lse.cpu().numpy().astype(np.float64).reshape(-1)
    r, m, le = rel_l2(got, ref), float(np.abs(got - ref).max()), lse_err(got_lse, ref_lse)
    log(f"  throughput {plan}: all units rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
    assert np.all(np.isfinite(got))
    assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS


# ---------------------------------------------------------------------------------------------
# lse_merge
# ---------------------------------------------------------------------------------------------

def _run_merge(m, lse_log2=False):
    x = dev(m["partials"]).view(torch.bfloat16)
    l2 = dev(m["lse"])
    S, T, H, D = m["partials"].shape
    out = torch.full((T, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    smla.lse_merge(x, l2, out, lse, lse_log2=lse_log2)
    torch.cuda.synchronize()
    return out, lse


def _check_merge(m, lse_log2=False, label=""):
    out, lse = _run_merge(m, lse_log2)
    ref, ref_lse = oracle.lse_merge(m["partials"], m["lse"], lse_log2=lse_log2)
    got = bf16_to_f64(out)
    assert np.all(np.isfinite(got)), "NaN from an empty source leaked"
    r, mx = rel_l2(got, ref), float(np.abs(got - ref).max())
    gl = lse.cpu().numpy().astype(np.float64)
    le = lse_err(gl, ref_lse)
    log(f"  merge {label}: rel_l2={r:.3e} max_abs={mx:.3e} lse={le:.3e}")
    # inputs and output are BF16: the only error is the output rounding (2^-9 relative) and
    # FP32 sums of at most 64 terms
    assert r <= 4e-3 and mx <= 2e-2 and le <= 1e-5 * max(1.0, np.abs(ref_lse[np.isfinite(ref_lse)]).max())
    none = ~np.isfinite(m["lse"]).any(axis=0)
    if none.any():
        bits = out.view(torch.int16).cpu().numpy()[none]
        assert np.all(bits == 0), "empty units must be +0.0"
        assert np.all(gl[none] == -np.inf)


def test_merge_config():
    m = inputs.config_merge()
    _check_merge(m, label=m["name"])


@pytest.mark.parametrize("S,T,H,D", [(1, 3, 5, 8), (2, 4, 16, 512), (5, 7, 3, 64), (17, 2, 8, 128),
                                     (64, 2, 2, 16)])
def test_merge_shapes(S, T, H, D):
    m = inputs.random_merge(500 + S, S, T, H, D, empty_frac=0.3, nan_lse=True)
    for lse_log2 in (False, True):
        _check_merge(m, lse_log2, label=f"S={S} T={T} H={H} D={D} log2={lse_log2}")


def test_merge_rejects_bad_sizes():
    m = inputs.random_merge(600, 2, 2, 2, 16)
    x = dev(m["partials"]).view(torch.bfloat16)
    out = torch.empty((2, 2, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(smla.SmlaError) as e:
        smla.lse_merge(x[..., :12], dev(m["lse"]), out[..., :12])
    assert e.value.status in (smla.SMLA_EUNSUPPORTED, smla.SMLA_EINVAL)
