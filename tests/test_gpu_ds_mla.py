"""656-byte fp8_ds_mla rows (E4M3 latent with an FP32 scale per 128 elements, BF16 rope): the
64-head kernel scales each latent block's QK product per key, takes the rope product in BF16 and
the P.V product in BF16 (V x scale rounded to BF16, P's E4M3 terms exact).  Parity with the
oracle (exact mode for two-term P, the recipe for one-term P and for the chunk-local recipe),
bit-identical results across head groupings and merges, and the host's checks."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, EXACT_REL_L2, LSE_ABS, MIMIC_MAX_ABS, MIMIC_REL_L2,
                          ONE_TERM_EXACT_REL_L2, DeviceProblem, bf16_to_f64, check_empty_rows_exact,
                          flip_stats, log, lse_err, mimic_max_abs_ok, rel_l2)

pytestmark = pytest.mark.gpu

SPREAD, LAST = smla.SMLA_MERGE_SPREAD, smla.SMLA_MERGE_LAST

CASES = {
    "H64_ragged_empty": dict(seed=920, T=3, H=64, W=300, lens=[300, 129, 0], neg_frac=0.1,
                             sinks=True),
    "verify_shape": dict(seed=921, T=5, H=128, W=320),
    "dsv4_shape_two_pools": dict(seed=922, T=12, H=16, W=640, two_pools=True, split_col=128,
                                 rows_b=6000, sinks=True, neg_frac=0.1),
    "H48_padded_long": dict(seed=923, T=2, H=48, W=1500, lens=[1500, 700], pool_rows=6000),
    "H128_scaled_values": dict(seed=924, T=2, H=128, W=200, value_scale=3.0, lens=[200, 64]),
}


def _problem(name):
    kw = dict(CASES[name])
    seed, T, H, W = kw.pop("seed"), kw.pop("T"), kw.pop("H"), kw.pop("W")
    if "lens" in kw:
        kw["lens"] = np.array(kw["lens"])
    kw.setdefault("pool_rows", 3000)
    return inputs.random_problem(seed, T, H, W, row_bytes=656, **kw)


def _bits(d):
    return d.out.view(torch.int16).cpu().clone(), d.lse.view(torch.int32).cpu().clone()


def _vs(p, out, lse, ref, ref_lse, what):
    r, m, le = rel_l2(out, ref), float(np.abs(out - ref).max()), lse_err(lse, ref_lse)
    log(f"{what}: rel_l2={r:.3e} max_abs={m:.3e} ({flip_stats(out, ref, MIMIC_MAX_ABS)}) "
        f"lse={le:.3e}")
    return r, m, le


@pytest.mark.parametrize("name", list(CASES))
def test_ds_mla_two_term_exact_and_plan_invariance(name):
    p = _problem(name)
    d = DeviceProblem(p)
    T, H, _ = p["q"].shape
    W = p["indices"].shape[1]
    ex, ex_lse = oracle.decode_exact(p)
    plans = [smla.plan_for(T, H, W, 656), smla.make_plan(1, 2), smla.make_plan(2, 2),
             smla.make_plan(3, 2), smla.make_plan(2, 2, heads=16)]
    if T * -(-H // 32) * 4 <= 256:
        plans.append(smla.make_plan(4, 2, SPREAD, heads=32))
    refs = {}
    for plan in plans:
        out, lse, use = d.run(plan=plan)
        check_empty_rows_exact(d.out, d.lse, p)
        r, m, le = _vs(p, out, lse, ex, ex_lse, f"{name} {use} two-term vs exact")
        # max-abs in units of the data's scale, as for E4M3 rows
        assert r <= EXACT_REL_L2 and le <= LSE_ABS
        assert m <= EXACT_MAX_ABS * max(1.0, p.get("value_scale", 1.0))
        # the same split count gives the same bits whatever the head grouping and merge
        key = use.splits
        if key in refs:
            assert torch.equal(_bits(d)[0], refs[key][0]) and torch.equal(_bits(d)[1],
                                                                          refs[key][1]), use
        else:
            refs[key] = _bits(d)


@pytest.mark.parametrize("name", ["H64_ragged_empty", "dsv4_shape_two_pools", "H48_padded_long"])
def test_ds_mla_one_term_matches_the_recipe(name):
    p = _problem(name)
    d = DeviceProblem(p)
    for plan in (smla.make_plan(1, 2), smla.make_plan(3, 2)):
        out, lse, use = d.run(plan=plan, one_term=True)
        check_empty_rows_exact(d.out, d.lse, p)
        ref, ref_lse = oracle.decode_mimic(p, use.splits, use.chunk, terms=1)
        r, m, le = _vs(p, out, lse, ref, ref_lse, f"{name} {use} one-term vs recipe")
        assert r <= MIMIC_REL_L2 and le <= LSE_ABS
        assert mimic_max_abs_ok(out, ref, MIMIC_MAX_ABS, EXACT_MAX_ABS)
        ex, ex_lse = oracle.decode_exact(p)
        r, m, le = _vs(p, out, lse, ex, ex_lse, f"{name} {use} one-term vs exact")
        assert r <= ONE_TERM_EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS


@pytest.mark.parametrize("name", ["H64_ragged_empty", "dsv4_shape_two_pools"])
def test_ds_mla_chunk_local(name):
    p = _problem(name)
    d = DeviceProblem(p)
    out, lse, plan = d.run(chunk_local=True)
    check_empty_rows_exact(d.out, d.lse, p)
    ref, ref_lse = oracle.decode_chunk_local(p)
    r, m, le = _vs(p, out, lse, ref, ref_lse, f"{name} {plan} chunk-local vs recipe")
    assert r <= MIMIC_REL_L2 and le <= LSE_ABS
    assert mimic_max_abs_ok(out, ref, MIMIC_MAX_ABS, EXACT_MAX_ABS)


def test_ds_mla_checks():
    p = _problem("H64_ragged_empty")
    d = DeviceProblem(p)
    with pytest.raises(smla.SmlaError) as e:
        d.run(plan=smla.make_plan(2, 1))        # the 32-head kernel reads E4M3 rows only
    assert e.value.status == smla.SMLA_EUNSUPPORTED
    plan = smla.plan_for(3, 64, 300, 656)
    assert plan.tiles == 2
    q512 = torch.zeros((3, 64, 512), dtype=torch.uint8, device="cuda")
    with pytest.raises(smla.SmlaError) as e:        # the score takes latent and rope
        smla.sparse_mla_decode(q512, d.kv_a, d.indices, d.lens, 0.1, 1.0, d.out, d.lse,
                               qk_dim=512, plan=plan, workspace=d.workspace(plan))
    assert e.value.status == smla.SMLA_EINVAL


def _sampled_units(T, H, count=48, seed=8):
    rng = np.random.default_rng(seed)
    units = {(0, 0), (T - 1, H - 1), (0, H - 1), (T - 1, 0), (31, 64), (32, 63)}
    while len(units) < count:
        units.add((int(rng.integers(T)), int(rng.integers(H))))
    return sorted(units)


def test_ds_mla_throughput_shape_sampled_parity():
    """The large-batch shape (T=64, H=128, 2048 columns over a 1M-row pool) on 656-byte rows,
    under its default plan (two-term P, against the exact oracle) and under the chunk-local
    recipe (against the oracle's chunk-local mode), on sampled (token, head) units."""
    log("generating the throughput workload on 656-byte rows on the device")
    w = inputs.config_throughput_ds_device("cuda")
    T, H, W = 64, 128, 2048
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    host = dict(q=w["q"].cpu().numpy(), kv_a=w["kv_a"].cpu().numpy(), kv_b=None, split_col=W,
                qk_dim=576, indices=w["indices"].cpu().numpy(), lens=w["lens"].cpu().numpy(),
                sinks=None, bmm1=w["bmm1"], bmm2=w["bmm2"])
    units = _sampled_units(T, H)
    ex, ex_lse = oracle.decode_exact(host, units=units)
    for chunk_local in (False, True):
        flags = smla.SMLA_P_CHUNK_LOCAL if chunk_local else 0
        plan = smla.plan_for(T, H, W, 656, flags)
        smla.sparse_mla_decode(w["q"], w["kv_a"], w["indices"], w["lens"], w["bmm1"], w["bmm2"],
                               out, lse, chunk_local=chunk_local, plan=plan,
                               workspace=smla.new_workspace(plan, T, H))
        torch.cuda.synchronize()
        assert np.all(np.isfinite(bf16_to_f64(out)))
        got = np.stack([bf16_to_f64(out[t, h]) for t, h in units])
        got_lse = np.array([float(lse[t, h]) for t, h in units])
        re, me, lee = rel_l2(got, ex), float(np.abs(got - ex).max()), lse_err(got_lse, ex_lse)
        if chunk_local:
            ref, ref_lse = oracle.decode_chunk_local(host, units=units)
            r, le = rel_l2(got, ref), lse_err(got_lse, ref_lse)
            log(f"656-byte throughput shape {plan} chunk-local: vs recipe rel_l2={r:.3e} "
                f"lse={le:.3e} ({flip_stats(got, ref, MIMIC_MAX_ABS)}); vs exact rel_l2={re:.3e} "
                f"max_abs={me:.3e} lse={lee:.3e} over {len(units)} units")
            assert r <= MIMIC_REL_L2 and le <= LSE_ABS
            assert mimic_max_abs_ok(got, ref, MIMIC_MAX_ABS, EXACT_MAX_ABS)
            assert re <= ONE_TERM_EXACT_REL_L2 and me <= EXACT_MAX_ABS and lee <= LSE_ABS
        else:
            log(f"656-byte throughput shape {plan}: vs exact rel_l2={re:.3e} max_abs={me:.3e} "
                f"lse={lee:.3e} over {len(units)} units")
            assert re <= EXACT_REL_L2 and me <= EXACT_MAX_ABS and lee <= LSE_ABS
