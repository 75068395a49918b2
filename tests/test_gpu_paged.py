"""Parity of paged_mla_decode (dense paged MLA decode on the sparse path's skeleton; the dcp
page's stock_decode: block table, causal q rows, split-KV with its merge) with the FP64
oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, EXACT_REL_L2, LSE_ABS, MIMIC_MAX_ABS, MIMIC_REL_L2,
                          bf16_to_f64, dev, flip_stats, log, lse_err, mimic_max_abs_ok, rel_l2)

pytestmark = pytest.mark.gpu


def _run(p, plan=None, one_term=False, lse_log2=False):
    q, cache = dev(p["q"]), dev(p["cache"])
    bt, lens = dev(p["block_table"]), dev(p["lengths"])
    T, H, _ = p["q"].shape
    B, max_pages = p["block_table"].shape
    page_size = p["cache"].shape[1]
    use = plan if plan is not None else smla.paged_plan_for(B, p["q_len"], H, max_pages,
                                                            page_size)
    ws = smla.new_workspace(use, T, H)
    out = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    smla.paged_mla_decode(q, cache, bt, lens, p["q_len"], p["bmm1"], p["bmm2"], out, lse,
                          lse_log2=lse_log2, one_term=one_term, plan=use, workspace=ws)
    torch.cuda.synchronize()
    return out, lse, use


def _empty_rows_exact(p, out, lse):
    B, max_pages = p["block_table"].shape
    W = max_pages * p["cache"].shape[1]
    for t in range(p["q"].shape[0]):
        b, i = divmod(t, p["q_len"])
        if int(np.clip(p["lengths"][b] - (p["q_len"] - 1 - i), 0, W)) == 0:
            assert torch.count_nonzero(out[t].view(torch.int16)) == 0, f"row {t} not +0.0"
            assert bool((lse[t] == float("-inf")).all()), f"row {t} LSE not -inf"


CASES = {
    "decode_pages16": dict(seed=1000, B=3, q_len=1, H=16, lengths=[150, 1, 64], page_size=16),
    "verify5_short_context": dict(seed=1001, B=2, q_len=5, H=128, lengths=[300, 3],
                                  page_size=64),
    "q4_empty_request": dict(seed=1002, B=4, q_len=4, H=64, lengths=[700, 64, 129, 0],
                             page_size=64),
    "long_context_two_ranges": dict(seed=1003, B=1, q_len=1, H=128, lengths=[4000],
                                    page_size=64),
    "H48_page32": dict(seed=1004, B=2, q_len=2, H=48, lengths=[333, 97], page_size=32),
}


def _problem(name):
    kw = dict(CASES[name])
    return inputs.paged_problem(kw.pop("seed"), kw.pop("B"), kw.pop("q_len"), kw.pop("H"),
                                kw.pop("lengths"), **kw)


@pytest.mark.parametrize("name", list(CASES))
def test_paged_exact_parity(name):
    p = _problem(name)
    log(f"paged case {name}")
    for lse_log2 in (False, True):
        out, lse, plan = _run(p, lse_log2=lse_log2)
        _empty_rows_exact(p, out, lse)
        ref, ref_lse = oracle.paged_decode_exact(p, lse_log2=lse_log2)
        got = bf16_to_f64(out).reshape(ref.shape)
        gl = lse.cpu().numpy().astype(np.float64).reshape(-1)
        if lse_log2:
            gl, ref_lse = gl * np.log(2), ref_lse * np.log(2)
        r, m, le = rel_l2(got, ref), float(np.abs(got - ref).max()), lse_err(gl, ref_lse)
        log(f"  {plan} log2={lse_log2}: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
        assert np.all(np.isfinite(got))
        assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS


@pytest.mark.parametrize("name", list(CASES))
def test_paged_one_term_matches_recipe(name):
    """The one-term path against mimic mode over the same rows (the sparse view of the paged
    problem: the same counts and key order, hence the same ranges and chunks)."""
    p = _problem(name)
    out, lse, plan = _run(p, one_term=True)
    _empty_rows_exact(p, out, lse)
    ref, ref_lse = oracle.decode_mimic(inputs.paged_as_sparse(p), plan.splits, plan.chunk,
                                       terms=1)
    got = bf16_to_f64(out).reshape(ref.shape)
    gl = lse.cpu().numpy().astype(np.float64).reshape(-1)
    r, m, le = rel_l2(got, ref), float(np.abs(got - ref).max()), lse_err(gl, ref_lse)
    log(f"  {name} one-term {plan}: vs recipe rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e} "
        f"({flip_stats(got, ref, MIMIC_MAX_ABS)})")
    assert r <= MIMIC_REL_L2 and le <= LSE_ABS
    assert mimic_max_abs_ok(got, ref, MIMIC_MAX_ABS, EXACT_MAX_ABS)


@pytest.mark.parametrize("splits", [1, 2, 3, 7])
def test_paged_split_plans(splits):
    p = inputs.paged_problem(1010 + splits, 3, 3, 64, [500, 130, 2], page_size=64)
    out, lse, plan = _run(p, plan=smla.make_plan(splits, 2))
    _empty_rows_exact(p, out, lse)
    ref, ref_lse = oracle.paged_decode_exact(p)
    got = bf16_to_f64(out).reshape(ref.shape)
    gl = lse.cpu().numpy().astype(np.float64).reshape(-1)
    r, m, le = rel_l2(got, ref), float(np.abs(got - ref).max()), lse_err(gl, ref_lse)
    log(f"  paged splits={splits}: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
    assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS


def test_paged_rejects_32_head_plans_and_overlong_ranges():
    p = inputs.paged_problem(1020, 1, 1, 16, [100], page_size=64)
    with pytest.raises(smla.SmlaError) as e:
        _run(p, plan=smla.make_plan(1, 1))
    assert e.value.status == smla.SMLA_EUNSUPPORTED
    p = inputs.paged_problem(1021, 1, 1, 16, [3000], page_size=64)
    with pytest.raises(smla.SmlaError) as e:
        _run(p, plan=smla.make_plan(1, 2))      # one range of 3008 > 2048 keys
    assert e.value.status == smla.SMLA_EUNSUPPORTED


def test_paged_decode_workload_sampled():
    """B=32 requests, one q row each, H=128, 4096-token contexts in 64-row pages (75.5 MB of
    KV gathered per call, the benchmark's paged leg), in its default plan, on sampled units."""
    p = inputs.paged_problem(1030, 32, 1, 128, [4096] * 32, page_size=64, poison=False)
    out, lse, plan = _run(p)
    rng = np.random.default_rng(1031)
    units = sorted({(int(rng.integers(32)), int(rng.integers(128))) for _ in range(24)} |
                   {(0, 0), (31, 127)})
    ref, ref_lse = oracle.paged_decode_exact(p, units=units)
    got = np.stack([bf16_to_f64(out[t, h]) for t, h in units])
    gl = np.array([float(lse[t, h]) for t, h in units])
    r, m, le = rel_l2(got, ref), float(np.abs(got - ref).max()), lse_err(gl, ref_lse)
    log(f"  paged workload {plan}: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e} over "
        f"{len(units)} units")
    assert bool(torch.isfinite(out.float()).all())
    assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS
