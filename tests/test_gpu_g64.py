"""Parity of the 64-head decode kernel (plan tiles=2: rows gathered straight into LDS) with the
FP64 oracle, and bit equality with the 32-head kernel: both run the same instructions per
(column tile, head tile) in the same order (QK steps, running maxima and rescale factors, P
bytes, accumulator rescales, P.V chunk order, l sums, split merge), so for the same split plan
their outputs must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, EXACT_REL_L2, LSE_ABS, MIMIC_MAX_ABS, MIMIC_REL_L2,
                          DeviceProblem, bf16_to_f64, check_empty_rows_exact, flip_stats, log,
                          lse_err, mimic_max_abs_ok, rel_l2)

pytestmark = pytest.mark.gpu

LN2 = np.log(2.0)


def _exact(p, out, lse, lse_log2, label):
    ref, ref_lse = oracle.decode_exact(p, lse_log2=lse_log2)
    if lse_log2:
        ref_lse, lse = ref_lse * LN2, lse * LN2
    r, m, le = rel_l2(out, ref), float(np.abs(out - ref).max()), lse_err(lse, ref_lse)
    log(f"{label}: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
    assert np.all(np.isfinite(out)), "non-finite output"
    tol_abs = EXACT_MAX_ABS * max(1.0, p.get("value_scale", 1.0))
    assert r <= EXACT_REL_L2 and m <= tol_abs and le <= LSE_ABS, (r, m, le)


def _mimic(p, out, lse, plan, label):
    """One-term path against mimic mode of the same plan (the attn_sparse page's recipe), at the
    tolerances stated in smla_testlib (one-code E4M3 flips from FP32 vs FP64 scores allowed on
    a few isolated elements)."""
    ref, ref_lse = oracle.decode_mimic(p, splits=plan.splits, chunk=plan.chunk, terms=1)
    r, m, le = rel_l2(out, ref), float(np.abs(out - ref).max()), lse_err(lse, ref_lse)
    tol_abs = MIMIC_MAX_ABS * max(1.0, p.get("value_scale", 1.0))
    log(f"{label} vs mimic: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e} "
        f"({flip_stats(out, ref, tol_abs)})")
    assert r <= MIMIC_REL_L2 and le <= LSE_ABS, (r, m, le)
    assert mimic_max_abs_ok(out, ref, tol_abs, EXACT_MAX_ABS * max(1.0, p.get("value_scale", 1.0))), (r, m, le)


def _same_bits(d, p, splits, one_term):
    """Run the 32-head and the 64-head kernel under the same split count; return both bit
    patterns (out as int16, lse as int32)."""
    res = []
    for tiles in (1, 2):
        d.run(plan=smla.make_plan(splits, tiles), one_term=one_term)
        res.append((d.out.view(torch.int16).cpu().clone(), d.lse.view(torch.int32).cpu().clone()))
    return res


CASES = {
    "H64_one_chunk": dict(seed=500, T=1, H=64, W=64),
    "H128_ragged": dict(seed=501, T=3, H=128, W=300, lens=[300, 129, 77], neg_frac=0.1),
    "H64_empty_rows": dict(seed=502, T=4, H=64, W=200, lens=[150, 0, -3, 200], neg_frac=0.05),
    "H48_padded_heads": dict(seed=503, T=2, H=48, W=260, lens=[260, 61], sinks=True),
    "H64_sinks_amax": dict(seed=504, T=3, H=64, W=390, kv_scale_to_amax=True, sinks=True,
                           lens=[390, 5, 255], neg_frac=0.1),
    "H64_large_scores": dict(seed=505, T=2, H=64, W=300, value_scale=4.0),
    "H64_duplicates": dict(seed=506, T=2, H=64, W=200, duplicates=True, pool_rows=50),
    "H64_W1": dict(seed=507, T=3, H=64, W=1, lens=[1, 0, 1]),
    "H64_rows512_two_pools": dict(seed=508, T=3, H=64, W=300, row_bytes=512, two_pools=True,
                                  split_col=128, rows_b=5000, sinks=True, neg_frac=0.1,
                                  lens=[300, 129, 250]),
    "H128_rows576_qk512": dict(seed=509, T=2, H=128, W=200, qk_dim=512, lens=[200, 71]),
    "H64_long_range": dict(seed=510, T=2, H=64, W=2048, lens=[2048, 1000], neg_frac=0.05,
                           pool_rows=6000),
    # one 32-head tile, or an odd count of them: the last 64-head group is padded
    "H16_padded_group": dict(seed=511, T=3, H=16, W=300, lens=[300, 0, 190], neg_frac=0.1,
                             sinks=True),
    "H96_three_tiles": dict(seed=512, T=2, H=96, W=200, lens=[200, 133]),
    "H16_rows512_two_pools": dict(seed=513, T=2, H=16, W=640, row_bytes=512, two_pools=True,
                                  split_col=128, rows_b=5000, sinks=True, neg_frac=0.1,
                                  lens=[640, 431]),
}


def _problem(name):
    kw = dict(CASES[name])
    seed, T, H, W = kw.pop("seed"), kw.pop("T"), kw.pop("H"), kw.pop("W")
    if "lens" in kw:
        kw["lens"] = np.array(kw["lens"])
    kw.setdefault("pool_rows", 3000)
    return inputs.random_problem(seed, T, H, W, **kw)


@pytest.mark.parametrize("name", list(CASES))
def test_g64_exact_parity(name):
    p = _problem(name)
    log(f"64-head case {name}")
    d = DeviceProblem(p)
    for splits in (1, 3):
        for lse_log2 in (False, True):
            out, lse, plan = d.run(plan=smla.make_plan(splits, 2), lse_log2=lse_log2)
            check_empty_rows_exact(d.out, d.lse, p)
            _exact(p, out, lse, lse_log2, f"{name} {plan} log2={lse_log2}")


@pytest.mark.parametrize("name", list(CASES))
def test_g64_one_term_matches_mimic(name):
    p = _problem(name)
    d = DeviceProblem(p)
    for splits in (1, 2):
        plan = smla.make_plan(splits, 2)
        out, lse, _ = d.run(plan=plan, one_term=True)
        check_empty_rows_exact(d.out, d.lse, p)
        _mimic(p, out, lse, plan, f"{name} {plan} one-term")


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("one_term", [False, True])
def test_g64_equals_32_head_kernel_bitwise(name, one_term):
    p = _problem(name)
    d = DeviceProblem(p)
    for splits in (1, 4):
        (o1, l1), (o2, l2) = _same_bits(d, p, splits, one_term)
        assert torch.equal(o1, o2), f"splits={splits}: outputs differ"
        assert torch.equal(l1, l2), f"splits={splits}: LSE differs"


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
def test_g64_split_plans(splits):
    p = inputs.random_problem(520 + splits, 3, 64, 300, pool_rows=3000,
                              lens=np.array([300, 40, 0]), neg_frac=0.1, sinks=True)
    d = DeviceProblem(p)
    out, lse, plan = d.run(plan=smla.make_plan(splits, 2))
    check_empty_rows_exact(d.out, d.lse, p)
    _exact(p, out, lse, False, f"64-head splits={splits}")
    out, lse, plan = d.run(plan=smla.make_plan(splits, 2), one_term=True)
    _mimic(p, out, lse, plan, f"64-head splits={splits} one-term")


def test_g64_rising_scores_rescale_every_chunk():
    """Scores climbing ~250 binades along the row: the running maximum rises at every chunk and
    the accumulators are rescaled each time (same problem as the 32-head kernel's test, at 64
    heads)."""
    from test_gpu_decode import _rising_scores_problem
    p = _rising_scores_problem(530, 2, 64, 700, [700, 377])
    d = DeviceProblem(p)
    for splits in (1, 2):
        plan = smla.make_plan(splits, 2)
        out, lse, _ = d.run(plan=plan)
        _exact(p, out, lse, False, f"64-head rising scores splits={splits}")
        out, lse, _ = d.run(plan=plan, one_term=True)
        _mimic(p, out, lse, plan, f"64-head rising scores splits={splits} one-term")
        (o1, l1), (o2, l2) = _same_bits(d, p, splits, False)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_g64_padded_q_strides():
    p = inputs.random_problem(531, 2, 64, 150, pool_rows=2000)
    d = DeviceProblem(p, q_pad_heads=16)
    out, lse, _ = d.run(plan=smla.make_plan(1, 2))
    _exact(p, out, lse, False, "64-head padded q")


def test_g64_verify_row_config():
    p = inputs.CONFIGS["verify"]()
    d = DeviceProblem(p)
    for splits in (1, 2, 4):
        out, lse, plan = d.run(plan=smla.make_plan(splits, 2))
        check_empty_rows_exact(d.out, d.lse, p)
        _exact(p, out, lse, p["lse_log2"], f"verify-row 64-head {plan}")


def test_g64_graph_replay_matches_eager():
    p = inputs.random_problem(532, 3, 128, 300, pool_rows=4000, neg_frac=0.1, sinks=True,
                              lens=np.array([300, 0, 177]))
    d = DeviceProblem(p)
    plan = smla.make_plan(3, 2)
    d.run(plan=plan, poison_out=False)
    ref_out = d.out.view(torch.int16).clone()
    ref_lse = d.lse.view(torch.int32).clone()
    ws = d.workspace(plan)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def call(stream):
        smla.sparse_mla_decode(d.q, d.kv_a, d.indices, d.lens, p["bmm1"], p["bmm2"], d.out,
                               d.lse, sinks=d.sinks, plan=plan, workspace=ws, stream=stream)
    with torch.cuda.stream(s):
        call(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(s)
        call(s)
    torch.cuda.synchronize()
    for rep in range(4):
        d.out.view(torch.int16).fill_(0x7FC0)
        d.lse.fill_(float("nan"))
        junk = torch.randn(1 << 16, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(d.out.view(torch.int16), ref_out), f"replay {rep}: out differs"
        assert torch.equal(d.lse.view(torch.int32), ref_lse), f"replay {rep}: lse differs"
        del junk


def test_g64_large_batch_split_merge_is_deterministic():
    """The large-batch launch (T=64, H=128, 2048 columns, two ranges per 64-head group: 256
    workgroups that all reach the split exchange together): eight calls on one workspace give
    the first call's bytes, equal to the 32-head kernel's under the same two-range plan (its
    store-first exchange), and within the exact-mode tolerance of a one-range launch (no
    exchange at all)."""
    w = inputs.config_throughput_device("cuda", index_sets=1)
    T, H = 64, 128
    idx = w["index_sets"][0]
    plan = smla.make_plan(2, 2)
    ws = smla.new_workspace(plan, T, H)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ref = torch.empty_like(out)
    ref_lse = torch.empty_like(lse)
    smla.sparse_mla_decode(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], ref, ref_lse,
                           plan=smla.make_plan(2, 1), workspace=smla.new_workspace(
                               smla.make_plan(2, 1), T, H))
    one = torch.empty_like(out)
    one_lse = torch.empty_like(lse)
    smla.sparse_mla_decode(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], one, one_lse,
                           plan=smla.make_plan(1, 2))
    torch.cuda.synchronize()
    a, b = ref.float().cpu().numpy(), one.float().cpu().numpy()
    r, m = rel_l2(a, b), float(np.abs(a - b).max())
    dl = float((ref_lse - one_lse).abs().max())
    log(f"large batch: two ranges vs one range rel_l2={r:.3e} max_abs={m:.3e} lse={dl:.3e}")
    assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and dl <= LSE_ABS
    first = None
    for i in range(8):
        out.view(torch.int16).fill_(0x7FC0)
        smla.sparse_mla_decode(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], out, lse,
                               plan=plan, workspace=ws)
        torch.cuda.synchronize()
        got = out.view(torch.int16).clone()
        if first is None:
            first = got
        bad = int((got != first).sum())
        assert bad == 0, f"call {i}: {bad} output elements differ from the first call"
        assert torch.equal(got, ref.view(torch.int16)), f"call {i}: differs from the 32-head kernel"
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


def test_g64_merge_wait_gives_up_loudly():
    """The merging range's wait is bounded.  Forced from the host (the test hook makes it wait
    for one partial more than exists, for 16 polls; every kernel still exits normally), each
    (token, head group) merge gives up: the workspace status word counts them, their outputs
    and LSEs are NaN, and after the workspace is zero-filled again the next call is correct."""
    p = inputs.random_problem(540, 3, 128, 300, pool_rows=3000, neg_frac=0.1, sinks=True,
                              lens=np.array([300, 170, 260]))
    d = DeviceProblem(p)
    plan = smla.make_plan(2, 2)
    ws = smla.new_workspace(plan, d.T, d.H)

    def call():
        smla.sparse_mla_decode(d.q, d.kv_a, d.indices, d.lens, p["bmm1"], p["bmm2"], d.out,
                               d.lse, sinks=d.sinks, plan=plan, workspace=ws)
        torch.cuda.synchronize()
    try:
        smla.testing_set_merge_wait(16, unreachable=True)
        call()
    finally:
        smla.testing_set_merge_wait()
    units = d.T * 2  # two 64-head groups per token
    assert smla.workspace_status(ws) == units
    assert torch.isnan(d.out.float()).all(), "a merge that gave up must not write a result"
    assert torch.isnan(d.lse).all()
    ws.zero_()
    call()
    assert smla.workspace_status(ws) == 0
    out = bf16_to_f64(d.out).reshape(d.T * d.H, 512)
    _exact(p, out, d.lse.cpu().numpy().astype(np.float64).reshape(-1), False,
           "after the workspace was zero-filled again")
