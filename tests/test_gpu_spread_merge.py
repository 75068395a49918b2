"""The spread split merge (plan merge = SMLA_MERGE_SPREAD): range s of a (token, head group)
merges output columns [s, s+1) * 512 / S of every head, after every range has published the
columns the others merge.  It performs the same FP32 operations in the same range order as the
last-arriver merge (weights 2^(m_s - M), sums from zero, range 0 first), so for the same plan
otherwise both merges must give the same bits; the tests here check that on both kernels and
the paged mode, parity with the FP64 oracle, repeated calls on one workspace (the counters are
reset by the last range to leave), graph replay, the host's validation, and the bounded
wait's loud give-up.  The spread merge is built into the 64-head kernel (plan tiles = 2)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, EXACT_REL_L2, LSE_ABS, DeviceProblem, bf16_to_f64,
                          check_empty_rows_exact, log, lse_err, rel_l2)

pytestmark = pytest.mark.gpu

LN2 = np.log(2.0)
SPREAD, LAST = smla.SMLA_MERGE_SPREAD, smla.SMLA_MERGE_LAST

CASES = {
    "H64_ragged_empty": dict(seed=700, T=4, H=64, W=900, lens=[900, 0, 333, 17], neg_frac=0.1,
                             sinks=True),
    "H128_verify_like": dict(seed=701, T=3, H=128, W=300, lens=[300, 200, 260]),
    "H48_padded_heads": dict(seed=702, T=2, H=48, W=700, lens=[700, 95], sinks=True),
    "H16_rows512_two_pools": dict(seed=703, T=3, H=16, W=640, row_bytes=512, two_pools=True,
                                  split_col=128, rows_b=5000, sinks=True, neg_frac=0.1,
                                  lens=[640, 431, 5]),
    "H64_amax": dict(seed=704, T=2, H=64, W=1200, kv_scale_to_amax=True, lens=[1200, 640],
                     neg_frac=0.05),
}


def _problem(name):
    kw = dict(CASES[name])
    seed, T, H, W = kw.pop("seed"), kw.pop("T"), kw.pop("H"), kw.pop("W")
    kw["lens"] = np.array(kw["lens"])
    kw.setdefault("pool_rows", 4000)
    return inputs.random_problem(seed, T, H, W, **kw)


def _bits(d):
    return d.out.view(torch.int16).cpu().clone(), d.lse.view(torch.int32).cpu().clone()


def _exact(p, out, lse, lse_log2, label):
    ref, ref_lse = oracle.decode_exact(p, lse_log2=lse_log2)
    if lse_log2:
        ref_lse, lse = ref_lse * LN2, lse * LN2
    r, m, le = rel_l2(out, ref), float(np.abs(out - ref).max()), lse_err(lse, ref_lse)
    log(f"{label}: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
    assert np.all(np.isfinite(out)), "non-finite output"
    assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS, (r, m, le)


@pytest.mark.parametrize("name", list(CASES))
def test_spread_merge_equals_last_arriver_bitwise(name):
    p = _problem(name)
    tiles = 2
    d = DeviceProblem(p)
    for one_term in (False, True):
        for splits in (2, 3, 4, 5, 7, 8, 16):
            log(f"spread merge {name} tiles={tiles} splits={splits} one_term={one_term}")
            d.run(plan=smla.make_plan(splits, tiles, LAST), one_term=one_term)
            ref = _bits(d)
            out, lse, plan = d.run(plan=smla.make_plan(splits, tiles, SPREAD), one_term=one_term)
            got = _bits(d)
            bad = int((got[0] != ref[0]).sum())
            assert bad == 0, f"{plan}: {bad} output elements differ from the last-arriver merge"
            assert torch.equal(got[1], ref[1]), f"{plan}: LSE differs"
            check_empty_rows_exact(d.out, d.lse, p)
            if not one_term and splits in (2, 16):
                _exact(p, out, lse, bool(p.get("lse_log2", False)), f"{name} {plan}")


@pytest.mark.parametrize("cfg", ["verify", "dsv4"])
def test_spread_merge_configs(cfg):
    """The verify-row (T=5, H=128) and DeepSeek-V4-shaped (T=12, H=16, two pools, sinks)
    workloads under spread plans that fill most compute units, against the oracle and the
    last-arriver merge."""
    p = inputs.CONFIGS[cfg]()
    d = DeviceProblem(p)
    for splits in (16, 8, 4, 2):
        tiles = 2
        d.run(plan=smla.make_plan(splits, tiles, LAST))
        ref = _bits(d)
        out, lse, plan = d.run(plan=smla.make_plan(splits, tiles, SPREAD))
        check_empty_rows_exact(d.out, d.lse, p)
        _exact(p, out, lse, bool(p.get("lse_log2", False)), f"{cfg} {plan}")
        got = _bits(d)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), plan


def test_spread_merge_repeated_calls_and_counters():
    """Ten calls on one workspace give the same bits, and the arrival and departure counters
    are back at zero after each call (the last range to leave resets them)."""
    p = inputs.random_problem(710, 5, 128, 1000, pool_rows=6000, neg_frac=0.1,
                              lens=np.array([1000, 0, 640, 999, 71]))
    d = DeviceProblem(p)
    for splits in (8, 2):
        plan = smla.make_plan(splits, 2, SPREAD)
        ws = d.workspace(plan)
        header = smla.workspace_header_bytes(plan, d.T, d.H)
        first = None
        for i in range(10):
            d.out.view(torch.int16).fill_(0x7FC0)
            smla.sparse_mla_decode(d.q, d.kv_a, d.indices, d.lens, p["bmm1"], p["bmm2"], d.out,
                                   d.lse, plan=plan, workspace=ws)
            torch.cuda.synchronize()
            assert int(torch.count_nonzero(ws[:header])) == 0, f"{plan} call {i}: header not zero"
            got = _bits(d)
            if first is None:
                first = got
            assert torch.equal(got[0], first[0]) and torch.equal(got[1], first[1]), (plan, i)


def test_spread_merge_graph_replay():
    """Two spread-merge calls captured in a graph replay to the eager bytes."""
    p = inputs.random_problem(711, 3, 128, 700, pool_rows=4000, neg_frac=0.1, sinks=True,
                              lens=np.array([700, 0, 377]))
    d = DeviceProblem(p)
    plan = smla.make_plan(4, 2, SPREAD)
    d.run(plan=plan, poison_out=False)
    ref = (d.out.view(torch.int16).clone(), d.lse.view(torch.int32).clone())
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
        assert torch.equal(d.out.view(torch.int16), ref[0]), f"replay {rep}: out differs"
        assert torch.equal(d.lse.view(torch.int32), ref[1]), f"replay {rep}: lse differs"
        del junk


def test_spread_merge_paged_equals_last_arriver():
    pp = inputs.paged_problem(712, B=3, q_len=2, H=128, lengths=np.array([1500, 0, 777]),
                              page_size=64, max_pages=24)
    T = 6
    q = torch.from_numpy(pp["q"]).cuda()
    cache = torch.from_numpy(pp["cache"]).cuda()
    bt = torch.from_numpy(pp["block_table"]).cuda()
    lens = torch.from_numpy(pp["lengths"]).cuda()
    ref, _ = oracle.paged_decode_exact(pp)
    for splits in (4, 2):  # two ranges: the two-range spread merge
        res = []
        for merge in (LAST, SPREAD):
            plan = smla.make_plan(splits, 2, merge)
            ws = smla.new_workspace(plan, T, 128)
            out = torch.full((T, 128, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
            lse = torch.full((T, 128), float("nan"), dtype=torch.float32, device="cuda")
            smla.paged_mla_decode(q, cache, bt, lens, 2, pp["bmm1"], pp["bmm2"], out, lse,
                                  plan=plan, workspace=ws)
            torch.cuda.synchronize()
            res.append((out.view(torch.int16).cpu(), lse.view(torch.int32).cpu()))
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), splits
        got = res[1][0].view(torch.bfloat16).to(torch.float64).numpy().reshape(ref.shape)
        r = rel_l2(got, ref)
        log(f"paged spread merge, {splits} ranges: rel_l2={r:.3e}")
        assert r <= EXACT_REL_L2


def test_two_range_spread_on_656_byte_rows_and_chunk_local():
    """The two-range spread merge on fp8_ds_mla rows (656 bytes) and under the chunk-local
    recipe with two 128-column windows: bit for bit the last-arriver merge of the same plan."""
    cases = [
        ("656-byte rows", inputs.random_problem(720, 3, 64, 300, pool_rows=3000, row_bytes=656,
                                                lens=np.array([300, 77, 0]), neg_frac=0.1,
                                                sinks=True), False),
        ("chunk-local, two windows", inputs.random_problem(721, 3, 128, 256, pool_rows=3000,
                                                           lens=np.array([256, 140, 100]),
                                                           neg_frac=0.1, sinks=True), True),
    ]
    for label, p, cl in cases:
        d = DeviceProblem(p)
        bits = []
        for merge in (LAST, SPREAD):
            plan = smla.make_plan(2, 2, merge)
            d.run(plan=plan, chunk_local=cl)
            bits.append(_bits(d))
        log(f"{label}: two ranges, spread vs last arriver")
        assert torch.equal(bits[0][0], bits[1][0]) and torch.equal(bits[0][1], bits[1][1]), label
        check_empty_rows_exact(d.out, d.lse, p)


def test_spread_merge_validation():
    """Spread plans the kernels cannot run are refused on the host before any launch: the
    32-head kernel, more ranges than the sixteen 32-column output tiles, grids larger than the
    compute-unit count (every workgroup must be resident at once), an unknown merge mode."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    p = inputs.random_problem(713, 2, 64, 300, pool_rows=2000, lens=np.array([300, 200]))
    d = DeviceProblem(p)
    for splits, tiles in ((17, 2), (32, 2), (2, 1), (4, 1)):
        with pytest.raises(smla.SmlaError) as e:
            d.run(plan=smla.make_plan(splits, tiles, SPREAD))
        assert e.value.status == smla.SMLA_EUNSUPPORTED
    with pytest.raises(smla.SmlaError) as e:
        d.run(plan=smla.make_plan(2, 2, 2))
    assert e.value.status == smla.SMLA_EINVAL
    # one (token, head group) more than fits: T * groups * splits = cus + 16
    T = cus // 16 + 1
    big = inputs.random_problem(714, T, 64, 200, pool_rows=2000)
    db = DeviceProblem(big)
    with pytest.raises(smla.SmlaError) as e:
        db.run(plan=smla.make_plan(16, 2, SPREAD))
    assert e.value.status == smla.SMLA_EUNSUPPORTED
    # a split count of 1 ignores the merge mode
    out, lse, plan = d.run(plan=smla.make_plan(1, 2, SPREAD))
    _exact(p, out, lse, False, f"{plan}")


def test_spread_merge_wait_gives_up_loudly():
    """Every range's wait is bounded.  Forced from the host (the test hook makes each range wait
    for one arrival more than exists, for 16 polls; every kernel still exits normally), every
    range gives up: the status word counts each of them, every output element and LSE is NaN,
    and once the workspace is zero-filled again the next call is correct."""
    p = inputs.random_problem(715, 3, 128, 600, pool_rows=3000, neg_frac=0.1, sinks=True,
                              lens=np.array([600, 170, 560]))
    d = DeviceProblem(p)
    for splits in (2, 4, 16):
        plan = smla.make_plan(splits, 2, SPREAD)
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
        assert smla.workspace_status(ws) == d.T * 2 * splits  # two 64-head groups
        assert torch.isnan(d.out.float()).all(), "a merge that gave up must not write a result"
        assert torch.isnan(d.lse).all()
        ws.zero_()
        call()
        assert smla.workspace_status(ws) == 0
        out = bf16_to_f64(d.out).reshape(d.T * d.H, 512)
        _exact(p, out, d.lse.cpu().numpy().astype(np.float64).reshape(-1), False,
               f"{plan} after the workspace was zero-filled again")
