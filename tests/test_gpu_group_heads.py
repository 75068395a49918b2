"""Plans with 16 or 32 real heads per 64-head workgroup (plan heads): every head's scores,
softmax, P.V column and merge depend on that head alone, so the output and LSE bits must equal
those of the default 64-head grouping under the same split count and merge mode; parity with the
FP64 oracle, the paged mode, and the host's checks of the field."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, EXACT_REL_L2, LSE_ABS, DeviceProblem, bf16_to_f64,
                          check_empty_rows_exact, dev, log, lse_err, rel_l2)

pytestmark = pytest.mark.gpu

SPREAD, LAST = smla.SMLA_MERGE_SPREAD, smla.SMLA_MERGE_LAST

CASES = {
    "H128_ragged_empty": dict(seed=800, T=3, H=128, W=700, lens=[700, 0, 333], neg_frac=0.1,
                              sinks=True),
    "H96_three_tiles": dict(seed=801, T=2, H=96, W=300, lens=[300, 129]),
    "H48_padded": dict(seed=802, T=2, H=48, W=520, lens=[520, 77], sinks=True),
    "H64_rows512_two_pools": dict(seed=803, T=3, H=64, W=640, row_bytes=512, two_pools=True,
                                  split_col=128, rows_b=5000, sinks=True, neg_frac=0.1,
                                  lens=[640, 431, 5]),
}


def _problem(name):
    kw = dict(CASES[name])
    seed, T, H, W = kw.pop("seed"), kw.pop("T"), kw.pop("H"), kw.pop("W")
    kw["lens"] = np.array(kw["lens"])
    kw.setdefault("pool_rows", 4000)
    return inputs.random_problem(seed, T, H, W, **kw)


def _bits(d):
    return d.out.view(torch.int16).cpu().clone(), d.lse.view(torch.int32).cpu().clone()


@pytest.mark.parametrize("name", list(CASES))
def test_group_heads_equal_default_grouping_bitwise(name):
    p = _problem(name)
    d = DeviceProblem(p)
    for one_term in (False, True):
        for splits, merge in ((1, LAST), (2, LAST), (3, LAST), (2, SPREAD), (4, SPREAD)):
            d.run(plan=smla.make_plan(splits, 2, merge), one_term=one_term)
            ref = _bits(d)
            for heads in (16, 32):
                plan = smla.make_plan(splits, 2, merge, heads=heads)
                log(f"{name} {plan} one_term={one_term}")
                out, lse, _ = d.run(plan=plan, one_term=one_term)
                got = _bits(d)
                bad = int((got[0] != ref[0]).sum())
                assert bad == 0, f"{plan}: {bad} output elements differ from 64-head groups"
                assert torch.equal(got[1], ref[1]), f"{plan}: LSE differs"
                check_empty_rows_exact(d.out, d.lse, p)


@pytest.mark.parametrize("cfg", ["verify", "dsv4"])
def test_group_heads_configs_exact(cfg):
    """The verify-row and DeepSeek-V4 workloads with 16 heads per workgroup against the exact
    oracle."""
    p = inputs.CONFIGS[cfg]()
    d = DeviceProblem(p)
    lse_log2 = bool(p.get("lse_log2", False))
    ln2 = np.log(2.0)
    for splits, merge in ((1, LAST), (2, SPREAD), (4, SPREAD)):
        plan = smla.make_plan(splits, 2, merge, heads=16)
        out, lse, _ = d.run(plan=plan)
        check_empty_rows_exact(d.out, d.lse, p)
        ref, ref_lse = oracle.decode_exact(p, lse_log2=lse_log2)
        if lse_log2:
            ref_lse, lse = ref_lse * ln2, lse * ln2
        r, m, le = rel_l2(out, ref), float(np.abs(out - ref).max()), lse_err(lse, ref_lse)
        log(f"{cfg} {plan}: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
        assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS


def test_group_heads_paged_equals_default():
    pp = inputs.paged_problem(804, B=2, q_len=3, H=128, lengths=np.array([900, 130]),
                              page_size=64, max_pages=16)
    T = 6
    q, cache = dev(pp["q"]), dev(pp["cache"])
    bt, lens = dev(pp["block_table"]), dev(pp["lengths"])
    res = []
    for heads in (0, 16, 32):
        plan = smla.make_plan(2, 2, LAST, heads=heads)
        ws = smla.new_workspace(plan, T, 128)
        out = torch.full((T, 128, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, 128), float("nan"), dtype=torch.float32, device="cuda")
        smla.paged_mla_decode(q, cache, bt, lens, 3, pp["bmm1"], pp["bmm2"], out, lse,
                              plan=plan, workspace=ws)
        torch.cuda.synchronize()
        res.append((out.view(torch.int16).cpu(), lse.view(torch.int32).cpu()))
    for got in res[1:]:
        assert torch.equal(got[0], res[0][0]) and torch.equal(got[1], res[0][1])
    ref, _ = oracle.paged_decode_exact(pp)
    got = res[1][0].view(torch.bfloat16).to(torch.float64).numpy().reshape(ref.shape)
    assert rel_l2(got, ref) <= EXACT_REL_L2


def test_group_heads_are_checked():
    """Only the 64-head kernel takes 16 or 32 real heads; any other width is refused."""
    p = inputs.random_problem(805, 2, 64, 200, pool_rows=2000)
    d = DeviceProblem(p)
    for tiles, heads in ((1, 16), (2, 8), (2, 48), (1, 64)):
        with pytest.raises(smla.SmlaError) as e:
            d.run(plan=smla.make_plan(2, tiles, heads=heads))
        assert e.value.status == smla.SMLA_EINVAL
    out, lse, plan = d.run(plan=smla.make_plan(1, 1, heads=32))   # the 32-head kernel's own
    ref, _ = oracle.decode_exact(p)
    assert rel_l2(out, ref) <= EXACT_REL_L2
