"""The no-allocation entry point (sparse_mla_decode_noalloc, the library's static per-device
scratch as the split-KV workspace) against sparse_mla_decode with a workspace of the caller's:
same kernels and plan, so the same bytes, on two calls in a row, the second smaller."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import DeviceProblem, log

pytestmark = pytest.mark.gpu


def _pair(d, p, plan, one_term=False, chunk_local=False):
    """(reference bytes with a caller workspace, no-alloc bytes), both out and LSE."""
    d.run(plan=plan, one_term=one_term, chunk_local=chunk_local)
    ref = d.out.view(torch.int16).clone(), d.lse.view(torch.int32).clone()
    d.out.view(torch.int16).fill_(0x7FC0)
    d.lse.fill_(float("nan"))
    smla.sparse_mla_decode_noalloc(d.q, d.kv_a, d.indices, d.lens, p["bmm1"], p["bmm2"], d.out,
                                   d.lse, kv_b=d.kv_b, split_col=p["split_col"], sinks=d.sinks,
                                   qk_dim=p["qk_dim"], lse_log2=bool(p.get("lse_log2", False)),
                                   one_term=one_term, plan=plan, chunk_local=chunk_local)
    torch.cuda.synchronize()
    return ref, (d.out.view(torch.int16).clone(), d.lse.view(torch.int32).clone())


def test_noalloc_matches_workspace_call_twice_second_smaller():
    log("no-alloc: large-batch call, default plan")
    w = inputs.config_throughput_device("cuda", index_sets=1)
    T, H, W = 64, 128, 2048
    idx = w["index_sets"][0]
    plan = smla.plan_for(T, H, W, 576)
    assert 0 < smla.workspace_size(plan, T, H) <= smla.NOALLOC_SCRATCH_BYTES
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    smla.sparse_mla_decode(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], out, lse,
                           plan=plan, workspace=smla.new_workspace(plan, T, H))
    torch.cuda.synchronize()
    ref_out, ref_lse = out.view(torch.int16).clone(), lse.view(torch.int32).clone()
    out.view(torch.int16).fill_(0x7FC0)
    smla.sparse_mla_decode_noalloc(w["q"], w["kv_a"], idx, w["lens"], w["bmm1"], w["bmm2"], out,
                                   lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out)
    assert torch.equal(lse.view(torch.int32), ref_lse)
    del w, out, lse
    log("no-alloc: smaller call after it (three ranges, 64-head and 32-head kernels)")
    p = inputs.random_problem(700, 3, 128, 300, pool_rows=3000, neg_frac=0.1, sinks=True,
                              lens=np.array([300, 0, 211]))
    d = DeviceProblem(p)
    for tiles in (2, 1):
        for one_term in (False, True):
            (ro, rl), (no, nl) = _pair(d, p, smla.make_plan(3, tiles), one_term)
            assert torch.equal(ro, no), (tiles, one_term)
            assert torch.equal(rl, nl), (tiles, one_term)
    # the verify-row shape under its default plan (a spread merge over 16- or 32-head groups)
    v = inputs.CONFIGS["verify"]()
    dv = DeviceProblem(v)
    (ro, rl), (no, nl) = _pair(dv, v, smla.plan_for(5, 128, 320, 576))
    assert torch.equal(ro, no) and torch.equal(rl, nl)


def test_noalloc_matches_for_the_chunk_local_recipe_and_fp8_ds_mla_rows():
    """The same entry point under the chunk-local recipe (DeepSeek-V4 workload, five windows
    under the spread merge) and on 656-byte rows (verify-row shape), default plans, two calls
    each."""
    p = inputs.CONFIGS["dsv4"]()
    d = DeviceProblem(p)
    plan = smla.plan_for(d.T, d.H, p["indices"].shape[1], 512, smla.SMLA_P_CHUNK_LOCAL)
    log(f"no-alloc: chunk-local {plan}")
    for _ in range(2):
        (ro, rl), (no, nl) = _pair(d, p, plan, chunk_local=True)
        assert torch.equal(ro, no) and torch.equal(rl, nl)
    p = inputs.random_problem(702, 5, 128, 320, pool_rows=3000, row_bytes=656, neg_frac=0.1,
                              sinks=True)
    d = DeviceProblem(p)
    plan = smla.plan_for(5, 128, 320, 656)
    log(f"no-alloc: 656-byte rows {plan}")
    for one_term in (False, True):
        (ro, rl), (no, nl) = _pair(d, p, plan, one_term)
        assert torch.equal(ro, no) and torch.equal(rl, nl)


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    """T=64, H=128 with 64 ranges of the 32-head kernel needs ~269 MB of workspace: rejected
    before anything is launched, and the outputs keep their bytes."""
    p = inputs.random_problem(701, 64, 128, 128, pool_rows=2000)
    d = DeviceProblem(p)
    plan = smla.make_plan(64, 1)
    assert smla.workspace_size(plan, 64, 128) > smla.NOALLOC_SCRATCH_BYTES
    d.out.view(torch.int16).fill_(0x1234)
    with pytest.raises(smla.SmlaError) as e:
        smla.sparse_mla_decode_noalloc(d.q, d.kv_a, d.indices, d.lens, p["bmm1"], p["bmm2"],
                                       d.out, d.lse, plan=plan)
    assert e.value.status == smla.SMLA_ESCRATCH
    torch.cuda.synchronize()
    assert bool((d.out.view(torch.int16) == 0x1234).all())
