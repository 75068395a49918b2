"""Grids that fill the device take the 64-head kernel variant whose index rows are loaded
alongside each token's count (the host selects it when T x head groups x ranges reaches the
compute-unit count).  Checked here on ragged counts (zero, negative, past W), unused (-1)
columns, two pools and sinks: against the FP64 oracle, bit-exact on empty rows, and bit for bit
against the same tokens decoded in two halves, whose grids are below the compute-unit count
and take the variant that loads the indices after the count."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import (EXACT_MAX_ABS, EXACT_REL_L2, LSE_ABS, DeviceProblem,
                          check_empty_rows_exact, log, lse_err, rel_l2)

pytestmark = pytest.mark.gpu


def _sub(p, lo, hi):
    """Tokens [lo, hi) of problem p (the pools, sinks and scales are shared)."""
    q = dict(p)
    for k in ("q", "indices", "lens"):
        q[k] = np.ascontiguousarray(p[k][lo:hi])
    return q


@pytest.mark.parametrize("splits,one_term", [(2, False), (2, True), (3, False)])
def test_full_grid_matches_oracle_and_half_grids(splits, one_term):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    H, W = 64, 300                                  # one 64-head group per token
    T = 2 * ((cus + 2 * splits - 1) // (2 * splits))  # T x splits >= cus, T even
    rng = np.random.default_rng(900 + splits)
    lens = rng.integers(-5, W + 20, size=T)
    lens[:4] = [W, 0, -2, W + 7]
    p = inputs.random_problem(900 + splits, T, H, W, pool_rows=6000, lens=lens, neg_frac=0.1,
                              two_pools=True, split_col=128, rows_b=5000, sinks=True)
    plan = smla.make_plan(splits, 2)
    d = DeviceProblem(p)
    log(f"full grid: T={T} H={H} W={W} {plan} one_term={one_term} ({T * splits} workgroups, "
        f"{cus} compute units)")
    got, got_lse, _ = d.run(plan=plan, one_term=one_term)
    check_empty_rows_exact(d.out, d.lse, p)
    if not one_term:
        ref, ref_lse = oracle.decode_exact(p)
        r, m, le = rel_l2(got, ref), float(np.abs(got - ref).max()), lse_err(got_lse, ref_lse)
        log(f"vs exact: rel_l2={r:.3e} max_abs={m:.3e} lse={le:.3e}")
        assert r <= EXACT_REL_L2 and m <= EXACT_MAX_ABS and le <= LSE_ABS, (r, m, le)
    full_bits = (d.out.view(torch.int16).cpu().clone(), d.lse.view(torch.int32).cpu().clone())
    for lo, hi in ((0, T // 2), (T // 2, T)):
        h = DeviceProblem(_sub(p, lo, hi))
        h.run(plan=plan, one_term=one_term)
        assert torch.equal(h.out.view(torch.int16).cpu(), full_bits[0][lo:hi]), (lo, hi)
        assert torch.equal(h.lse.view(torch.int32).cpu(), full_bits[1][lo:hi]), (lo, hi)
