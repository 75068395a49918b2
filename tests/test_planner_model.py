"""The planner's cost model exists twice: in the library (predicted_us, csrc/smla_api.hip) and in
plan_fit.py, which fits it and mirrors its choice.  These CPU checks keep the two in step: the
same coefficient table, and features that behave as the model's terms say."""
import os
import re

from sparse_mla_attention_amd import build, plan_fit


def _library_table():
    src = open(os.path.join(build.CSRC, "smla_api.hip")).read()
    block = src[src.index("kCoef[5][10]"):]
    block = block[:block.index("};")]
    rows = re.findall(r"\{([^{}]*)\}", block)
    return [[float(x) for x in r.split(",")] for r in rows]


def test_coefficient_tables_agree():
    assert _library_table() == plan_fit.LIBRARY_COEF


def test_features_of_each_kind():
    # one range: no split terms
    f = plan_fit.features(64, 128, 2048, 1, 2, 0, 0)
    assert f[5:] == [0.0] * 5
    # last arriver: S - 1 partials moved, no spread term
    f = plan_fit.features(64, 128, 2048, 2, 2, 0, 0)
    assert f[5] == 2 and f[9] == 0.0
    assert f[7] == 64 * 128 * 1 * 4096.0 / 1e6
    # spread: S partials moved, ranges/16 x occupancy (200 of 256 compute units here)
    f = plan_fit.features(5, 128, 320, 5, 2, 1, 16)
    assert f[7] == 5 * 128 * 5 * 4096.0 / 1e6
    assert abs(f[9] - 5 / 16 * 200 / 256) < 1e-12
    # a full device: the grid's rounds
    f = plan_fit.features(64, 128, 2048, 2, 1, 0, 0)
    assert f[1] == 2  # 64 x 4 x 2 = 512 workgroups: two rounds on 256 compute units


def test_candidates_respect_the_kernels_limits():
    for T, H, W in [(1, 16, 64), (5, 128, 320), (12, 16, 640), (64, 128, 2048), (3, 64, 4096)]:
        for s, t, m, h in plan_fit.candidates(T, H, W):
            gw = h or 32 * t
            if t == 2:
                assert -(-W // s) <= 2048
            if m == 1:
                assert 2 <= s <= 16 and T * -(-H // gw) * s <= plan_fit.CUS
        assert plan_fit.library_plan(T, H, W) in plan_fit.candidates(T, H, W)
