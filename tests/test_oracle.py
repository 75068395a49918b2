"""Pins of the FP64 oracle to things other than itself (CPU only).

Each test checks the oracle against a library routine, a closed form, an invariant of the
softmax, or brute force on tiny inputs, chosen so that a plausible slip in the oracle (a
dropped term, a wrong sign, base or index, a transposed operand) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_amd import inputs

LN2 = math.log(2.0)


# ---------------------------------------------------------------------------
# number formats (pinned to torch's casts: a library routine)
# ---------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = np.array([oracle.e4m3_value(c) for c in codes])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.array_equal(ref[~nan], ours[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_rne_and_saturates():
    codes = np.arange(0, 0x7F)
    vals = np.array([oracle.e4m3_value(c) for c in codes])
    mids = (vals[:-1] + vals[1:]) / 2  # exact ties: round half to even
    rng = np.random.default_rng(0)
    xs = np.concatenate([vals, mids, mids * (1 + 1e-6), mids * (1 - 1e-6),
                         rng.uniform(0, 480, 4000), rng.uniform(0, 2.0 ** -6, 2000),
                         [448.0, 449.0, 463.9, 464.0, 500.0, 1e6]])
    xs = np.concatenate([xs, -xs]).astype(np.float32).astype(np.float64)
    ours = np.array([oracle.e4m3_encode(x) for x in xs], dtype=np.uint8)
    ref = torch.from_numpy(xs.astype(np.float32)).clamp(-448, 448).to(torch.float8_e4m3fn)
    ref = ref.view(torch.uint8).numpy()
    # torch keeps the sign of a negative value that rounds to zero, as does the oracle
    assert np.array_equal(ours, ref), xs[ours != ref][:10]
    for c in codes:  # every finite code is a fixed point
        assert oracle.e4m3_encode(oracle.e4m3_value(c)) == c


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=5000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ours = np.array([oracle.bf16_value(b) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


# ---------------------------------------------------------------------------
# exact mode against dense float64 attention (brute force, a library routine)
# ---------------------------------------------------------------------------

def _e4m3_f64(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64)


def _dense_reference(p, lse_log2=False):
    """Materialise each token's active rows and run torch's float64 SDPA on them.  A sink is an
    extra key with k = 0, v = 0 and an additive score bias equal to the sink."""
    T, H, _ = p["q"].shape
    W = p["indices"].shape[1]
    out = np.zeros((T, H, 512))
    lse = np.full((T, H), -np.inf)
    q = _e4m3_f64(p["q"])[..., :p["qk_dim"]]
    for t in range(T):
        n = int(np.clip(p["lens"][t], 0, W))
        rows = []
        for c in range(n):
            i = int(p["indices"][t, c])
            if i < 0:
                continue
            pool = p["kv_b"] if (p["kv_b"] is not None and c >= p["split_col"]) else p["kv_a"]
            rows.append(pool[i])
        if not rows:
            continue
        kv = _e4m3_f64(np.stack(rows))
        k = kv[:, :p["qk_dim"]]
        v = kv[:, :512]
        bias = torch.zeros((H, k.shape[0]), dtype=torch.float64)
        if p["sinks"] is not None:
            k = torch.cat([k, torch.zeros((1, k.shape[1]), dtype=torch.float64)])
            v = torch.cat([v, torch.zeros((1, 512), dtype=torch.float64)])
            sink = torch.from_numpy(p["sinks"].astype(np.float64))[:, None]
            bias = torch.cat([bias, sink], dim=1)
        qt = q[t][None]  # [1, H, d]
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, k[None].expand(1, -1, -1), v[None].expand(1, -1, -1), attn_mask=bias[None],
            scale=p["bmm1"])
        out[t] = (o[0] * p["bmm2"]).numpy()
        scores = p["bmm1"] * (q[t] @ k.T) + bias
        lse[t] = torch.logsumexp(scores, dim=1).numpy()
    if lse_log2:
        lse = lse / LN2
    return out.reshape(T * H, 512), lse.reshape(T * H)


@pytest.mark.parametrize("kw", [
    dict(T=1, H=16, W=32, row_bytes=576),
    dict(T=2, H=16, W=24, row_bytes=576, lens=[24, 17]),
    dict(T=2, H=16, W=20, row_bytes=512, sinks=True),
    dict(T=2, H=16, W=30, row_bytes=512, two_pools=True, split_col=7, sinks=True, rows_b=300),
    dict(T=1, H=16, W=16, row_bytes=576, kv_scale_to_amax=True),
    dict(T=2, H=16, W=32, row_bytes=576, qk_dim=512),
])
def test_exact_matches_dense_attention(kw):
    kw = dict(kw)
    T, H, W = kw.pop("T"), kw.pop("H"), kw.pop("W")
    p = inputs.random_problem(11 + W, T, H, W, pool_rows=256, **kw)
    for log2 in (False, True):
        out, lse = oracle.decode_exact(p, lse_log2=log2)
        ref_out, ref_lse = _dense_reference(p, lse_log2=log2)
        np.testing.assert_allclose(out, ref_out, rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_exact_units_subset_equals_full():
    p = inputs.random_problem(5, 3, 16, 40, pool_rows=300, neg_frac=0.2, lens=[40, 33, 0])
    full, lse = oracle.decode_exact(p)
    units = [(2, 5), (0, 0), (1, 15), (0, 9)]
    sub, sub_lse = oracle.decode_exact(p, units=units)
    for k, (t, h) in enumerate(units):
        assert np.array_equal(sub[k], full[t * 16 + h])
        assert sub_lse[k] == lse[t * 16 + h] or (np.isinf(lse[t * 16 + h]) and np.isinf(sub_lse[k]))


# ---------------------------------------------------------------------------
# softmax invariants and closed forms
# ---------------------------------------------------------------------------

def test_permuting_columns_and_adding_unused_columns_changes_nothing():
    p = inputs.random_problem(7, 2, 16, 48, pool_rows=400, neg_frac=0.25, lens=[48, 31],
                              sinks=True)
    out, lse = oracle.decode_exact(p)
    rng = np.random.default_rng(3)
    q = dict(p)
    idx = p["indices"].copy()
    for t in range(2):
        n = int(p["lens"][t])
        idx[t, :n] = idx[t, rng.permutation(n)]
    q["indices"] = idx
    out2, lse2 = oracle.decode_exact(q)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    # widen W with -1 columns inside the count
    r = dict(p)
    wide = np.full((2, 64), -1, np.int32)
    wide[:, :48] = p["indices"]
    for t in range(2):
        n = int(p["lens"][t])
        wide[t, :n + 16] = np.concatenate([p["indices"][t, :n], np.full(16, -1, np.int32)])
    r["indices"], r["lens"] = wide, p["lens"] + 16
    out3, lse3 = oracle.decode_exact(r)
    np.testing.assert_allclose(out3, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse3, lse, rtol=1e-13)


def test_duplicating_every_column_adds_ln2_to_lse():
    p = inputs.random_problem(8, 2, 16, 24, pool_rows=300, neg_frac=0.1)
    out, lse = oracle.decode_exact(p)
    d = dict(p)
    d["indices"] = np.concatenate([p["indices"], p["indices"]], axis=1)
    d["lens"] = p["lens"] * 2
    d["split_col"] = 48
    out2, lse2 = oracle.decode_exact(d)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse + LN2, rtol=1e-13)


def test_single_active_column_returns_its_row():
    p = inputs.random_problem(9, 1, 16, 8, pool_rows=64, lens=1, row_bytes=576)
    out, lse = oracle.decode_exact(p)
    row = _e4m3_f64(p["kv_a"][p["indices"][0, 0]]).numpy()
    for h in range(16):
        assert np.array_equal(out[h], p["bmm2"] * row[:512])
    s = p["bmm1"] * (_e4m3_f64(p["q"][0]).numpy() @ row)
    np.testing.assert_allclose(lse, s, rtol=1e-13, atol=1e-13)


def test_equal_scores_give_the_mean_row_and_weights_sum_to_one():
    p = inputs.random_problem(10, 1, 16, 20, pool_rows=100, sinks=True)
    p["q"] = np.zeros_like(p["q"])  # every score 0
    out, lse = oracle.decode_exact(p)
    rows = _e4m3_f64(p["kv_a"][p["indices"][0]]).numpy()[:, :512]
    sinks = p["sinks"].astype(np.float64)
    for h in range(16):
        z = 20.0 + math.exp(sinks[h])
        np.testing.assert_allclose(out[h], p["bmm2"] * rows.sum(0) / z, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(lse[h], math.log(z), rtol=1e-14)
    # all-ones V: out = bmm2 * (1 - sink weight) with the sink weight e^{sink - lse}
    p2 = inputs.random_problem(12, 2, 16, 20, pool_rows=100, sinks=True, lens=[20, 9])
    p2["kv_a"] = p2["kv_a"].copy()
    p2["kv_a"][:, :512] = 0x38  # E4M3 1.0
    out2, lse2 = oracle.decode_exact(p2)
    sink_w = np.exp(np.tile(p2["sinks"].astype(np.float64), 2) - lse2)
    np.testing.assert_allclose(out2, (p2["bmm2"] * (1 - sink_w))[:, None] * np.ones((1, 512)),
                               rtol=1e-12)


@pytest.mark.parametrize("case", ["lens0", "all_neg", "lens_negative"])
def test_zero_count_rule_is_exact(case):
    p = inputs.random_problem(13, 3, 16, 16, pool_rows=64, sinks=True)
    if case == "lens0":
        p["lens"] = np.array([16, 0, 16], np.int32)
    elif case == "all_neg":
        p["indices"] = p["indices"].copy()
        p["indices"][1] = -1
    else:
        p["lens"] = np.array([16, -5, 16], np.int32)
    out, lse = oracle.decode_exact(p)
    assert np.array_equal(out[16:32], np.zeros((16, 512)))
    assert not np.signbit(out[16:32]).any()
    assert np.all(lse[16:32] == -np.inf)
    assert np.all(np.isfinite(lse[:16])) and np.all(np.isfinite(lse[32:]))
    om, lm = oracle.decode_mimic(p, splits=2, chunk=8, terms=2)
    assert np.array_equal(om[16:32], np.zeros((16, 512))) and np.all(lm[16:32] == -np.inf)


def test_out_of_range_and_nan_inputs_are_rejected():
    p = inputs.random_problem(14, 1, 16, 8, pool_rows=32, poison=False)
    bad = dict(p)
    bad["indices"] = p["indices"].copy()
    bad["indices"][0, 3] = 32
    with pytest.raises(oracle.OracleError):
        oracle.decode_exact(bad)
    nan = dict(p)
    nan["kv_a"] = p["kv_a"].copy()
    nan["kv_a"][p["indices"][0, 2], 5] = 0x7F
    with pytest.raises(oracle.OracleError):
        oracle.decode_exact(nan)
    # an index past lens, or a poisoned row that is never active, is never read
    ok = dict(p)
    ok["indices"] = p["indices"].copy()
    ok["lens"] = np.array([5], np.int32)
    ok["indices"][0, 6] = 10 ** 6
    oracle.decode_exact(ok)


# ---------------------------------------------------------------------------
# mimic mode
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("splits,chunk", [(1, 64), (3, 8), (4, 5), (7, 128)])
def test_mimic_without_quantization_is_exact(splits, chunk):
    p = inputs.random_problem(15, 2, 16, 40, pool_rows=300, neg_frac=0.2, lens=[40, 23],
                              sinks=True)
    out, lse = oracle.decode_exact(p)
    om, lm = oracle.decode_mimic(p, splits=splits, chunk=chunk, quantize=False)
    np.testing.assert_allclose(om, out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lm, lse, rtol=1e-12)


def test_mimic_single_chunk_matches_recipe_with_torch_quantizer():
    """One split, one chunk: P = 2^(s2 - max + log2 448) quantized by torch's E4M3 cast."""
    p = inputs.random_problem(16, 1, 16, 32, pool_rows=200)
    rows = _e4m3_f64(p["kv_a"][p["indices"][0]]).numpy()
    q = _e4m3_f64(p["q"][0]).numpy()
    s2 = p["bmm1"] * (q @ rows[:, :576].T) / LN2  # [H, n]
    m = s2.max(axis=1, keepdims=True)
    pv = np.exp2(s2 - m + math.log2(448.0))
    for terms in (1, 2):
        hi = torch.from_numpy(pv).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
        phat = hi.numpy()
        if terms == 2:
            res = torch.from_numpy(16 * (pv - phat)).clamp(-448, 448).to(torch.float8_e4m3fn)
            phat = phat + res.to(torch.float64).numpy() / 16
        ref = p["bmm2"] * (phat @ rows[:, :512]) / pv.sum(1, keepdims=True)
        ref_lse = (m[:, 0] - math.log2(448.0) + np.log2(pv.sum(1))) * LN2
        om, lm = oracle.decode_mimic(p, splits=1, chunk=32, terms=terms)
        np.testing.assert_allclose(om, ref, rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(lm, ref_lse, rtol=1e-12)


def test_mimic_equal_scores_quantize_exactly():
    """Equal scores put every P at the anchor 448, which E4M3 holds exactly."""
    p = inputs.random_problem(17, 1, 16, 40, pool_rows=100)
    p["q"] = np.zeros_like(p["q"])
    out, lse = oracle.decode_exact(p)
    om, lm = oracle.decode_mimic(p, splits=1, chunk=64, terms=1)
    np.testing.assert_allclose(om, out, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lm, lse, rtol=1e-13)


def test_mimic_two_terms_is_much_closer_than_one():
    p = inputs.random_problem(18, 2, 16, 128, pool_rows=600)
    out, _ = oracle.decode_exact(p)
    e1 = np.linalg.norm(oracle.decode_mimic(p, 2, 64, terms=1)[0] - out) / np.linalg.norm(out)
    e2 = np.linalg.norm(oracle.decode_mimic(p, 2, 64, terms=2)[0] - out) / np.linalg.norm(out)
    assert 2e-3 < e1 < 5e-2  # E4M3's 3 mantissa bits: percent-level per P
    assert e2 < e1 / 16


def test_mimic_lse_ignores_p_quantization():
    """The running sums use the unquantized P, so the LSE matches exact mode closely."""
    p = inputs.random_problem(19, 2, 16, 64, pool_rows=300, sinks=True, neg_frac=0.1)
    _, lse = oracle.decode_exact(p)
    _, lm = oracle.decode_mimic(p, 3, 16, terms=1)
    np.testing.assert_allclose(lm, lse, rtol=1e-12)


def _one_head_problem(dots, marker_row, marker_col, c=2.0 / 3.0):
    """One head, q = e_0, row r = dots[r] at column 0 (and 448 at marker_col of marker_row):
    base-2 score of row r = c * dots[r]."""
    def e4(x):
        return int(torch.tensor([x], dtype=torch.float64).to(torch.float8_e4m3fn)
                   .view(torch.uint8)[0])
    n = len(dots)
    q = np.zeros((1, 1, 576), np.uint8)
    q[0, 0, 0] = e4(1.0)
    kv = np.zeros((n, 576), np.uint8)
    for r, x in enumerate(dots):
        assert float(torch.tensor([x]).to(torch.float8_e4m3fn).to(torch.float64)[0]) == x
        kv[r, 0] = e4(x)
    kv[marker_row, marker_col] = e4(448.0)
    return dict(q=q, kv_a=kv, kv_b=None, split_col=n, qk_dim=576,
                indices=np.arange(n, dtype=np.int32)[None], lens=np.array([n], np.int32),
                sinks=None, bmm1=c * LN2, bmm2=1.0)


def test_mimic_recipe_worked_example_with_rescale():
    """Hand-worked recipe (attn_sparse page, module docstring: P at 448 of the running maximum,
    E4M3, unquantized sums, rescale when the maximum rises), one head, chunks of one column,
    base-2 scores 3/2, 0, 3 (dot products 2.25, 0, 4.5 at 2/3 per unit); only the second row
    has latent column 100 = 448.
      chunk 0: m = 3/2, P = 448 (exact), l = 448.
      chunk 1: m = 3/2, P = 448 * 2^-1.5 = 158.392 -> E4M3 160 (the grid step is 16 on
               [128, 256)); l = 606.392.
      chunk 2: m = 3, alpha = 2^-1.5 rescales acc and l; P = 448 (exact).
    So out[100] = 160 * 448 * 2^-1.5 / L and out[0] = (448 * 2.25 * 2^-1.5 + 448 * 4.5) / L,
    L = 606.392 * 2^-1.5 + 448; LSE2 = 3 - log2(448) + log2(L).  Two terms: the second term is
    E4M3(16 (158.392 - 160)) = E4M3(-25.73) = -26 (step 2 on [16, 32)), so P = 160 - 26/16."""
    p = _one_head_problem([2.25, 0.0, 4.5], 1, 100)
    r = 2.0 ** -1.5
    p1 = 448.0 * r
    L = (448.0 + p1) * r + 448.0
    out, lse = oracle.decode_mimic(p, splits=1, chunk=1, terms=1, lse_log2=True)
    assert abs(out[0, 100] - 160.0 * 448.0 * r / L) < 1e-12
    assert abs(out[0, 0] - (448.0 * 2.25 * r + 448.0 * 4.5) / L) < 1e-12
    assert abs(lse[0] - (3.0 - math.log2(448.0) + math.log2(L))) < 1e-12
    out2, _ = oracle.decode_mimic(p, splits=1, chunk=1, terms=2, lse_log2=True)
    assert abs(out2[0, 100] - (160.0 - 26.0 / 16.0) * 448.0 * r / L) < 1e-12
    # one chunk of three columns anchors all three at the final maximum: P = 448 * 2^-1.5
    # = 158.392 -> 160 for the first row as well, 448 * 2^-3 = 56 (exact) for the second
    out3, _ = oracle.decode_mimic(p, splits=1, chunk=3, terms=1, lse_log2=True)
    L3 = p1 + 56.0 + 448.0
    assert abs(out3[0, 100] - 56.0 * 448.0 / L3) < 1e-12
    assert abs(out3[0, 0] - (160.0 * 2.25 + 448.0 * 4.5) / L3) < 1e-12


def test_mimic_recipe_underflowing_rescale():
    """A maximum that rises by more than the FP64 exponent range underflows alpha to zero:
    base-2 scores 0 and 1120 (dot products 0 and 448 at c = 2.5): everything before the rise
    is weighted 2^-1120 (zero in double), so the output is the second row and the LSE its
    score; exact mode agrees."""
    p = _one_head_problem([0.0, 448.0], 0, 200, c=2.5)
    out, lse = oracle.decode_mimic(p, splits=1, chunk=1, terms=1, lse_log2=True)
    assert out[0, 200] == 0.0  # alpha = 0: the first row's contribution is gone
    assert abs(out[0, 0] / 448.0 - 1.0) < 1e-13
    assert abs(lse[0] / 1120.0 - 1.0) < 1e-13
    ex, ex_lse = oracle.decode_exact(p, lse_log2=True)
    assert ex[0, 200] == 0.0
    assert abs(ex[0, 0] / 448.0 - 1.0) < 1e-13 and abs(ex_lse[0] / 1120.0 - 1.0) < 1e-13


def test_mimic_anchor_holds_the_running_max_exactly():
    """Every chunk whose maximum is the running maximum quantizes that P to exactly 448, so a
    row that holds the running maximum in every chunk (scores rising chunk by chunk) carries no
    quantization error: with chunks of one column the recipe equals exact mode."""
    p = _one_head_problem([0.0, 1.0, 2.5, 4.0, 7.0, 12.0], 5, 300, c=1.0)
    for terms in (1, 2):
        out, lse = oracle.decode_mimic(p, splits=1, chunk=1, terms=terms)
        ex, ex_lse = oracle.decode_exact(p)
        np.testing.assert_allclose(out, ex, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse, ex_lse, rtol=1e-13)
    # falling scores: every later P is below the anchor and rounds
    p = _one_head_problem([12.0, 7.0, 4.0, 2.5, 1.0, 0.0], 5, 300, c=1.0)
    out, _ = oracle.decode_mimic(p, splits=1, chunk=1, terms=1)
    ex, _ = oracle.decode_exact(p)
    assert np.abs(out - ex).max() > 1e-6


# ---------------------------------------------------------------------------
# chunk-local mode (the sparse_mla_cute page, "How.": one softmax per 128-column chunk at the
# chunk's own maximum, P = 256 exp2(S - m_c) as FP8, chunks merged by exp2(m_c - M) / L)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("width", [128, 7, 1])
def test_chunk_local_without_quantization_is_exact(width):
    p = inputs.random_problem(40, 3, 16, 300, pool_rows=900, neg_frac=0.2, lens=[300, 129, 0],
                              sinks=True, two_pools=True, split_col=128, rows_b=700)
    out, lse = oracle.decode_exact(p)
    oc, lc = oracle.decode_chunk_local(p, width=width, quantize=False)
    np.testing.assert_allclose(oc, out, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(lc[np.isfinite(lse)], lse[np.isfinite(lse)], rtol=1e-12)
    assert np.all(oc[~np.isfinite(lse)] == 0) and np.all(lc[~np.isfinite(lse)] == -np.inf)


def test_chunk_local_is_the_lse_merge_of_its_chunks():
    """Each chunk's output is its own quantized P.V over its own unquantized sum, so decoding
    every chunk alone (the other columns masked) and combining the results by their LSEs
    (out = sum_k 2^(lse_k - M) out_k / sum_k 2^(lse_k - M), lse = M + log2 sum_k 2^(lse_k - M))
    gives the whole call, P rounding included; a mistake in a chunk's weight, its maximum, the
    anchor's place in the LSE or the chunk boundaries breaks the identity."""
    p = inputs.random_problem(41, 2, 16, 300, pool_rows=900, neg_frac=0.1, lens=[300, 200])
    for terms in (1, 2):
        whole, whole_lse = oracle.decode_chunk_local(p, terms=terms, lse_log2=True)
        outs, lses = [], []
        for lo in (0, 128, 256):
            q = dict(p)
            idx = np.full_like(p["indices"], -1)
            idx[:, lo:lo + 128] = p["indices"][:, lo:lo + 128]
            q["indices"] = idx
            o, l = oracle.decode_chunk_local(q, terms=terms, lse_log2=True)
            outs.append(o)
            lses.append(l)
        lses = np.stack(lses)                   # [3, T*H]
        top = lses.max(axis=0)
        wgt = np.where(np.isfinite(lses), np.exp2(lses - top), 0.0)
        merged = (wgt[:, :, None] * np.stack(outs)).sum(axis=0) / wgt.sum(axis=0)[:, None]
        np.testing.assert_allclose(merged, whole, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(top + np.log2(wgt.sum(axis=0)), whole_lse, rtol=1e-12)


def _rows_problem(dots, markers, c=2.0 / 3.0):
    """One head, q = e_0, row r holds dots[r] at column 0 (base-2 score c * dots[r]) and 448 at
    column col for each (row, col) in markers."""
    def e4(x):
        return int(torch.tensor([x], dtype=torch.float64).to(torch.float8_e4m3fn)
                   .view(torch.uint8)[0])
    n = len(dots)
    q = np.zeros((1, 1, 576), np.uint8)
    q[0, 0, 0] = e4(1.0)
    kv = np.zeros((n, 576), np.uint8)
    for r, x in enumerate(dots):
        kv[r, 0] = e4(x)
    for r, col in markers:
        kv[r, col] = e4(448.0)
    return dict(q=q, kv_a=kv, kv_b=None, split_col=n, qk_dim=576,
                indices=np.arange(n, dtype=np.int32)[None], lens=np.array([n], np.int32),
                sinks=None, bmm1=c * LN2, bmm2=1.0)


def test_chunk_local_worked_example():
    """Hand-worked chunk-local recipe, chunks of two columns, base-2 scores 3, 2.5 | 1.5, 0.5
    (dot products 4.5, 3.75, 2.25, 0.75 at 2/3 per unit); row 1 has 448 at column 100, row 3
    at column 200.
      chunk 0: m = 3: P = 256 (exact), 256 * 2^-0.5 = 181.019 -> E4M3 176 (grid step 16 on
               [128, 256)); l_0 = 437.019.
      chunk 1: its own m = 1.5: P = 256, 128 (both exact); l_1 = 384; weight 2^(1.5 - 3).
    L = 437.019 + 384 * 2^-1.5 = 572.784; out[100] = 176 * 448 / L; out[200] = 128 * 2^-1.5
    * 448 / L (a running maximum would have rounded that P: 256 * 2^-2.5 = 45.25 -> 44);
    LSE2 = 3 - log2(256) + log2(L).  At anchor 448 row 1's P is 448 * 2^-0.5 = 316.78 -> 320
    (step 32).  Two terms: E4M3(16 (181.019 - 176)) = E4M3(80.31) = 80, so P = 176 + 5."""
    p = _rows_problem([4.5, 3.75, 2.25, 0.75], [(1, 100), (3, 200)])
    r = 2.0 ** -1.5
    p1 = 256.0 * 2.0 ** -0.5
    L = 256.0 + p1 + 384.0 * r
    out, lse = oracle.decode_chunk_local(p, width=2, terms=1, lse_log2=True)
    assert abs(out[0, 100] - 176.0 * 448.0 / L) < 1e-12
    assert abs(out[0, 200] - 128.0 * r * 448.0 / L) < 1e-12
    assert abs(out[0, 0] - (256.0 * 4.5 + 176.0 * 3.75 + r * (256.0 * 2.25 + 128.0 * 0.75)) / L) \
        < 1e-12
    assert abs(lse[0] - (3.0 - 8.0 + math.log2(L))) < 1e-12
    out2, _ = oracle.decode_chunk_local(p, width=2, terms=2, lse_log2=True)
    assert abs(out2[0, 100] - 181.0 * 448.0 / L) < 1e-12
    out448, _ = oracle.decode_chunk_local(p, width=2, anchor=448.0, terms=1, lse_log2=True)
    L448 = (256.0 + p1 + 384.0 * r) * 448.0 / 256.0
    assert abs(out448[0, 100] - 320.0 * 448.0 / L448) < 1e-12
    # the attn_sparse recipe (running maximum over chunks of two) rounds row 3's P
    om, _ = oracle.decode_mimic(p, splits=1, chunk=2, anchor=256.0, terms=1, lse_log2=True)
    assert abs(om[0, 200] - 44.0 * 448.0 / L) < 1e-12


def test_chunk_local_single_chunk_matches_recipe_with_torch_quantizer():
    """One chunk: P = 256 * 2^(s2 - max) quantized by torch's E4M3 cast, over the unquantized
    sum."""
    p = inputs.random_problem(42, 1, 16, 100, pool_rows=200)
    rows = _e4m3_f64(p["kv_a"][p["indices"][0]]).numpy()
    q = _e4m3_f64(p["q"][0]).numpy()
    s2 = p["bmm1"] * (q @ rows[:, :576].T) / LN2
    m = s2.max(axis=1, keepdims=True)
    pv = np.exp2(s2 - m + 8.0)
    phat = torch.from_numpy(pv).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    ref = p["bmm2"] * (phat @ rows[:, :512]) / pv.sum(1, keepdims=True)
    ref_lse = (m[:, 0] - 8.0 + np.log2(pv.sum(1))) * LN2
    oc, lc = oracle.decode_chunk_local(p, terms=1)
    np.testing.assert_allclose(oc, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lc, ref_lse, rtol=1e-13)


def test_chunk_local_zero_count_rule():
    p = inputs.random_problem(43, 2, 16, 140, pool_rows=300, lens=[0, 140])
    p["indices"][1, :] = -1
    out, lse = oracle.decode_chunk_local(p)
    assert np.all(out == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------------------
# 656-byte fp8_ds_mla rows (E4M3 latent with an FP32 scale per 128 elements, BF16 rope)
# ---------------------------------------------------------------------------

def _ds_rows_f64(rows):
    """Materialize fp8_ds_mla rows [n, 656] as K [n, 576] in float64 with numpy and torch
    casts (a path independent of the oracle's decoder)."""
    rows = np.ascontiguousarray(rows)
    lat = _e4m3_f64(rows[:, :512]).numpy()
    scale = rows[:, 512:528].copy().view(np.float32).astype(np.float64)
    rope = torch.from_numpy(rows[:, 528:656].copy().view(np.int16)).view(torch.bfloat16)
    k = np.empty((rows.shape[0], 576))
    k[:, :512] = lat * np.repeat(scale, 128, axis=1)
    k[:, 512:] = rope.to(torch.float64).numpy()
    return k


def test_ds_mla_exact_matches_dense_attention_on_materialized_rows():
    p = inputs.random_problem(44, 2, 16, 90, pool_rows=300, row_bytes=656, neg_frac=0.2,
                              lens=[90, 41], sinks=True)
    out, lse = oracle.decode_exact(p)
    q = _e4m3_f64(p["q"]).numpy()
    for t in range(2):
        n = int(p["lens"][t])
        cols = [c for c in range(n) if p["indices"][t, c] >= 0]
        k = _ds_rows_f64(p["kv_a"][p["indices"][t, cols]])
        s = p["bmm1"] * (q[t] @ k.T)                     # [H, n]
        s = np.concatenate([s, p["sinks"].astype(np.float64)[:, None]], axis=1)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        ref = p["bmm2"] * (e[:, :-1] @ k[:, :512]) / e.sum(1, keepdims=True)
        np.testing.assert_allclose(out[t * 16:(t + 1) * 16], ref, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[t * 16:(t + 1) * 16],
                                   m[:, 0] + np.log(e.sum(1)), rtol=1e-12)


def test_ds_mla_rows_with_unit_scales_equal_the_576_byte_rows():
    """A 656-byte row whose scales are 1 and whose BF16 rope holds the E4M3 rope's values (exact
    in BF16) is the same row as the 576-byte one: every mode gives the same result."""
    p = inputs.random_problem(45, 2, 16, 200, pool_rows=400, neg_frac=0.1, lens=[200, 150],
                              sinks=True)
    kv = p["kv_a"]
    ds = np.zeros((kv.shape[0], 656), np.uint8)
    ds[:, :512] = kv[:, :512]
    ds[:, 512:528] = np.ones((kv.shape[0], 4), np.float32).view(np.uint8)
    rope = _e4m3_f64(kv[:, 512:576]).numpy()
    ds[:, 528:656] = inputs.bf16_bits(rope.astype(np.float32)).view(np.uint8).reshape(-1, 128)
    pd = dict(p, kv_a=ds)
    for f in (lambda x: oracle.decode_exact(x),
              lambda x: oracle.decode_mimic(x, splits=3, chunk=64, terms=2),
              lambda x: oracle.decode_chunk_local(x)):
        a, la = f(p)
        b, lb = f(pd)
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(la, lb)


def test_ds_mla_rows_quantize_each_block_at_its_own_scale():
    """The generator's rows: each 128-element block's largest magnitude encodes as 448 times its
    scale, so a block scaled by 2^k gets a scale 2^k larger and the same bytes."""
    rng = np.random.default_rng(46)
    lat = rng.standard_normal((3, 512)).astype(np.float32)
    lat2 = lat.copy()
    lat2[:, 128:256] *= 8.0
    a = inputs.ds_mla_rows(lat, np.zeros((3, 64)))
    b = inputs.ds_mla_rows(lat2, np.zeros((3, 64)))
    np.testing.assert_array_equal(a[:, :512], b[:, :512])
    sa, sb = a[:, 512:528].copy().view(np.float32), b[:, 512:528].copy().view(np.float32)
    np.testing.assert_array_equal(sb[:, 1], 8 * sa[:, 1])
    np.testing.assert_array_equal(sb[:, [0, 2, 3]], sa[:, [0, 2, 3]])
    k = _ds_rows_f64(a)
    for blk in range(4):
        assert np.abs(k[:, 128 * blk:128 * (blk + 1)]).max(axis=1) == pytest.approx(
            np.abs(lat[:, 128 * blk:128 * (blk + 1)]).max(axis=1), rel=1e-6)


# ---------------------------------------------------------------------------
# lse_merge
# ---------------------------------------------------------------------------

def _bf16_to_f64(bits):
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


def test_merge_single_source_is_identity():
    m = inputs.random_merge(20, 1, 3, 8, 64, empty_frac=0.3)
    out, lse = oracle.lse_merge(m["partials"], m["lse"])
    valid = np.isfinite(m["lse"][0])
    np.testing.assert_array_equal(out[valid], _bf16_to_f64(m["partials"][0])[valid])
    np.testing.assert_allclose(lse[valid], m["lse"][0][valid].astype(np.float64) * LN2, rtol=1e-15)
    assert np.all(out[~valid] == 0) and np.all(lse[~valid] == -np.inf)


def test_merge_closed_form_two_sources():
    x = inputs.bf16_bits(np.array([[[[1.0, 2.0]]], [[[3.0, -4.0]]]], np.float32))
    lse = np.array([[[2.0]], [[3.0]]], np.float32)  # base 2: weights 1/3 and 2/3
    out, l = oracle.lse_merge(x, lse, lse_log2=True)
    np.testing.assert_allclose(out[0, 0], [1 / 3 + 2.0, 2 / 3 - 8 / 3], rtol=1e-15)
    np.testing.assert_allclose(l[0, 0], 3.0 + math.log2(1.5), rtol=1e-15)


def test_merge_empty_encodings_and_nan_partials_do_not_propagate():
    m = inputs.random_merge(21, 5, 4, 8, 32, empty_frac=0.4, nan_lse=True)
    out, lse = oracle.lse_merge(m["partials"], m["lse"])
    assert np.all(np.isfinite(out))
    none = ~np.isfinite(m["lse"]).any(axis=0)
    assert none[0, 0]
    assert np.all(out[none] == 0) and np.all(lse[none] == -np.inf)
    assert np.all(np.isfinite(lse[~none]))


def test_merge_recovers_full_decode_from_two_column_ranges():
    """Decoding columns [0,k) and [k,n) separately (base-2 LSE), rounding to BF16, and merging
    gives the full decode within BF16 rounding; this also cross-checks exact mode against the
    merge."""
    p = inputs.random_problem(22, 2, 16, 64, pool_rows=400, neg_frac=0.1)
    full, full_lse = oracle.decode_exact(p)
    parts, lses = [], []
    for lo, hi in ((0, 25), (25, 64)):
        q = dict(p)
        idx = np.full_like(p["indices"], -1)
        idx[:, lo:hi] = p["indices"][:, lo:hi]
        q["indices"] = idx
        o, l = oracle.decode_exact(q, lse_log2=True)
        parts.append(inputs.bf16_bits(o.reshape(2, 16, 512).astype(np.float32)))
        lses.append(l.reshape(2, 16).astype(np.float32))
    out, lse = oracle.lse_merge(np.stack(parts), np.stack(lses))
    err = np.linalg.norm(out.reshape(-1, 512) - full) / np.linalg.norm(full)
    assert err < 4e-3
    np.testing.assert_allclose(lse.reshape(-1), full_lse, rtol=1e-6)


def test_dominant_sink_does_not_overflow():
    """A sink far above every score: the stabiliser m must include the sink, the output goes
    to ~0 and the LSE to the sink (closed form ln(e^sink + sum e^s) ~ sink)."""
    p = inputs.random_problem(23, 1, 16, 16, pool_rows=64, sinks=True)
    p["sinks"] = np.full(16, 800.0, np.float32)
    out, lse = oracle.decode_exact(p)
    assert np.all(np.isfinite(lse)) and np.all(np.isfinite(out))
    np.testing.assert_allclose(lse, 800.0, rtol=1e-12)
    assert np.abs(out).max() < 1e-300
    om, lm = oracle.decode_mimic(p, 2, 8, terms=1)
    np.testing.assert_allclose(lm, 800.0, rtol=1e-12)
    assert np.all(np.isfinite(om)) and np.abs(om).max() < 1e-300


# ---------------------------------------------------------------------------
# mla_value: LSE merge, W_UV and the sigmoid gate (dcp page, DcpValue.merge)
# ---------------------------------------------------------------------------

def _bf16(x):
    return torch.as_tensor(np.asarray(x, np.float32)).to(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def _value_problem(seed, S, T, H, empty_frac=0.2):
    m = inputs.random_merge(seed, S, T, H, 512, empty_frac=empty_frac)
    rng = np.random.default_rng(seed + 1)
    w = _bits(_bf16(rng.standard_normal((H, 512, 128)) / 16.0))
    g = _bits(_bf16(rng.standard_normal((T, H * 128)) * 2.0))
    return m["partials"], m["lse"], w, g


def test_mla_value_matches_torch_float64():
    """The merge weights, the BF16 latent, a float64 matmul with W_UV, BF16, times torch's
    sigmoid of the gate, BF16 (torch on the CPU, independent of the oracle's loops): equal up
    to one BF16 step where torch's float64 -> BF16 cast rounds twice (through float32)."""
    x, l2, w, g = _value_problem(800, 3, 5, 4)
    got = oracle.mla_value(x, l2, w, g)
    xs = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double()  # [S,T,H,512]
    ls = torch.from_numpy(l2).double()
    fin = torch.isfinite(ls)
    top = torch.where(fin, ls, torch.tensor(-np.inf, dtype=torch.float64)).amax(0)
    wts = torch.where(fin, torch.exp2(ls - top), torch.zeros_like(ls))
    wts = wts / wts.sum(0).clamp_min(1e-300)
    lat = (wts[..., None] * torch.nan_to_num(xs)).sum(0).to(torch.bfloat16).double()
    W = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double()   # [H,512,128]
    acc = torch.einsum("thk,hkv->thv", lat, W)
    G = torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).double().reshape(5, 4, 128)
    ref = (acc.to(torch.bfloat16).double() * torch.sigmoid(G)).to(torch.bfloat16).double()
    ref = ref.reshape(5, 512).numpy()
    diff = np.abs(got - ref)
    step = np.abs(ref) * 2.0 ** -7 + 1e-30
    assert np.all(diff <= step)
    assert (diff == 0).mean() > 0.99


def test_mla_value_selection_weights_and_gates_in_closed_form():
    """W_UV picking latent column v + 32 h for value v (one product with 1) reproduces the merged
    BF16 latent; a gate of 30 (sigmoid 1 - 9e-14) leaves it unchanged after BF16 rounding, a
    gate of 0 halves it exactly.  One source with a finite LSE merges to itself."""
    S, T, H = 1, 3, 2
    rng = np.random.default_rng(801)
    x = _bits(_bf16(rng.standard_normal((S, T, H, 512))))
    l2 = np.full((S, T, H), 3.5, np.float32)
    w = np.zeros((H, 512, 128), np.uint16)
    one = _bits(_bf16([1.0]))[0]
    for h in range(H):
        w[h, np.arange(128) + 32 * h, np.arange(128)] = one
    xv = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()[0]
    for gval, factor in ((30.0, 1.0), (0.0, 0.5)):
        g = _bits(_bf16(np.full((T, H * 128), gval)))
        got = oracle.mla_value(x, l2, w, g).reshape(T, H, 128)
        for h in range(H):
            np.testing.assert_array_equal(got[:, h], xv[:, h, 32 * h:32 * h + 128] * factor)


def test_mla_value_padded_rows_are_zero_and_empty_sources_merge_to_zero():
    """Rows of a request whose total is 0 are zeros even when their gate is NaN (two rows per
    request here); a live row whose sources are all empty merges to a zero latent, so its
    values are 0 * sigmoid(gate) = 0."""
    x, l2, w, g = _value_problem(802, 2, 6, 2, empty_frac=0.0)
    totals = np.array([5, 0, 7], np.int32)             # rows 2, 3 padded
    g[2:4] = _bits(_bf16([np.nan]))[0]
    l2[:, 4, :] = -np.inf                               # row 4: every source empty
    x[:, 4, :, :] = 0x7FC0                              # (never read)
    out = oracle.mla_value(x, l2, w, g, totals=totals, rows_per_request=2)
    assert np.all(out[2:4] == 0.0)
    assert np.all(out[4] == 0.0)
    assert np.all(np.isfinite(out)) and np.any(out[0] != 0.0)


# ---------------------------------------------------------------------------
# paged decode (dcp page, stock_decode)
# ---------------------------------------------------------------------------

def test_paged_equals_sparse_over_the_materialized_rows():
    """The paged oracle on a block table equals the (independently pinned) sparse exact mode
    over the same rows listed as indices with the causal counts."""
    p = inputs.paged_problem(60, 3, 4, 16, [150, 3, 64], page_size=16)
    out, lse = oracle.paged_decode_exact(p)
    ref, ref_lse = oracle.decode_exact(inputs.paged_as_sparse(p))
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(np.isfinite(lse), np.isfinite(ref_lse))
    fin = np.isfinite(lse)
    np.testing.assert_allclose(lse[fin], ref_lse[fin], rtol=1e-13)


def test_paged_causal_mask_matches_sdpa():
    """float64 scaled-dot-product attention over each request's materialized context with the
    causal offset mask (row i of q_len sees keys < length - (q_len - 1 - i))."""
    p = inputs.paged_problem(61, 2, 3, 16, [40, 9], page_size=8, poison=False)
    out, lse = oracle.paged_decode_exact(p)
    cache = _e4m3_f64(p["cache"]).numpy()
    q = _e4m3_f64(p["q"]).numpy()
    H = 16
    for b in range(2):
        L = int(p["lengths"][b])
        rows = np.stack([cache[p["block_table"][b, k // 8], k % 8] for k in range(L)])
        K = torch.from_numpy(rows[:, :576])
        V = torch.from_numpy(rows[:, :512])
        Q = torch.from_numpy(q[3 * b:3 * b + 3])                   # [3, H, 576]
        mask = torch.full((3, L), float("-inf"), dtype=torch.float64)
        for i in range(3):
            mask[i, :L - (3 - 1 - i)] = 0.0
        for h in range(H):
            o = torch.nn.functional.scaled_dot_product_attention(
                Q[:, h][None], K[None], V[None], attn_mask=mask[None], scale=p["bmm1"])[0]
            ls = torch.logsumexp(p["bmm1"] * (Q[:, h] @ K.T) + mask, dim=1)
            for i in range(3):
                u = (3 * b + i) * H + h
                np.testing.assert_allclose(out[u], p["bmm2"] * o[i].numpy(), rtol=1e-10,
                                           atol=1e-12)
                assert abs(lse[u] - float(ls[i])) < 1e-10


def test_paged_rows_without_keys_are_zero_and_lse_minus_inf():
    """A request with fewer keys than query rows leaves its early rows without keys; a request
    with length 0 has none at all: +0.0 output and LSE -inf."""
    p = inputs.paged_problem(62, 2, 4, 16, [2, 0], page_size=16)
    out, lse = oracle.paged_decode_exact(p)
    # request 0 (length 2): rows i = 0, 1 see 2 - (3 - i) <= 0 keys; rows 2, 3 see 1 and 2
    for t in (0, 1, 4, 5, 6, 7):
        assert np.all(out[t * 16:(t + 1) * 16] == 0.0)
        assert np.all(lse[t * 16:(t + 1) * 16] == -np.inf)
    assert np.all(np.isfinite(lse[2 * 16:4 * 16]))
