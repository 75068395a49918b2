"""Parity of mla_value (the split merge, W_UV and the sigmoid gate; dcp page, DcpValue.merge)
with the FP64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_amd as smla
from sparse_mla_attention_amd import inputs
from smla_testlib import bf16_to_f64, dev, log, rel_l2

pytestmark = pytest.mark.gpu


def _run(v, use_totals=True):
    x = dev(v["partials"]).view(torch.bfloat16)
    l2 = dev(v["lse"])
    S, T, H, _ = v["partials"].shape
    w_t = dev(v["w_uv_t"]).view(torch.bfloat16)           # [H, 128, 512]
    w = w_t.transpose(1, 2)                                # [H, 512, 128], latent stride 1
    g = dev(v["gate"]).view(torch.bfloat16)
    tot = dev(v["totals"]) if use_totals else None
    out = torch.full((T, H * 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    smla.mla_value(x, l2, w, g, out, totals=tot, rows_per_request=v["rows_per_request"])
    torch.cuda.synchronize()
    return bf16_to_f64(out)


def _check(v, label, use_totals=True):
    got = _run(v, use_totals)
    w = np.ascontiguousarray(np.transpose(v["w_uv_t"], (0, 2, 1)))  # [H, 512, 128]
    ref = oracle.mla_value(v["partials"], v["lse"], w, v["gate"],
                           totals=v["totals"] if use_totals else None,
                           rows_per_request=v["rows_per_request"])
    assert np.all(np.isfinite(got)), "a padded row's NaN gate leaked, or an empty source was read"
    diff = np.abs(got - ref)
    exact = float((diff == 0).mean())
    r = rel_l2(got, ref)
    log(f"  {label}: rel_l2={r:.3e} max_abs={diff.max():.3e} exact={exact:.4f}")
    # BF16 in, BF16 out.  The kernel merges the sources in FP32, the oracle in FP64, so a
    # merged latent value within rounding distance of a BF16 midpoint can round to the
    # neighbouring BF16 value on the two sides: one step (<= 2^-7 of |latent|, and |latent| <=
    # max |x_s| since the merge is a convex combination) times W_UV moves every value of the
    # (row, head) by up to max|W| 2^-7 max|x|.  The product and the gated result can then land
    # one BF16 step (2^-8 .. 2^-7 relative) apart as well.  Allowed: two latent flips plus two
    # result steps per element; rel-L2 and the exact fraction are held tight besides.
    xs = torch.from_numpy(v["partials"].view(np.int16)).view(torch.bfloat16).float().numpy()
    ws = torch.from_numpy(v["w_uv_t"].view(np.int16)).view(torch.bfloat16).float().numpy()
    live = np.isfinite(v["lse"])
    xmax = float(np.abs(np.where(live[..., None], np.nan_to_num(xs), 0.0)).max())
    atol = 2.0 * 2.0 ** -7 * float(np.abs(ws).max()) * xmax
    bad = diff > np.abs(ref) * 2.0 ** -6 + atol
    if bad.any():
        for t, c in np.argwhere(bad)[:5]:
            log(f"    t={t} col={c}: got {got[t, c]!r} ref {ref[t, c]!r}")
    assert not bad.any(), label
    assert r <= 4e-3 and exact >= 0.95, label
    return got, ref


def test_value_workload_shape():
    """8 sources, T=32, H=128 (the merge workload with W_UV [128, 512, 128] and gates)."""
    v = inputs.value_problem(900, 8, 32, 128)
    _check(v, "S=8 T=32 H=128")


@pytest.mark.parametrize("S,T,H,rpr,pad", [(1, 5, 4, 1, 0), (3, 37, 4, 2, 3), (17, 16, 2, 4, 1),
                                            (64, 3, 1, 1, 0)])
def test_value_shapes_padding_and_empty_sources(S, T, H, rpr, pad):
    v = inputs.value_problem(910 + S, S, T, H, empty_frac=0.3, padded_requests=pad,
                             rows_per_request=rpr)
    got, _ = _check(v, f"S={S} T={T} H={H} rows/request={rpr} padded={pad}")
    if pad:
        assert np.all(got[:pad * rpr] == 0.0), "padded rows must be zeros"


def test_value_without_totals_every_row_is_live():
    v = inputs.value_problem(920, 2, 9, 3)
    _check(v, "no totals", use_totals=False)


def test_value_rejects_bad_arguments():
    v = inputs.value_problem(930, 2, 4, 2)
    x = dev(v["partials"]).view(torch.bfloat16)
    w = dev(v["w_uv_t"]).view(torch.bfloat16).transpose(1, 2)
    g = dev(v["gate"]).view(torch.bfloat16)
    out = torch.empty((4, 256), dtype=torch.bfloat16, device="cuda")
    L = smla.library()
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = L.mla_value(P(x), P(dev(v["lse"])), 65, 4, 2, P(w), w.stride(0), w.stride(2), P(g),
                     None, 1, P(out), 0, None)
    assert st == smla.SMLA_EINVAL                    # S > 64
    st = L.mla_value(P(x), P(dev(v["lse"])), 2, 4, 2, P(w), w.stride(0), 3, P(g), None, 1,
                     P(out), 0, None)
    assert st == smla.SMLA_EINVAL                    # value stride not a multiple of 8
