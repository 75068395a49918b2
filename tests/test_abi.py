"""The C ABI without a GPU: the library loads, exports every function include/smla.h declares,
and the host-side checks reject bad arguments before anything touches the device."""
import ctypes

import pytest

import sparse_mla_attention_amd as smla


def _lib():
    import os
    if not os.path.exists(smla.LIB_PATH):  # nothing built yet: build it (hipcc cross-compiles)
        from sparse_mla_attention_amd import build
        build.build()
    return smla.library()


def test_exports_every_declared_function():
    L = _lib()
    names = smla.declared_functions()
    assert {"sparse_mla_decode", "lse_merge", "smla_decode_plan", "smla_decode_workspace_size",
            "smla_strerror"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/smla.h but not exported"


def test_strerror():
    L = _lib()
    for st in range(5):
        assert L.smla_strerror(st) not in (None, b"", b"unknown status")
    assert L.smla_strerror(99) == b"unknown status"


def test_workspace_size_formula():
    def expect(T, H, splits, tiles):
        groups = -(-((H + 31) // 32) // tiles)
        # status word, counters from byte 16, padded to 256
        counters = (16 + T * groups * 2 * 4 + 255) // 256 * 256
        # FP32 partials (512 per head) and FP32 (m, l) pairs
        return counters + T * groups * splits * 32 * tiles * (512 + 2) * 4
    for splits, tiles, T, H in [(2, 1, 7, 128), (3, 1, 7, 96), (64, 1, 3, 16), (5, 1, 2, 48),
                                (2, 2, 7, 128), (4, 2, 3, 64), (3, 2, 2, 48), (2, 2, 7, 96),
                                (2, 2, 1, 16)]:
        plan = smla.make_plan(splits, tiles)
        assert smla.workspace_size(plan, T, H) == expect(T, H, splits, tiles)
    assert smla.workspace_size(smla.make_plan(1, 1), 7, 128) == 0
    # bad plans and sizes report 0
    assert smla.workspace_size(smla.make_plan(0, 1), 7, 128) == 0
    assert smla.workspace_size(smla.make_plan(65, 1), 7, 128) == 0
    assert smla.workspace_size(smla.make_plan(2, 4), 7, 128) == 0   # 1 or 2 tiles per WG
    assert smla.workspace_size(smla.make_plan(2, 1), 7, 120) == 0   # H % 16 != 0
    # fewer real heads per 64-head workgroup: ceil(H / heads) groups
    for heads, T, H in [(16, 5, 128), (32, 3, 96), (16, 2, 48)]:
        groups = -(-H // heads)
        counters = (16 + T * groups * 2 * 4 + 255) // 256 * 256
        plan = smla.make_plan(4, 2, heads=heads)
        assert smla.workspace_size(plan, T, H) == counters + T * groups * 4 * 64 * (512 + 2) * 4
        assert smla.workspace_header_bytes(plan, T, H) == counters
    for tiles, heads in [(1, 16), (2, 48), (2, 8), (1, 64)]:     # not a kernel's width
        assert smla.workspace_size(smla.make_plan(2, tiles, heads=heads), 7, 128) == 0


def _decode(T=1, H=16, W=64, row_bytes=576, qk_dim=576, flags=0, plan=None, q=16, kv=16,
            idx=16, lens=16, out=16, bmm1=0.1, stride_t=None, stride_h=None, kv_b=None,
            rows_b=0, split_col=64, rows_a=10, ws=None, ws_bytes=0):
    """Call the entry point with fake (never dereferenced) addresses."""
    L = _lib()
    P = ctypes.c_void_p
    return L.sparse_mla_decode(
        P(q) if q else None, H * 576 if stride_t is None else stride_t,
        576 if stride_h is None else stride_h, P(kv) if kv else None, rows_a,
        P(kv_b) if kv_b else None, rows_b, split_col, row_bytes, qk_dim,
        P(idx) if idx else None, P(lens) if lens else None, T, H, W, bmm1, 1.0, None,
        P(out) if out else None, None, flags, None if plan is None else ctypes.byref(plan),
        P(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("kw", [
    dict(T=-1), dict(H=0), dict(H=24), dict(W=0), dict(row_bytes=640), dict(qk_dim=448),
    dict(row_bytes=512, qk_dim=576), dict(flags=0x8), dict(bmm1=float("nan")),
    dict(bmm1=float("inf")), dict(plan=smla.make_plan(0, 1)), dict(plan=smla.make_plan(1, 3)),
    dict(plan=smla.make_plan(1, 0)), dict(plan=smla.make_plan(65, 2)),
    dict(q=0), dict(kv=0), dict(idx=0), dict(lens=0), dict(out=0), dict(rows_a=0),
    dict(q=24), dict(kv=8), dict(out=40), dict(idx=18), dict(lens=2), dict(stride_h=8),
    dict(stride_t=-576), dict(kv_b=16, rows_b=0), dict(kv_b=16, rows_b=5, split_col=65),
    dict(kv_b=16, rows_b=5, split_col=-1), dict(kv_b=24, rows_b=5),
])
def test_decode_rejects_bad_arguments(kw):
    assert _decode(**kw) == smla.SMLA_EINVAL


def test_chunk_local_plans_are_checked():
    """The chunk-local recipe runs the 64-head kernel with one range per 128-column window: any
    other plan is refused before anything is launched; a matching plan gets as far as the
    workspace check."""
    cl = smla.SMLA_P_CHUNK_LOCAL
    assert _decode(W=64, flags=cl, plan=smla.make_plan(1, 1)) == smla.SMLA_EUNSUPPORTED
    assert _decode(W=64, flags=cl, plan=smla.make_plan(2, 2)) == smla.SMLA_EUNSUPPORTED
    assert _decode(W=300, flags=cl, plan=smla.make_plan(2, 2)) == smla.SMLA_EUNSUPPORTED
    assert _decode(W=300, flags=cl, plan=smla.make_plan(4, 2)) == smla.SMLA_EUNSUPPORTED
    assert _decode(W=300, flags=cl, plan=smla.make_plan(3, 2)) == smla.SMLA_EWORKSPACE
    assert _decode(W=300, flags=cl | smla.SMLA_P_ONE_TERM,
                   plan=smla.make_plan(3, 2, heads=16)) == smla.SMLA_EWORKSPACE


def test_64_head_plan_limits_the_range_length():
    """The 64-head kernel stages a key range's row indices in LDS (at most 2048 columns): a plan
    whose ranges could be longer is refused before anything is launched."""
    g64 = smla.make_plan(1, 2)
    assert _decode(H=64, W=4096, plan=g64) == smla.SMLA_EUNSUPPORTED
    assert _decode(H=64, W=2049, plan=g64) == smla.SMLA_EUNSUPPORTED


def test_decode_rejects_missing_or_small_workspace():
    plan = smla.make_plan(4, 1)
    need = smla.workspace_size(plan, 1, 16)
    assert need > 0
    assert _decode(plan=plan) == smla.SMLA_EWORKSPACE
    assert _decode(plan=plan, ws=256, ws_bytes=need - 1) == smla.SMLA_EWORKSPACE
    assert _decode(plan=plan, ws=8, ws_bytes=need) == smla.SMLA_EWORKSPACE  # misaligned


def test_decode_empty_batch_is_a_noop_without_pointers():
    assert _decode(T=0, q=0, kv=0, idx=0, lens=0, out=0) == smla.SMLA_OK
    assert _decode(T=0, q=0, kv=0, idx=0, lens=0, out=0, plan=smla.make_plan(3, 1)) == smla.SMLA_OK
    # the size checks still run first
    assert _decode(T=0, H=8, q=0, kv=0, idx=0, lens=0, out=0) == smla.SMLA_EINVAL


def test_plan_rejects_bad_sizes():
    L = _lib()
    p = smla.Plan()
    for args in [(-1, 16, 64, 576, 0), (1, 0, 64, 576, 0), (1, 8, 64, 576, 0), (1, 16, 0, 576, 0),
                 (1, 16, 64, 600, 0), (1, 16, 64, 576, 0x10)]:
        assert L.smla_decode_plan(*args, ctypes.byref(p)) == smla.SMLA_EINVAL
    assert L.smla_decode_plan(1, 16, 64, 576, 0, None) == smla.SMLA_EINVAL


@pytest.mark.parametrize("args,status", [
    ((0, 1, 1, 8), smla.SMLA_EINVAL), ((1, -1, 1, 8), smla.SMLA_EINVAL),
    ((1, 1, 0, 8), smla.SMLA_EINVAL), ((1, 1, 1, 0), smla.SMLA_EINVAL),
    ((65, 1, 1, 8), smla.SMLA_EUNSUPPORTED), ((2, 1, 1, 12), smla.SMLA_EUNSUPPORTED),
])
def test_lse_merge_rejects_bad_sizes(args, status):
    L = _lib()
    P = ctypes.c_void_p
    S, T, H, D = args
    assert L.lse_merge(P(16), P(16), S, T, H, D, P(16), None, 0, None) == status


def test_lse_merge_pointer_checks():
    L = _lib()
    P = ctypes.c_void_p
    assert L.lse_merge(None, P(16), 2, 1, 1, 8, P(16), None, 0, None) == smla.SMLA_EINVAL
    assert L.lse_merge(P(8), P(16), 2, 1, 1, 8, P(16), None, 0, None) == smla.SMLA_EINVAL
    assert L.lse_merge(P(16), P(16), 2, 1, 1, 8, P(16), None, 0x2, None) == smla.SMLA_EINVAL
    assert L.lse_merge(None, None, 2, 0, 1, 8, None, None, 0, None) == smla.SMLA_OK


def test_noalloc_scratch_size_matches_header():
    """The binding's scratch bound is the header's SMLA_NOALLOC_SCRATCH_BYTES."""
    import re
    text = open(smla.HEADER_PATH).read()
    m = re.search(r"#define SMLA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m, "SMLA_NOALLOC_SCRATCH_BYTES not found"
    assert smla.NOALLOC_SCRATCH_BYTES == int(m.group(1)) << int(m.group(2))
    # the large-batch default plan fits; 64 ranges of 32 heads at T=64, H=128 do not
    assert smla.workspace_size(smla.make_plan(2, 2), 64, 128) <= smla.NOALLOC_SCRATCH_BYTES
    assert smla.workspace_size(smla.make_plan(64, 1), 64, 128) > smla.NOALLOC_SCRATCH_BYTES
