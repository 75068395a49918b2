"""Sparse MLA decode and split-KV LSE merge on AMD MI355X (gfx950).

A thin ctypes binding of the C ABI in ``include/smla.h`` (library ``_build/libsmla.so``):
argument marshalling only.  Every step of the computation runs in the library's HIP kernels;
PyTorch supplies device memory and the current stream.  Importing this package does not load
the library; the first call does, and raises if it is missing (build it with
``python -m sparse_mla_attention_amd.build`` or ``__graft_entry__.build()``).  There is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_build", "libsmla.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "smla.h")

SMLA_OK, SMLA_EINVAL, SMLA_EUNSUPPORTED, SMLA_EWORKSPACE, SMLA_EHIP = 0, 1, 2, 3, 4
SMLA_ESCRATCH = 5
NOALLOC_SCRATCH_BYTES = 48 << 20
SMLA_LSE_LOG2 = 0x1
SMLA_P_ONE_TERM = 0x2
SMLA_P_CHUNK_LOCAL = 0x4
SMLA_MERGE_LAST, SMLA_MERGE_SPREAD = 0, 1


class SmlaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_load().smla_strerror(status).decode()} (status {status})")


class Plan(ctypes.Structure):
    _fields_ = [("splits", ctypes.c_int32), ("tiles", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("merge", ctypes.c_int32),
                ("heads", ctypes.c_int32)]

    def __repr__(self):
        heads = f", heads={self.heads}" if self.heads else ""
        return (f"Plan(splits={self.splits}, tiles={self.tiles}, chunk={self.chunk}, "
                f"merge={self.merge}{heads})")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"the HIP library is not built ({LIB_PATH} is missing)")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, U32, F, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                               ctypes.c_float, ctypes.c_size_t)
    L.smla_strerror.argtypes = [I32]
    L.smla_strerror.restype = ctypes.c_char_p
    L.smla_decode_plan.argtypes = [I32, I32, I32, I32, U32, ctypes.POINTER(Plan)]
    L.smla_decode_plan.restype = I32
    L.smla_decode_workspace_size.argtypes = [ctypes.POINTER(Plan), I32, I32]
    L.smla_decode_workspace_size.restype = SZ
    L.sparse_mla_decode.argtypes = [P, I64, I64, P, I64, P, I64, I32, I32, I32, P, P, I32, I32,
                                    I32, F, F, P, P, P, U32, ctypes.POINTER(Plan), P, SZ, P]
    L.sparse_mla_decode.restype = I32
    L.lse_merge.argtypes = [P, P, I32, I32, I32, I32, P, P, U32, P]
    L.lse_merge.restype = I32
    L.sparse_mla_decode_noalloc.argtypes = [P, I64, I64, P, I64, P, I64, I32, I32, I32, P, P,
                                            I32, I32, I32, F, F, P, P, P, U32,
                                            ctypes.POINTER(Plan), P]
    L.sparse_mla_decode_noalloc.restype = I32
    L.paged_mla_decode.argtypes = [P, I64, I64, P, I64, I32, I64, P, I32, P, I32, I32, I32, F, F,
                                   P, P, U32, ctypes.POINTER(Plan), P, SZ, P]
    L.paged_mla_decode.restype = I32
    L.smla_paged_decode_plan.argtypes = [I32, I32, I32, I32, I32, U32, ctypes.POINTER(Plan)]
    L.smla_paged_decode_plan.restype = I32
    L.mla_value.argtypes = [P, P, I32, I32, I32, P, I64, I64, P, P, I32, P, U32, P]
    L.mla_value.restype = I32
    L.smla_testing_set_merge_wait.argtypes = [I32, I32]
    L.smla_testing_set_merge_wait.restype = I32
    _lib = L
    return L


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def declared_functions() -> list[str]:
    """Names of the functions include/smla.h declares (for the export check)."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "while", "for", "sizeof", "return"})


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def plan_for(T: int, H: int, W: int, row_bytes: int = 576, flags: int = 0) -> Plan:
    p = Plan()
    st = _load().smla_decode_plan(T, H, W, row_bytes, flags, ctypes.byref(p))
    if st != SMLA_OK:
        raise SmlaError(st, "smla_decode_plan")
    return p


def workspace_size(plan: Plan, T: int, H: int) -> int:
    return int(_load().smla_decode_workspace_size(ctypes.byref(plan), T, H))


def new_workspace(plan: Plan, T: int, H: int, device="cuda"):
    """A zero-filled workspace for `plan` (None when the plan needs none)."""
    import torch
    n = workspace_size(plan, T, H)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def workspace_header_bytes(plan: Plan, T: int, H: int) -> int:
    """Bytes at the start of a workspace that must be zero before a call: the status word and
    the arrival counters, padded to 256 (the layout include/smla.h states)."""
    gw = plan.heads or 32 * plan.tiles
    groups = -(-H // gw)
    return (16 + T * groups * 2 * 4 + 255) // 256 * 256


def workspace_status(workspace) -> int:
    """The workspace's status word (split merges that gave up waiting); synchronizes."""
    if workspace is None:
        return 0
    return int(workspace[:4].view(__import__("torch").int32).item())


def testing_set_merge_wait(max_polls: int = 0, unreachable: bool = False) -> None:
    """Test hook: bound (and optionally make unreachable) the split-merge wait of the 64-head
    kernel; testing_set_merge_wait() restores the default."""
    st = _load().smla_testing_set_merge_wait(int(max_polls), 1 if unreachable else 0)
    if st != SMLA_OK:
        raise SmlaError(st, "smla_testing_set_merge_wait")


def make_plan(splits: int, tiles: int, merge: int = SMLA_MERGE_LAST, heads: int = 0) -> Plan:
    return Plan(splits, tiles, 64, merge, heads)


def _decode_args(q, kv_a, indices, lens, bmm1_scale, bmm2_scale, out, lse, kv_b, split_col,
                 sinks, qk_dim, lse_log2, one_term, plan, workspace, stream, chunk_local=False):
    T, H, qd = q.shape
    W = indices.shape[1]
    row_bytes = kv_a.shape[1]
    qk_dim = qd if qk_dim is None else qk_dim
    flags = ((SMLA_LSE_LOG2 if lse_log2 else 0) | (SMLA_P_ONE_TERM if one_term else 0) |
             (SMLA_P_CHUNK_LOCAL if chunk_local else 0))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(q), q.stride(0) * q.element_size(), q.stride(1) * q.element_size(),
            _ptr(kv_a), kv_a.shape[0],
            _ptr(kv_b), 0 if kv_b is None else kv_b.shape[0],
            W if split_col is None else int(split_col),
            row_bytes, qk_dim, _ptr(indices), _ptr(lens), T, H, W,
            float(bmm1_scale), float(bmm2_scale), _ptr(sinks), _ptr(out), _ptr(lse), flags,
            None if plan is None else ctypes.byref(plan), _ptr(workspace), ws_bytes,
            _stream(stream))


def sparse_mla_decode(q, kv_a, indices, lens, bmm1_scale, bmm2_scale, out, lse=None, *,
                      kv_b=None, split_col=None, sinks=None, qk_dim=None, lse_log2=False,
                      one_term=False, plan=None, workspace=None, stream=None, chunk_local=False):
    """Call sparse_mla_decode on device tensors.

    q: uint8 [T, H, qk_dim] (any strides with unit last stride, 16-byte multiples);
    kv_a / kv_b: uint8 [rows, row_bytes]; indices int32 [T, W]; lens int32 [T];
    out bf16 [T, H, 512]; lse float32 [T, H] or None; sinks float32 [H] or None.
    workspace: a uint8 device tensor of at least workspace_size(plan, T, H) bytes when the plan
    splits the columns (None otherwise), zero-filled before its first use (see
    new_workspace).  chunk_local selects SMLA_P_CHUNK_LOCAL (the plan, if given, from
    plan_for(..., flags=SMLA_P_CHUNK_LOCAL))."""
    st = _load().sparse_mla_decode(*_decode_args(
        q, kv_a, indices, lens, bmm1_scale, bmm2_scale, out, lse, kv_b, split_col, sinks,
        qk_dim, lse_log2, one_term, plan, workspace, stream, chunk_local))
    if st != SMLA_OK:
        raise SmlaError(st, "sparse_mla_decode")
    return out, lse


def sparse_mla_decode_noalloc(q, kv_a, indices, lens, bmm1_scale, bmm2_scale, out, lse=None, *,
                              kv_b=None, split_col=None, sinks=None, qk_dim=None, lse_log2=False,
                              one_term=False, plan=None, stream=None, chunk_local=False):
    """sparse_mla_decode without a workspace argument: the library's static per-device scratch
    serves as the workspace (no allocation anywhere; calls that overlap on one GPU race)."""
    a = _decode_args(q, kv_a, indices, lens, bmm1_scale, bmm2_scale, out, lse, kv_b, split_col,
                     sinks, qk_dim, lse_log2, one_term, plan, None, stream, chunk_local)
    st = _load().sparse_mla_decode_noalloc(*a[:22], a[24])
    if st != SMLA_OK:
        raise SmlaError(st, "sparse_mla_decode_noalloc")
    return out, lse


def prepare_decode(q, kv_a, indices, lens, bmm1_scale, bmm2_scale, out, lse=None, *,
                   kv_b=None, split_col=None, sinks=None, qk_dim=None, lse_log2=False,
                   one_term=False, plan=None, workspace=None, stream=None, chunk_local=False):
    """The same call with its arguments converted once, for loops that launch it repeatedly on
    the same buffers: returns a function of no arguments that launches it (on `stream`, else on
    the stream current when this was called) and raises SmlaError on a bad status.  The tensors
    must stay alive and in place while the function is used."""
    f = _load().sparse_mla_decode
    args = _decode_args(q, kv_a, indices, lens, bmm1_scale, bmm2_scale, out, lse, kv_b,
                        split_col, sinks, qk_dim, lse_log2, one_term, plan, workspace, stream,
                        chunk_local)
    keep = (q, kv_a, indices, lens, out, lse, kv_b, sinks, plan, workspace)

    def launch():
        st = f(*args)
        if st != SMLA_OK:
            raise SmlaError(st, "sparse_mla_decode")
        return keep[4], keep[5]

    return launch


def paged_plan_for(B: int, q_len: int, H: int, max_pages: int, page_size: int,
                   flags: int = 0) -> Plan:
    p = Plan()
    st = _load().smla_paged_decode_plan(B, q_len, H, max_pages, page_size, flags, ctypes.byref(p))
    if st != SMLA_OK:
        raise SmlaError(st, "smla_paged_decode_plan")
    return p


def paged_mla_decode(q, cache, block_table, lengths, q_len, bmm1_scale, bmm2_scale, out,
                     lse=None, *, lse_log2=False, one_term=False, plan=None, workspace=None,
                     stream=None):
    """Dense paged MLA decode: q uint8 [B*q_len, H, 576]; cache uint8 [num_pages, page_size,
    576] (any page stride, unit row layout); block_table int32 [B, max_pages]; lengths int32
    [B]; out bf16 [B*q_len, H, 512]; lse float32 [B*q_len, H] or None."""
    T, H, qd = q.shape
    num_pages, page_size, rb = cache.shape
    B, max_pages = block_table.shape
    assert qd == 576 and rb == 576 and T == B * q_len
    assert cache.stride(2) == 1 and cache.stride(1) == 576
    flags = (SMLA_LSE_LOG2 if lse_log2 else 0) | (SMLA_P_ONE_TERM if one_term else 0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _load().paged_mla_decode(
        _ptr(q), q.stride(0) * q.element_size(), q.stride(1) * q.element_size(), _ptr(cache),
        num_pages, page_size, cache.stride(0) * cache.element_size(), _ptr(block_table),
        max_pages, _ptr(lengths), B, q_len, H, float(bmm1_scale), float(bmm2_scale), _ptr(out),
        _ptr(lse), flags, None if plan is None else ctypes.byref(plan), _ptr(workspace),
        ws_bytes, _stream(stream))
    if st != SMLA_OK:
        raise SmlaError(st, "paged_mla_decode")
    return out, lse


def mla_value(partials, lse2, w_uv, gate, out, *, totals=None, rows_per_request=1, stream=None):
    """partials bf16 [S, T, H, 512]; lse2 float32 [S, T, H] (base 2); w_uv bf16 viewed as
    [H, 512, 128] with unit latent stride (e.g. a transposed view of a [H, 128, 512] tensor);
    gate bf16 [T, H * 128]; out bf16 [T, H * 128]; totals int32 per request or None."""
    S, T, H, D = partials.shape
    assert D == 512 and tuple(w_uv.shape) == (H, 512, 128) and w_uv.stride(1) == 1
    st = _load().mla_value(_ptr(partials), _ptr(lse2), S, T, H, _ptr(w_uv), w_uv.stride(0),
                           w_uv.stride(2), _ptr(gate), _ptr(totals), rows_per_request, _ptr(out),
                           0, _stream(stream))
    if st != SMLA_OK:
        raise SmlaError(st, "mla_value")
    return out


def lse_merge(partials, lse2, out, lse_out=None, *, lse_log2=False, stream=None):
    """partials bf16 [S, T, H, D]; lse2 float32 [S, T, H] (base 2); out bf16 [T, H, D];
    lse_out float32 [T, H] or None."""
    S, T, H, D = partials.shape
    st = _load().lse_merge(_ptr(partials), _ptr(lse2), S, T, H, D, _ptr(out), _ptr(lse_out),
                           SMLA_LSE_LOG2 if lse_log2 else 0, _stream(stream))
    if st != SMLA_OK:
        raise SmlaError(st, "lse_merge")
    return out, lse_out
