"""FP64 CPU oracle for sparse MLA decode and the split-KV LSE merge (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
this package.  The product library never links or calls it, and it imports nothing from the
product package.  The arithmetic lives in ``smla_oracle.c`` (plain C, double precision); this
module only builds it with gcc and marshals numpy arrays through ctypes.

What each function computes, and the passage it follows, is stated in ``smla_oracle.c``:
exact mode follows the formula of the sparse_mla_cute page ("What this module computes"),
mimic mode the E4M3-P recipe of the attn_sparse page (module docstring and the merge method),
``lse_merge`` the DcpValue.merge method of the dcp page, and ``mla_value`` that merge followed by
W_UV and the sigmoid gate (the DcpValue class docstring and merge method).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "smla_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libsmla_oracle.so")

LSE_LOG2 = 1

OK, EBADARG, ERANGE, ENAN = 0, 1, 2, 3
_ERRORS = {EBADARG: "bad argument", ERANGE: "index out of range", ENAN: "E4M3 NaN in an input"}


class OracleError(RuntimeError):
    pass


def build() -> str:
    """Compile the oracle with gcc (-O2, no fast-math: IEEE double throughout)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P, I32, I64, U32, D = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                               ctypes.c_uint32, ctypes.c_double)
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = D
        L.oracle_e4m3_encode.argtypes = [D]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_value.restype = D
        common = [P, I64, I64, P, I64, P, I64, I32, I32, I32, P, P, I32, I32, I32, D, D, P, U32]
        L.oracle_decode_exact.argtypes = common + [P, I32, P, P]
        L.oracle_decode_exact.restype = ctypes.c_int
        L.oracle_decode_mimic.argtypes = common + [I32, I32, D, I32, I32, P, I32, P, P]
        L.oracle_decode_mimic.restype = ctypes.c_int
        L.oracle_decode_chunk_local.argtypes = common + [I32, D, I32, I32, P, I32, P, P]
        L.oracle_decode_chunk_local.restype = ctypes.c_int
        L.oracle_lse_merge.argtypes = [P, P, I32, I32, I32, I32, U32, P, P]
        L.oracle_lse_merge.restype = ctypes.c_int
        L.oracle_paged_decode_exact.argtypes = [P, I64, I64, P, I64, I32, I64, P, I32, P, I32,
                                                I32, I32, D, D, U32, P, I32, P, P]
        L.oracle_paged_decode_exact.restype = ctypes.c_int
        L.oracle_mla_value.argtypes = [P, P, I32, I32, I32, P, I64, I64, P, P, I32, P]
        L.oracle_mla_value.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(status):
    if status != OK:
        raise OracleError(_ERRORS.get(status, f"status {status}"))


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def e4m3_encode(x: float) -> int:
    return int(lib().oracle_e4m3_encode(float(x)))


def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(int(bits))


def _problem_args(p):
    """Marshal a decode problem (a dict of numpy arrays and scalars, see inputs.py)."""
    q = np.ascontiguousarray(p["q"], dtype=np.uint8)
    T, H, qk_stride = q.shape
    kv_a = np.ascontiguousarray(p["kv_a"], dtype=np.uint8)
    kv_b = p.get("kv_b")
    kv_b = None if kv_b is None else np.ascontiguousarray(kv_b, dtype=np.uint8)
    ind = np.ascontiguousarray(p["indices"], dtype=np.int32)
    lens = np.ascontiguousarray(p["lens"], dtype=np.int32)
    sinks = p.get("sinks")
    sinks = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float32)
    W = ind.shape[1]
    keep = (q, kv_a, kv_b, ind, lens, sinks)
    args = [_ptr(q), H * qk_stride, qk_stride, _ptr(kv_a), kv_a.shape[0],
            _ptr(kv_b), 0 if kv_b is None else kv_b.shape[0], int(p.get("split_col", W)),
            kv_a.shape[1], int(p["qk_dim"]), _ptr(ind), _ptr(lens), T, H, W,
            float(p["bmm1"]), float(p["bmm2"]), _ptr(sinks)]
    return args, keep, T, H


def _units_array(units):
    if units is None:
        return None, 0
    u = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
    return u, u.shape[0]


def decode_exact(p, lse_log2=False, units=None):
    """Exact mode: returns (out [n,512] float64, lse [n] float64) for every (t,h), or for the
    given (t,h) pairs.  Raises OracleError on an out-of-range index or an E4M3 NaN."""
    args, keep, T, H = _problem_args(p)
    u, n = _units_array(units)
    count = n if u is not None else T * H
    out = np.empty((count, 512), dtype=np.float64)
    lse = np.empty((count,), dtype=np.float64)
    _check(lib().oracle_decode_exact(*args, LSE_LOG2 if lse_log2 else 0, _ptr(u), n,
                                     _ptr(out), _ptr(lse)))
    del keep
    return out, lse


def decode_mimic(p, splits, chunk, anchor=448.0, terms=1, quantize=True, lse_log2=False,
                 units=None):
    """Mimic mode: the E4M3-P recipe (P anchored at the running maximum, accumulators and sums
    rescaled when it rises) with the given split count and chunk size."""
    args, keep, T, H = _problem_args(p)
    u, n = _units_array(units)
    count = n if u is not None else T * H
    out = np.empty((count, 512), dtype=np.float64)
    lse = np.empty((count,), dtype=np.float64)
    _check(lib().oracle_decode_mimic(*args, LSE_LOG2 if lse_log2 else 0, int(splits), int(chunk),
                                     float(anchor), int(terms), 1 if quantize else 0,
                                     _ptr(u), n, _ptr(out), _ptr(lse)))
    del keep
    return out, lse


def decode_chunk_local(p, width=128, anchor=256.0, terms=1, quantize=True, lse_log2=False,
                       units=None):
    """Chunk-local mode (the sparse_mla_cute page, "How."): one softmax per chunk of `width`
    columns at the chunk's own maximum, P at `anchor` of it as E4M3, the chunks merged with
    weights 2^(m_k - M) over the chunks and the sink."""
    args, keep, T, H = _problem_args(p)
    u, n = _units_array(units)
    count = n if u is not None else T * H
    out = np.empty((count, 512), dtype=np.float64)
    lse = np.empty((count,), dtype=np.float64)
    _check(lib().oracle_decode_chunk_local(*args, LSE_LOG2 if lse_log2 else 0, int(width),
                                           float(anchor), int(terms), 1 if quantize else 0,
                                           _ptr(u), n, _ptr(out), _ptr(lse)))
    del keep
    return out, lse


def lse_merge(partials_bits, lse2, lse_log2=False):
    """partials_bits: uint16 BF16 bits [S,T,H,D]; lse2: float32 [S,T,H] (base 2).
    Returns (out [T,H,D] float64, lse [T,H] float64)."""
    x = np.ascontiguousarray(partials_bits, dtype=np.uint16)
    l2 = np.ascontiguousarray(lse2, dtype=np.float32)
    S, T, H, D = x.shape
    assert l2.shape == (S, T, H)
    out = np.empty((T, H, D), dtype=np.float64)
    lse = np.empty((T, H), dtype=np.float64)
    _check(lib().oracle_lse_merge(_ptr(x), _ptr(l2), S, T, H, D, LSE_LOG2 if lse_log2 else 0,
                                  _ptr(out), _ptr(lse)))
    return out, lse


def mla_value(partials_bits, lse2, w_uv_bits, gate_bits, totals=None, rows_per_request=1):
    """The MLA value tail: LSE merge of S sources (BF16 bits [S,T,H,512], base-2 LSE [S,T,H]),
    one BF16 rounding, W_UV (BF16 bits [H,512,128], element (h,k,v)), BF16 rounding, times
    sigmoid(gate) (BF16 bits [T, H*128]), BF16 rounding; rows with totals[t // rows_per_request]
    <= 0 are zeros.  Returns out [T, H*128] float64 (each a BF16 value)."""
    x = np.ascontiguousarray(partials_bits, dtype=np.uint16)
    l2 = np.ascontiguousarray(lse2, dtype=np.float32)
    w = np.ascontiguousarray(w_uv_bits, dtype=np.uint16)
    g = np.ascontiguousarray(gate_bits, dtype=np.uint16)
    S, T, H, D = x.shape
    assert D == 512 and l2.shape == (S, T, H) and w.shape == (H, 512, 128)
    assert g.shape == (T, H * 128)
    tot = None if totals is None else np.ascontiguousarray(totals, dtype=np.int32)
    out = np.empty((T, H * 128), dtype=np.float64)
    # element (h, k, v) of the [H, 512, 128] array: h * 512 * 128 + k * 128 + v; the oracle
    # addresses it as h * stride_h + v * stride_v + k, so pass the transposed copy
    wt = np.ascontiguousarray(np.transpose(w, (0, 2, 1)))  # [H, 128, 512]: k contiguous
    _check(lib().oracle_mla_value(_ptr(x), _ptr(l2), S, T, H, _ptr(wt), 128 * 512, 512, _ptr(g),
                                  _ptr(tot), int(rows_per_request), _ptr(out)))
    return out


def paged_decode_exact(p, lse_log2=False, units=None):
    """Dense paged MLA decode (the dcp page's stock_decode), exact FP64: p holds q [B*q_len, H,
    576] E4M3 bytes, cache [num_pages, page_size, 576] bytes, block_table [B, max_pages] int32,
    lengths [B] int32, q_len, bmm1, bmm2.  Returns (out [n, 512], lse [n]) for every (t, h) or
    the given (t, h) pairs."""
    q = np.ascontiguousarray(p["q"], dtype=np.uint8)
    cache = np.ascontiguousarray(p["cache"], dtype=np.uint8)
    bt = np.ascontiguousarray(p["block_table"], dtype=np.int32)
    lens = np.ascontiguousarray(p["lengths"], dtype=np.int32)
    T, H, qd = q.shape
    assert qd == 576
    num_pages, page_size, rb = cache.shape
    assert rb == 576
    B, max_pages = bt.shape
    q_len = int(p["q_len"])
    assert T == B * q_len
    u, n = _units_array(units)
    count = n if u is not None else T * H
    out = np.empty((count, 512), dtype=np.float64)
    lse = np.empty((count,), dtype=np.float64)
    _check(lib().oracle_paged_decode_exact(
        _ptr(q), H * 576, 576, _ptr(cache), num_pages, page_size, page_size * 576, _ptr(bt),
        max_pages, _ptr(lens), B, q_len, H, float(p["bmm1"]), float(p["bmm2"]),
        LSE_LOG2 if lse_log2 else 0, _ptr(u), n, _ptr(out), _ptr(lse)))
    return out, lse
