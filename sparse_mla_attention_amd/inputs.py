"""Seeded synthetic inputs for sparse MLA decode and the LSE merge.

This module holds input generation only: random draws, E4M3 / BF16 encoding of the draws
(torch's own casts), index sets and counts.  It contains none of the method's arithmetic and
imports neither the kernels nor the oracle, so both sides can take their inputs from it.

A decode problem is a dict:
  q        uint8 [T, H, qk_dim]   E4M3 bytes
  kv_a     uint8 [rows_a, row_bytes]   E4M3 bytes (pool A; the only pool when kv_b is None), or
           656-byte fp8_ds_mla rows (ds_mla_rows)
  kv_b     uint8 [rows_b, row_bytes] or None   (pool B: columns >= split_col)
  split_col  int   (W when there is one pool)
  qk_dim   int   (576 with 512 latent + 64 rope bytes, or 512)
  indices  int32 [T, W]   storage rows, -1 for unused columns
  lens     int32 [T]      active counts (clamped to [0, W] by the method)
  sinks    float32 [H] or None   (natural-log units)
  bmm1, bmm2   float   (score scale, natural-log units; output scale)
  lse_log2 bool  (whether the caller wants a base-2 LSE)

The shapes, distributions and structure follow the pages' workloads: the Kimi K3.1 DSA
layer's 576-byte rows at the DCP latency checkpoint (attn_sparse page, "Why"), and the
DeepSeek-V4 sparse set of 128 sliding-window columns plus top-k compressed columns with -1
holes and per-head sinks (sparse_mla_cute page, "The problem").  The pages measure on no
public dataset; these stand in for model activations and caches.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3_MAX = 448.0
NAN_E4M3 = 0x7F          # an E4M3 NaN code: poison for rows that must never be read
NAN_BF16 = 0x7FC0        # a BF16 quiet NaN


def e4m3_bytes(x) -> np.ndarray:
    """E4M3 (OCP e4m3fn) bytes of x: torch's float32 -> float8_e4m3fn cast after clamping to
    the finite range (the cast itself does not saturate)."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).clamp_(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def bf16_bits(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


DS_MLA_ROW_BYTES = 656


def ds_mla_rows(latent, rope) -> np.ndarray:
    """656-byte fp8_ds_mla rows of a latent [n, 512] and a rope [n, 64] (the dsa_indexer page's
    MLA cache entry, read as: E4M3 latent bytes 0..511, four FP32 scales at 512..527, one per 128
    latent elements, the BF16 rope at 528..655).  Each 128-element block is quantized the way a
    cache writer does it: scale = its largest magnitude / 448 (FP32), bytes = E4M3(x / scale)."""
    latent = np.asarray(latent, dtype=np.float32)
    n = latent.shape[0]
    out = np.zeros((n, DS_MLA_ROW_BYTES), dtype=np.uint8)
    blocks = latent.reshape(n, 4, 128)
    scale = (np.abs(blocks).max(axis=2) / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    out[:, :512] = e4m3_bytes((blocks / scale[:, :, None]).reshape(n, 512))
    out[:, 512:528] = np.ascontiguousarray(scale).view(np.uint8).reshape(n, 16)
    out[:, 528:656] = np.ascontiguousarray(bf16_bits(rope)).view(np.uint8).reshape(n, 128)
    return out


def _poison_unused(pool: np.ndarray, used: np.ndarray) -> None:
    mask = np.ones(pool.shape[0], dtype=bool)
    mask[used] = False
    pool[mask] = NAN_E4M3


def _junk_rows(rng, pool_rows: int, used: np.ndarray, count: int) -> np.ndarray:
    """In-range row numbers outside `used` (poisoned when poisoning is on), for the index
    entries past lens[t] that the method must never read."""
    free = np.setdiff1d(np.arange(pool_rows), used)
    if free.size == 0:
        return np.full(count, -1, dtype=np.int32)
    return rng.choice(free, size=count, replace=True).astype(np.int32)


def random_problem(seed: int, T: int, H: int, W: int, *, pool_rows: int = 4096,
                   row_bytes: int = 576, qk_dim: int | None = None, lens=None,
                   neg_frac: float = 0.0, two_pools: bool = False, split_col: int = 128,
                   rows_b: int | None = None, sinks: bool = False, value_scale: float = 1.0,
                   kv_scale_to_amax: bool = False, poison: bool = True,
                   duplicates: bool = False, lse_log2: bool = False) -> dict:
    """A general seeded problem for tests.  lens: None (= W), an int, or an array [T].
    neg_frac: probability that an entry below lens is -1.  duplicates: draw rows with
    replacement (repeated rows count once per column)."""
    rng = np.random.default_rng(seed)
    ds = row_bytes == DS_MLA_ROW_BYTES              # fp8_ds_mla rows: per-block scales
    qk_dim = (576 if ds else row_bytes) if qk_dim is None else qk_dim
    q = e4m3_bytes(rng.standard_normal((T, H, qk_dim)) * value_scale)
    x = rng.standard_normal((pool_rows, row_bytes))
    k_scale = 1.0
    if ds:
        kv_a = ds_mla_rows(x[:, :512] * value_scale, x[:, 512:576] * value_scale)
    elif kv_scale_to_amax:
        k_scale = float(np.abs(x).max()) / E4M3_MAX
        kv_a = e4m3_bytes(x / k_scale)
    else:
        kv_a = e4m3_bytes(x * value_scale)
    kv_b = None
    nb = rows_b if rows_b is not None else pool_rows
    if two_pools:
        xb = rng.standard_normal((nb, row_bytes)) * value_scale
        kv_b = ds_mla_rows(xb[:, :512], xb[:, 512:576]) if ds else e4m3_bytes(xb)
    else:
        split_col = W
    if lens is None:
        lens_arr = np.full(T, W, dtype=np.int32)
    elif np.isscalar(lens):
        lens_arr = np.full(T, int(lens), dtype=np.int32)
    else:
        lens_arr = np.asarray(lens, dtype=np.int32).copy()
    indices = np.full((T, W), -1, dtype=np.int32)
    for t in range(T):
        n = int(np.clip(lens_arr[t], 0, W))
        for lo, hi, rows in ((0, min(n, split_col), pool_rows), (min(n, split_col), n, nb)):
            if hi <= lo:
                continue
            k = hi - lo
            indices[t, lo:hi] = rng.choice(rows, size=k, replace=duplicates or k > rows)
        if neg_frac > 0 and n > 0:
            holes = rng.random(n) < neg_frac
            indices[t, :n][holes] = -1
    used_a = np.unique(np.concatenate(
        [indices[t, :min(int(np.clip(lens_arr[t], 0, W)), split_col)] for t in range(T)]
        + [np.zeros(0, np.int32)]))
    used_a = used_a[used_a >= 0]
    used_b = np.zeros(0, np.int32)
    if two_pools:
        used_b = np.unique(np.concatenate(
            [indices[t, split_col:int(np.clip(lens_arr[t], 0, W))] for t in range(T)]
            + [np.zeros(0, np.int32)]))
        used_b = used_b[used_b >= 0]
    # entries past the count: in-range junk pointing at unused (poisoned) rows
    for t in range(T):
        n = int(np.clip(lens_arr[t], 0, W))
        if n >= W:
            continue
        cols = np.arange(n, W)
        in_b = two_pools & (cols >= split_col)
        if (~in_b).any():
            indices[t, cols[~in_b]] = _junk_rows(rng, pool_rows, used_a, int((~in_b).sum()))
        if in_b.any():
            indices[t, cols[in_b]] = _junk_rows(rng, nb, used_b, int(in_b.sum()))
    if poison:
        _poison_unused(kv_a, used_a)
        if two_pools:
            _poison_unused(kv_b, used_b)
    sk = rng.standard_normal(H).astype(np.float32) if sinks else None
    bmm1 = k_scale / np.sqrt(qk_dim)
    return dict(name=f"random{seed}", q=q, kv_a=kv_a, kv_b=kv_b, split_col=int(split_col),
                qk_dim=int(qk_dim), indices=indices, lens=lens_arr, sinks=sk,
                bmm1=float(bmm1), bmm2=float(k_scale), lse_log2=lse_log2,
                value_scale=float(value_scale))


def config_tiny(poison: bool = True) -> dict:
    """T=1, H=16, pool [4096,576] of E4M3(0.5 N(0,1)), 64 distinct active columns, lens 64,
    k_scale 1, bmm1 = 1/sqrt(576), no sink, base-2 LSE."""
    rng = np.random.default_rng(1)
    q = e4m3_bytes(rng.standard_normal((1, 16, 576)) * 0.5)
    kv = e4m3_bytes(rng.standard_normal((4096, 576)) * 0.5)
    idx = rng.choice(4096, size=64, replace=False).astype(np.int32)[None, :]
    if poison:
        _poison_unused(kv, idx[0])
    return dict(name="tiny T=1 H=16 W=64", q=q, kv_a=kv, kv_b=None, split_col=64, qk_dim=576,
                indices=idx, lens=np.array([64], np.int32), sinks=None,
                bmm1=1.0 / 24.0, bmm2=1.0, lse_log2=True)


def config_verify(poison: bool = True) -> dict:
    """One rank's share at the DCP verify-row checkpoint: T=5 rows, H=128 gathered heads,
    flat pool [65536,576] (N(0,1) scaled per tensor to amax 448), lens ~ U{200..300} except an
    interior row with lens 0, W=320, distinct indices, natural-log LSE."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((65536, 576)).astype(np.float32)
    k_scale = float(np.abs(x).max()) / E4M3_MAX
    kv = e4m3_bytes(x / k_scale)
    del x
    q = e4m3_bytes(rng.standard_normal((5, 128, 576)))
    W = 320
    lens = rng.integers(200, 301, size=5).astype(np.int32)
    lens[2] = 0
    idx = np.empty((5, W), np.int32)
    for t in range(5):
        idx[t, :lens[t]] = rng.choice(65536, size=lens[t], replace=False)
    used = np.unique(np.concatenate([idx[t, :lens[t]] for t in range(5)]))
    for t in range(5):
        idx[t, lens[t]:] = _junk_rows(rng, 65536, used, W - lens[t])
    if poison:
        _poison_unused(kv, used)
    return dict(name="verify-row T=5 H=128 W=320", q=q, kv_a=kv, kv_b=None, split_col=W,
                qk_dim=576, indices=idx, lens=lens, sinks=None, bmm1=k_scale / 24.0,
                bmm2=k_scale, lse_log2=False)


def config_dsv4(poison: bool = True) -> dict:
    """DeepSeek-V4 shape: T=12 tokens (2 requests x 6 speculative tokens), H=16, 512-byte rows;
    pool A [8192,512] sliding window, pool B [262144,512] compressed; W=640 = 128 contiguous
    window rows + 512 distinct top-k rows of B; every column -1 with p=0.1; lens ~ U{384..640};
    per-head sinks N(0,1); bmm1 = 1/sqrt(512), bmm2 = 1, natural-log LSE."""
    rng = np.random.default_rng(3)
    kv_a = e4m3_bytes(rng.standard_normal((8192, 512)))
    kv_b = e4m3_bytes(rng.standard_normal((262144, 512)))
    q = e4m3_bytes(rng.standard_normal((12, 16, 512)))
    W, window = 640, 128
    idx = np.empty((12, W), np.int32)
    starts = rng.integers(1000, 8000, size=2)
    for t in range(12):
        pos = int(starts[t // 6]) + t % 6
        idx[t, :window] = (pos - (window - 1) + np.arange(window)) % 8192
        idx[t, window:] = rng.choice(262144, size=W - window, replace=False)
    holes = rng.random((12, W)) < 0.1
    idx[holes] = -1
    lens = rng.integers(384, 641, size=12).astype(np.int32)
    used_a = np.unique(np.concatenate([idx[t, :min(lens[t], window)] for t in range(12)]))
    used_a = used_a[used_a >= 0]
    used_b = np.unique(np.concatenate([idx[t, window:lens[t]] for t in range(12)]))
    used_b = used_b[used_b >= 0]
    for t in range(12):
        if lens[t] < W:
            idx[t, lens[t]:] = _junk_rows(rng, 262144, used_b, W - lens[t])
    sinks = rng.standard_normal(16).astype(np.float32)
    if poison:
        _poison_unused(kv_a, used_a)
        _poison_unused(kv_b, used_b)
    return dict(name="dsv4 T=12 H=16 W=640 two pools + sinks", q=q, kv_a=kv_a, kv_b=kv_b,
                split_col=window, qk_dim=512, indices=idx, lens=lens, sinks=sinks,
                bmm1=1.0 / np.sqrt(512.0), bmm2=1.0, lse_log2=False)


THROUGHPUT_ROWS = 1 << 20


def config_throughput_device(device, index_sets: int = 8):
    """Large-batch shape: T=64, H=128, pool [1048576,576] (N(0,1) scaled per tensor to amax
    448, ~604 MB, drawn on the device with a seeded torch generator), 2048 distinct indices per
    token, lens 2048, natural-log LSE.  `index_sets` independent index sets (seeds 40..) are
    returned so that timed calls can rotate through them.  Returns a dict of device tensors
    (pool as uint8) plus host scalars; the host copy for the oracle is taken from the device."""
    g = torch.Generator(device=device)
    g.manual_seed(4)
    rows, rb = THROUGHPUT_ROWS, 576
    pool = torch.empty((rows, rb), dtype=torch.uint8, device=device)
    amax = 0.0
    step = 1 << 16
    # two passes over the same seeded stream: the amax first, then the encoding
    for p in range(2):
        g.manual_seed(4)
        for r0 in range(0, rows, step):
            x = torch.randn((step, rb), generator=g, device=device, dtype=torch.float32)
            if p == 0:
                amax = max(amax, float(x.abs().max()))
            else:
                y = (x / (amax / E4M3_MAX)).clamp_(-E4M3_MAX, E4M3_MAX)
                pool[r0:r0 + step] = y.to(torch.float8_e4m3fn).view(torch.uint8)
    k_scale = amax / E4M3_MAX
    q = torch.randn((64, 128, 576), generator=g, device=device, dtype=torch.float32)
    q = q.clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    sets = []
    for s in range(index_sets):
        rng = np.random.default_rng(40 + s)
        idx = np.stack([rng.choice(rows, size=2048, replace=False) for _ in range(64)])
        sets.append(torch.from_numpy(idx.astype(np.int32)).to(device))
    lens = torch.full((64,), 2048, dtype=torch.int32, device=device)
    return dict(name="throughput T=64 H=128 W=2048", q=q, kv_a=pool, kv_b=None, split_col=2048,
                qk_dim=576, index_sets=sets, lens=lens, sinks=None, bmm1=k_scale / 24.0,
                bmm2=k_scale, lse_log2=False)


def config_throughput_ds_device(device) -> dict:
    """The large-batch shape on 656-byte fp8_ds_mla rows: T=64, H=128, a [1048576, 656] pool
    (~688 MB) whose latent N(0,1) is quantized per 128-element block at amax / 448 and whose
    rope is BF16(N(0,1)), drawn on the device with a seeded torch generator; 2048 distinct
    indices per token, lens 2048, bmm1 = 1/24, bmm2 = 1."""
    g = torch.Generator(device=device)
    g.manual_seed(14)
    rows = THROUGHPUT_ROWS
    pool = torch.empty((rows, DS_MLA_ROW_BYTES), dtype=torch.uint8, device=device)
    step = 1 << 16
    for r0 in range(0, rows, step):
        x = torch.randn((step, 4, 128), generator=g, device=device, dtype=torch.float32)
        scale = (x.abs().amax(dim=2) / E4M3_MAX).clamp_min_(1e-30)
        lat = (x / scale[:, :, None]).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
        pool[r0:r0 + step, :512] = lat.view(torch.uint8).reshape(step, 512)
        pool[r0:r0 + step, 512:528] = scale.contiguous().view(torch.uint8).reshape(step, 16)
        rope = torch.randn((step, 64), generator=g, device=device, dtype=torch.float32)
        pool[r0:r0 + step, 528:] = rope.to(torch.bfloat16).view(torch.uint8).reshape(step, 128)
    q = torch.randn((64, 128, 576), generator=g, device=device, dtype=torch.float32)
    q = q.clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    rng = np.random.default_rng(41)
    idx = np.stack([rng.choice(rows, size=2048, replace=False) for _ in range(64)])
    return dict(name="throughput on fp8_ds_mla rows T=64 H=128 W=2048", q=q, kv_a=pool,
                kv_b=None, split_col=2048, qk_dim=576,
                indices=torch.from_numpy(idx.astype(np.int32)).to(device),
                lens=torch.full((64,), 2048, dtype=torch.int32, device=device), sinks=None,
                bmm1=1.0 / 24.0, bmm2=1.0, lse_log2=False)


def config_merge() -> dict:
    """8 split-KV sources [8, T=32, H=128, 512] of BF16(N(0,1)) with base-2 LSEs ~ N(5,2);
    each (source, t, h) empty (-inf) with p=0.1; (t=0, h=0..3) empty in every source; the
    partials of empty sources are NaN (never to be read); natural-log LSE out."""
    rng = np.random.default_rng(5)
    S, T, H, D = 8, 32, 128, 512
    x = bf16_bits(rng.standard_normal((S, T, H, D)).astype(np.float32))
    lse = (5.0 + 2.0 * rng.standard_normal((S, T, H))).astype(np.float32)
    empty = rng.random((S, T, H)) < 0.1
    empty[:, 0, 0:4] = True
    lse[empty] = -np.inf
    x[empty] = NAN_BF16
    return dict(name="lse merge S=8 T=32 H=128 D=512", partials=x, lse=lse, lse_log2_out=False)


def random_merge(seed: int, S: int, T: int, H: int, D: int = 512, empty_frac: float = 0.1,
                 nan_lse: bool = False) -> dict:
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((S, T, H, D)).astype(np.float32))
    lse = (5.0 + 2.0 * rng.standard_normal((S, T, H))).astype(np.float32)
    empty = rng.random((S, T, H)) < empty_frac
    if T > 0 and H > 0:
        empty[:, 0, 0] = True
    lse[empty] = -np.inf
    if nan_lse:
        # other non-finite encodings of "empty": NaN and +inf
        sel = empty & (rng.random((S, T, H)) < 0.5)
        lse[sel] = np.nan
        sel2 = empty & ~sel & (rng.random((S, T, H)) < 0.3)
        lse[sel2] = np.inf
    x[empty] = NAN_BF16
    return dict(name=f"merge{seed}", partials=x, lse=lse, lse_log2_out=False)


CONFIGS = {
    "tiny": config_tiny,
    "verify": config_verify,
    "dsv4": config_dsv4,
}


def value_problem(seed: int, S: int, T: int, H: int, empty_frac: float = 0.1,
                  padded_requests: int = 0, rows_per_request: int = 1) -> dict:
    """Inputs of the MLA value tail: the split partials and LSEs of random_merge, a BF16 W_UV
    stored [H, 128, 512] (latent-contiguous; N(0,1)/16, so the 512-term products are unit
    scale), BF16 gates N(0, 2^2) [T, H*128], and per-request totals (the first
    `padded_requests` requests are padding: total 0, their gates NaN)."""
    m = random_merge(seed, S, T, H, 512, empty_frac=empty_frac)
    rng = np.random.default_rng(seed + 1)
    w_t = bf16_bits(rng.standard_normal((H, 128, 512)).astype(np.float32) / 16.0)
    gate = bf16_bits((2.0 * rng.standard_normal((T, H * 128))).astype(np.float32))
    nreq = -(-T // rows_per_request)
    totals = rng.integers(1, 4096, size=nreq).astype(np.int32)
    totals[:padded_requests] = 0
    for r in range(padded_requests):
        gate[r * rows_per_request:(r + 1) * rows_per_request] = NAN_BF16
    return dict(name=f"value{seed}", partials=m["partials"], lse=m["lse"], w_uv_t=w_t,
                gate=gate, totals=totals, rows_per_request=rows_per_request)


def paged_problem(seed: int, B: int, q_len: int, H: int, lengths, *, page_size: int = 64,
                  max_pages: int | None = None, spare_pages: int = 8, kv_scale_to_amax=True,
                  poison: bool = True) -> dict:
    """A dense paged MLA decode problem (the dcp page's stock_decode): B requests of q_len
    query rows each (row t = b * q_len + i), H heads, a paged FP8 cache [num_pages, page_size,
    576] (N(0,1) scaled per tensor to amax 448), block_table [B, max_pages] of distinct pages in
    random order (entries past a request's context point at other, poisoned pages), context
    lengths [B]; bmm1 = k_scale / sqrt(576), bmm2 = k_scale, natural-log LSE.  Cache rows no
    request's context covers are E4M3 NaN when `poison` is set."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int32)
    need = [-(-int(max(l, 0)) // page_size) for l in lengths]
    max_pages = max(1, max(need)) if max_pages is None else max_pages
    num_pages = sum(need) + spare_pages
    x = rng.standard_normal((num_pages * page_size, 576)).astype(np.float32)
    k_scale = float(np.abs(x).max()) / E4M3_MAX if kv_scale_to_amax else 1.0
    cache = e4m3_bytes(x / k_scale).reshape(num_pages, page_size, 576)
    del x
    q = e4m3_bytes(rng.standard_normal((B * q_len, H, 576)))
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.empty((B, max_pages), np.int32)
    pos = 0
    spare = perm[sum(need):]
    for b in range(B):
        bt[b, :need[b]] = perm[pos:pos + need[b]]
        pos += need[b]
        bt[b, need[b]:] = rng.choice(spare, size=max_pages - need[b]) if spare.size else 0
    if poison:
        used = np.zeros((num_pages, page_size), dtype=bool)
        for b in range(B):
            for k in range(int(max(lengths[b], 0))):
                used[bt[b, k // page_size], k % page_size] = True
        cache[~used] = NAN_E4M3
    return dict(name=f"paged B={B} q_len={q_len} H={H}", q=q, cache=cache, block_table=bt,
                lengths=lengths, q_len=q_len, bmm1=k_scale / 24.0, bmm2=k_scale, lse_log2=False)


def paged_as_sparse(p: dict) -> dict:
    """The same paged problem as a sparse one over the flattened cache: row t's indices are its
    context's storage rows in order, its count the causal count."""
    num_pages, page_size, _ = p["cache"].shape
    B, max_pages = p["block_table"].shape
    q_len = p["q_len"]
    W = max_pages * page_size
    T = B * q_len
    idx = np.full((T, W), -1, np.int32)
    lens = np.zeros(T, np.int32)
    k = np.arange(W)
    for t in range(T):
        b, i = divmod(t, q_len)
        n = int(np.clip(p["lengths"][b] - (q_len - 1 - i), 0, W))
        lens[t] = n
        idx[t, :n] = p["block_table"][b, k[:n] // page_size] * page_size + k[:n] % page_size
    return dict(name=p["name"] + " as sparse", q=p["q"],
                kv_a=p["cache"].reshape(num_pages * page_size, 576), kv_b=None, split_col=W,
                qk_dim=576, indices=idx, lens=lens, sinks=None, bmm1=p["bmm1"], bmm2=p["bmm2"],
                lse_log2=p["lse_log2"])
