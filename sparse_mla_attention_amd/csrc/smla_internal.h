// Internal declarations shared by the library's own source files (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla.h"

namespace smla {

// One sparse_mla_decode launch, fully resolved on the host.
struct DecodeParams {
    const uint8_t *q;
    int64_t q_st, q_sh;         // q strides in bytes (token, head)
    const uint8_t *kv_a;        // pool A
    const uint8_t *kv_b;        // pool B or null
    int32_t split_col;          // columns >= split_col use pool B (when kv_b is set)
    const int32_t *indices;     // [T, W]
    const int32_t *lens;        // [T]
    int32_t T, H, W;
    float scale_log2;           // bmm1 * log2(e)
    float bmm2;
    const float *sinks;         // [H] natural-log units, or null
    uint16_t *out;              // BF16 [T, H, 512]
    float *lse;                 // [T, H] or null
    int32_t lse_log2;           // 1: base-2 LSE
    float *ws_o;                // FP32 partials: a block of (heads per group) x 512 floats per
                                // (token, group, range), in the kernel's register order
    float *ws_ml;               // (m, l) [T, groups, splits, heads per group, 2]
    int32_t *counters;          // [T, groups, 2]: arrival ticket, ready count; zero between
                                // calls (splits > 1)
    int32_t *status;            // workspace status word: merges that gave up waiting
    int32_t wait_polls;         // bound of the 64-head kernel's merge wait (polls)
    int32_t wait_extra;         // 0; 1 makes that wait unreachable (a test hook)
    int32_t splits;             // key ranges per (token, head group)
    int32_t groups;             // head groups per token = ceil(H / gw)
    int32_t gw;                 // real heads per workgroup (the 64-head kernel: 16, 32 or 64)
    int32_t merge;              // 0: the last range to arrive merges; 1: distributed (each
                                // range merges 512 / splits columns; cooperative launch)
    // paged addressing (64-head kernel only): when set, `lens` holds one context length per
    // request of q_len rows, row t = b q_len + i sees the first lens[b] - (q_len - 1 - i) keys,
    // and key k is row k % page_size of page block_table[b][k / page_size] of kv_a
    int32_t paged;
    const int32_t *block_table; // [requests, max_pages]
    int32_t max_pages, page_size, q_len;
    int64_t page_stride;        // bytes
    // 1: the 64-head kernel loads the indices of every column a range can hold alongside the
    // token's count, not after it (the host sets it when the grid fills the device: measured
    // faster there, slower for small grids)
    int32_t spec_idx;
};

// Longest key range (columns) the 64-head kernel takes: its range's row indices are staged in
// LDS.  The host picks or checks split counts against it.
constexpr int G64_MAX_RANGE = 2048;

// Launch the decode (the split merge is fused into it) on `stream`: 32 heads per workgroup
// (tiles = 1) or the 64-head kernel (tiles = 2).  chunk_local selects the chunk-local recipe
// (64-head kernel only: one range per 128-column window, P at 256 of its own maximum).
hipError_t launch_decode(const DecodeParams &p, int tiles, int row_bytes, int qk_dim,
                         bool two_term, bool chunk_local, hipStream_t stream);
hipError_t launch_decode_g64(const DecodeParams &p, int row_bytes, int qk_dim, bool two_term,
                             bool chunk_local, hipStream_t stream);

struct LseMergeParams {
    const uint16_t *partials;   // BF16 [S, T, H, D]
    const float *lse2;          // [S, T, H] base 2
    int32_t S, T, H, D;
    uint16_t *out;              // BF16 [T, H, D]
    float *lse_out;             // [T, H] or null
    int32_t lse_log2;
};

hipError_t launch_lse_merge(const LseMergeParams &p, hipStream_t stream);

// One mla_value launch: the split merge of S sources, W_UV and the sigmoid gate.
struct ValueParams {
    const uint16_t *partials;   // BF16 [S, T, H, 512]
    const float *lse2;          // [S, T, H] base 2
    int32_t S, T, H;
    const uint16_t *w_uv;       // BF16, element (h, k, v) at h * w_sh + v * w_sv + k
    int64_t w_sh, w_sv;         // strides in elements
    const uint16_t *gate;       // BF16 [T, H * 128]
    const int32_t *totals;      // per request, or null (every row live)
    int32_t rows_per_request;
    uint16_t *out;              // BF16 [T, H * 128]
};

hipError_t launch_mla_value(const ValueParams &p, hipStream_t stream);

// Bytes at the start of a workspace under `plan` that must be zero before a call: the status
// word and the arrival counters, padded to 256.
size_t workspace_header_bytes(const smla_plan *plan, int32_t T, int32_t H);

// sparse_mla_decode with, when clear_header is set and the plan needs a workspace, a small
// kernel that zeroes the workspace's header on `stream` first (the caller's workspace then
// needs no zero-fill of its own).
smla_status decode_impl(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                        const void *kv_a, int64_t rows_a,
                        const void *kv_b, int64_t rows_b, int32_t split_col,
                        int32_t row_bytes, int32_t qk_dim,
                        const int32_t *indices, const int32_t *lens,
                        int32_t T, int32_t H, int32_t W,
                        float bmm1_scale, float bmm2_scale, const float *sinks,
                        void *out, float *lse, uint32_t flags,
                        const smla_plan *plan, void *workspace, size_t workspace_bytes,
                        bool clear_header, hipStream_t stream);

}  // namespace smla
