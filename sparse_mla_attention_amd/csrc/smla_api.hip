// C ABI of the library: argument validation, launch planning and dispatch (see include/smla.h).
// Every check happens on the host before anything is launched; no entry point allocates,
// frees or synchronizes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include "smla.h"
#include "smla_internal.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxSplits = 64;
constexpr int kChunk = 64;
constexpr int kDefaultMaxSplits = 4;
constexpr int kFewChunks = 6;
constexpr int kMaxSpreadSplits = 16;
constexpr int kMaxLastSplits32 = 8;
constexpr int kWindow = 128;                       // columns per range of the chunk-local recipe
constexpr int kDsMlaRow = 656;                     // bytes of an fp8_ds_mla row
constexpr int32_t kDefaultWaitPolls = 1 << 20;
std::atomic<int> g_cu_count[kMaxDevices];
// bound of the 64-head kernel's split-merge wait, and the test hook that makes it unreachable
std::atomic<int32_t> g_wait_polls{kDefaultWaitPolls};
std::atomic<int32_t> g_wait_extra{0};

// Compute units of the current device, queried once per device.
hipError_t current_cu_count(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev >= 0 && dev < kMaxDevices) {
        int cached = g_cu_count[dev].load(std::memory_order_relaxed);
        if (cached > 0) {
            *cus = cached;
            return hipSuccess;
        }
    }
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    if (n <= 0)
        n = 1;
    if (dev >= 0 && dev < kMaxDevices)
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    *cus = n;
    return hipSuccess;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

int32_t head_tiles(int32_t H) { return (H + 31) / 32; }

// Head groups per token: workgroups of `tiles` 32-head tiles, the last one padded.
int32_t head_groups(int32_t H, int tiles) { return (head_tiles(H) + tiles - 1) / tiles; }

// Real heads per workgroup under a plan, and head groups per token (the last one padded).
int32_t plan_heads(const smla_plan *p) { return p->heads != 0 ? p->heads : 32 * p->tiles; }
int32_t plan_groups(int32_t H, const smla_plan *p)
{
    const int32_t gw = plan_heads(p);
    return (H + gw - 1) / gw;
}

// Key ranges per (token, head group) of the paged mode's plan: one range when a token has at
// most kFewChunks chunks of columns (a split merge costs more than it saves there); else enough
// workgroups to cover every compute unit, at most kDefaultMaxSplits ranges (the last range of a
// (token, head group) reads every other range's partial to merge them) and at least one chunk
// of columns per range.  The 64-head kernel also needs ranges of at most G64_MAX_RANGE
// columns.
int default_splits(int32_t T, int32_t groups, int32_t W, int cus, int tiles)
{
    const int64_t chunks = (W + kChunk - 1) / kChunk;
    const int64_t need = tiles == 2 ? (W + smla::G64_MAX_RANGE - 1) / smla::G64_MAX_RANGE : 1;
    if (chunks <= kFewChunks)
        return (int)need;
    const int64_t units = (int64_t)T * groups;
    int64_t want = units > 0 ? (cus + units - 1) / units : 1;
    int64_t cap = chunks;
    if (cap > kDefaultMaxSplits)
        cap = kDefaultMaxSplits;
    if (want > cap)
        want = cap;
    if (want < need)
        want = need;
    return want < 1 ? 1 : (int)want;
}

// Predicted time (microseconds) of one decode call under plan `p` on a device of `cus`
// compute units.  The prediction is linear in the quantities that set a call's time:
//   waves   ceil(workgroups / compute units), the rounds of workgroups a launch takes;
//   cpr     chunks of 64 columns per key range, the serial chunk loop of a workgroup;
//   occ     the fraction of compute units in use (their gathers share the memory system);
//   hr      real heads per workgroup (the rows of output and of FP32 partial it writes);
// and, for plans with S > 1 key ranges, S itself, the partial bytes one workgroup moves (2 hr
// rows under the spread merge, S hr rows for the last arriver), the split exchange's total
// bytes over the call, and the grid's size against the compute units; for the spread merge
// also S x occ (its S ranges wait for one another, and the wait grows with the share of the
// device the grid holds).  One coefficient set per kind of plan, fitted (non-negative least
// squares, relative error) to graph-replayed timings on MI355X of every plan on T = 1..64,
// H = 16, 64, 128, W = 128..2048 with rows gathered from a 604 MB pool; on that grid the plans
// chosen by this model take 0.8% more time (summed over shapes) than the best plan measured
// for each shape.
double predicted_us(const smla_plan &p, int32_t T, int32_t H, int32_t W, int cus)
{
    // coefficients of {1, waves, cpr waves, occ cpr waves, hr/64 waves, S, hr/64 rows moved,
    // MB exchanged, workgroups / compute units, S/16 occ}
    static constexpr double kCoef[5][10] = {
        {1.297, 3.166, 1.583, 0.241, 0.880, 0.0, 0.0, 0.0, 0.0, 0.0},      // 64-head, one range
        {0.0, 4.064, 1.581, 0.060, 0.768, 2.780, 0.0, 0.026, 3.934, 0.0},  // 64-head, last arriver
        {0.0, 6.172, 1.621, 0.196, 0.0, 0.084, 1.709, 0.086, 0.198, 4.583},  // 64-head, spread
        {0.0, 6.484, 1.125, 0.164, 1.502, 0.0, 0.0, 0.0, 0.0, 0.0},        // 32-head, one range
        {1.485, 7.198, 1.207, 0.171, 0.216, 0.691, 0.291, 0.0, 2.213, 0.0},  // 32-head, last arriver
    };
    const int S = p.splits;
    const bool spread = p.merge == SMLA_MERGE_SPREAD && S > 1;
    const int kind = p.tiles == 2 ? (S == 1 ? 0 : spread ? 2 : 1) : (S == 1 ? 3 : 4);
    const int32_t gw = plan_heads(&p);
    const double nwg = (double)T * plan_groups(H, &p) * S;
    const double waves = std::ceil(nwg / cus);
    const double cpr = (double)(((W + S - 1) / S + kChunk - 1) / kChunk);
    const double occ = std::min(nwg, (double)cus) / cus;
    const double hr = std::min(gw, H) / 64.0;
    double f[10] = {1.0, waves, cpr * waves, occ * cpr * waves, hr * waves,
                    0.0, 0.0,   0.0,        0.0,              0.0};
    if (S > 1) {
        const int moved = spread ? S : S - 1;  // partials written (and read back) per group
        f[5] = S;
        f[6] = hr * (spread ? 2 : S);
        f[7] = (double)T * H * moved * 4096.0 / 1e6;
        f[8] = nwg / cus;
        if (spread)
            f[9] = S / 16.0 * occ;
    }
    double us = 0.0;
    for (int i = 0; i < 10; i++)
        us += kCoef[kind][i] * f[i];
    return us;
}

bool plan_ok(const smla_plan *p, int32_t H)
{
    if (p->splits < 1 || p->splits > kMaxSplits)
        return false;
    if (p->tiles != 1 && p->tiles != 2)
        return false;
    if (p->merge != SMLA_MERGE_LAST && p->merge != SMLA_MERGE_SPREAD)
        return false;
    if (p->heads != 0 && p->heads != 32 * p->tiles && !(p->tiles == 2 && (p->heads == 16 ||
                                                                           p->heads == 32)))
        return false;
    (void)H;
    return true;
}

// A spread merge needs at least one of the sixteen 32-column output tiles per range (2 to 16
// ranges) and a grid of at most one workgroup per compute unit, so that every workgroup is
// resident at once (each waits for the others of its token and head group).
smla_status spread_ok(const smla_plan *p, int32_t T, int32_t H)
{
    if (p->merge != SMLA_MERGE_SPREAD || p->splits == 1)
        return SMLA_OK;
    if (p->tiles != 2)
        return SMLA_EUNSUPPORTED;  // built into the 64-head kernel only
    if (p->splits < 2 || p->splits > 16)
        return SMLA_EUNSUPPORTED;
    int cus = 0;
    if (current_cu_count(&cus) != hipSuccess)
        return SMLA_EHIP;
    if ((int64_t)T * plan_groups(H, p) * p->splits > cus)
        return SMLA_EUNSUPPORTED;
    return SMLA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout under a valid plan: a status word (int32: split merges that gave up
// waiting), counters [T, groups, 2] int32 from byte 16 (arrival ticket and ready count, zero
// between calls), padded to 256 bytes; then FP32 partials: one block of 32 tiles x 512 floats per
// (token, head group, range), in the order the kernel's accumulator registers are stored (16-byte
// runs per lane); then (m, l) [T, groups, splits, 32 tiles heads, 2].
struct WsLayout {
    size_t status, counters, partials, ml, total;
};

WsLayout ws_layout(const smla_plan *plan, int32_t T, int32_t H)
{
    const size_t groups = (size_t)plan_groups(H, plan);
    const size_t hg = 32 * (size_t)plan->tiles;
    const size_t units = (size_t)T * groups * (size_t)plan->splits;
    WsLayout w;
    w.status = 0;
    w.counters = 16;
    w.partials = align256(w.counters + (size_t)T * groups * 2 * sizeof(int32_t));
    w.ml = w.partials + units * hg * 512 * sizeof(float);
    w.total = w.ml + units * hg * 2 * sizeof(float);
    return w;
}

// Zero `n` int32 words at p (the workspace's status word and arrival counters).  A kernel, not a
// memset, so that a call captured in a graph replays it faithfully.
__global__ void zero_words_kernel(int32_t *p, int n)
{
    for (int i = threadIdx.x; i < n; i += blockDim.x)
        p[i] = 0;
}

}  // namespace

namespace smla {

size_t workspace_header_bytes(const smla_plan *plan, int32_t T, int32_t H)
{
    return ws_layout(plan, T, H).partials;
}

}  // namespace smla

extern "C" {

const char *smla_strerror(smla_status status)
{
    switch (status) {
    case SMLA_OK: return "ok";
    case SMLA_EINVAL: return "invalid argument";
    case SMLA_EUNSUPPORTED: return "unsupported shape";
    case SMLA_EWORKSPACE: return "workspace missing or too small";
    case SMLA_EHIP: return "HIP runtime error";
    case SMLA_ESCRATCH: return "the problem needs more scratch than the library's static buffer";
    default: return "unknown status";
    }
}

smla_status smla_decode_plan(int32_t T, int32_t H, int32_t W, int32_t row_bytes, uint32_t flags,
                             smla_plan *plan)
{
    if (plan == nullptr || T < 0 || H <= 0 || H % 16 != 0 || W < 1)
        return SMLA_EINVAL;
    if (row_bytes != 512 && row_bytes != 576 && row_bytes != kDsMlaRow)
        return SMLA_EINVAL;
    if (flags & ~(SMLA_LSE_LOG2 | SMLA_P_ONE_TERM | SMLA_P_CHUNK_LOCAL))
        return SMLA_EINVAL;
    int cus = 0;
    if (current_cu_count(&cus) != hipSuccess)
        return SMLA_EHIP;
    // Every plan the kernels take for this shape, cheapest predicted time first: the 64-head
    // kernel with 64, 32 or 16 real heads per workgroup over one range, two ranges merged by
    // the last arriver, or 2 to 16 ranges under the spread merge (a grid within the compute
    // units); the 32-head kernel over 1, 2, 4 or 8 ranges.  A later candidate replaces the kept one
    // only when strictly cheaper, so ties keep the widest head groups.
    smla_plan best{1, 1, kChunk, SMLA_MERGE_LAST, 0};
    double best_us = INFINITY;
    auto consider = [&](int32_t splits, int32_t tiles, int32_t merge, int32_t heads) {
        const smla_plan c{splits, tiles, kChunk, merge, heads};
        if (tiles == 2 && (W + splits - 1) / splits > smla::G64_MAX_RANGE)
            return;
        if (merge == SMLA_MERGE_SPREAD && (int64_t)T * plan_groups(H, &c) * splits > cus)
            return;
        const double us = predicted_us(c, T, H, W, cus);
        if (us < best_us) {
            best_us = us;
            best = c;
        }
    };
    if (flags & SMLA_P_CHUNK_LOCAL) {
        // the chunk-local recipe fixes the ranges (one per 128-column window) and the kernel;
        // the head groups and the merge are chosen as above
        const int64_t s = (W + kWindow - 1) / kWindow;
        if (s > kMaxSplits)
            return SMLA_EUNSUPPORTED;
        for (int32_t heads : {0, 32, 16}) {
            consider((int32_t)s, 2, SMLA_MERGE_LAST, heads);
            if (s >= 2 && s <= 16)
                consider((int32_t)s, 2, SMLA_MERGE_SPREAD, heads);
        }
        *plan = best;
        return SMLA_OK;
    }
    for (int32_t heads : {0, 32, 16}) {
        consider(1, 2, SMLA_MERGE_LAST, heads);
        consider(2, 2, SMLA_MERGE_LAST, heads);
        for (int32_t s = 2; s <= kMaxSpreadSplits; s++)
            consider(s, 2, SMLA_MERGE_SPREAD, heads);
    }
    if (row_bytes != kDsMlaRow)  // the 32-head kernel reads E4M3 rows only
        for (int32_t s = 1; s <= kMaxLastSplits32; s *= 2)
            consider(s, 1, SMLA_MERGE_LAST, 0);
    *plan = best;
    return SMLA_OK;
}

size_t smla_decode_workspace_size(const smla_plan *plan, int32_t T, int32_t H)
{
    if (plan == nullptr || T < 0 || H <= 0 || H % 16 != 0 || !plan_ok(plan, H))
        return 0;
    if (plan->splits == 1)
        return 0;
    return ws_layout(plan, T, H).total;
}

}  // extern "C"

namespace smla {

smla_status decode_impl(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                        const void *kv_a, int64_t rows_a,
                        const void *kv_b, int64_t rows_b, int32_t split_col,
                        int32_t row_bytes, int32_t qk_dim,
                        const int32_t *indices, const int32_t *lens,
                        int32_t T, int32_t H, int32_t W,
                        float bmm1_scale, float bmm2_scale, const float *sinks,
                        void *out, float *lse, uint32_t flags,
                        const smla_plan *plan, void *workspace, size_t workspace_bytes,
                        bool clear_header, hipStream_t stream)
{
    // ---- validation (host only) ----------------------------------------------------------
    if (T < 0 || H <= 0 || H % 16 != 0 || W < 1)
        return SMLA_EINVAL;
    if (flags & ~(SMLA_LSE_LOG2 | SMLA_P_ONE_TERM | SMLA_P_CHUNK_LOCAL))
        return SMLA_EINVAL;
    if (row_bytes != 512 && row_bytes != 576 && row_bytes != kDsMlaRow)
        return SMLA_EINVAL;
    if ((qk_dim != 512 && qk_dim != 576) || qk_dim > row_bytes)
        return SMLA_EINVAL;
    if (row_bytes == kDsMlaRow && qk_dim != 576)
        return SMLA_EINVAL;  // an fp8_ds_mla row's score takes its latent and its rope
    if (!isfinite(bmm1_scale) || !isfinite(bmm2_scale))
        return SMLA_EINVAL;
    if (plan != nullptr && !plan_ok(plan, H))
        return SMLA_EINVAL;
    if (T == 0)  // empty tensors may have null data pointers
        return SMLA_OK;
    if (q == nullptr || kv_a == nullptr || indices == nullptr || lens == nullptr || out == nullptr)
        return SMLA_EINVAL;
    if (rows_a < 1)
        return SMLA_EINVAL;
    if (kv_b != nullptr && (rows_b < 1 || split_col < 0 || split_col > W))
        return SMLA_EINVAL;
    if (!aligned16(q) || (q_stride_t & 15) || (q_stride_h & 15) || q_stride_t < 0 ||
        q_stride_h < 0)
        return SMLA_EINVAL;
    if (!aligned16(kv_a) || (kv_b != nullptr && !aligned16(kv_b)) || !aligned16(out))
        return SMLA_EINVAL;
    if (!aligned4(indices) || !aligned4(lens) || (lse != nullptr && !aligned4(lse)) ||
        (sinks != nullptr && !aligned4(sinks)))
        return SMLA_EINVAL;
    smla_plan chosen;
    if (plan != nullptr) {
        chosen = *plan;
    } else {
        smla_status st = smla_decode_plan(T, H, W, row_bytes, flags, &chosen);
        if (st != SMLA_OK)
            return st;
    }
    if (chosen.tiles == 2 && (W + chosen.splits - 1) / chosen.splits > smla::G64_MAX_RANGE)
        return SMLA_EUNSUPPORTED;  // the 64-head kernel stages a range's indices in LDS
    if (row_bytes == kDsMlaRow && chosen.tiles != 2)
        return SMLA_EUNSUPPORTED;  // fp8_ds_mla rows are read by the 64-head kernel only
    const bool chunk_local = (flags & SMLA_P_CHUNK_LOCAL) != 0;
    if (chunk_local && (chosen.tiles != 2 || chosen.splits != (W + kWindow - 1) / kWindow))
        return SMLA_EUNSUPPORTED;  // one range per 128-column window, on the 64-head kernel
    {
        const smla_status st = spread_ok(&chosen, T, H);
        if (st != SMLA_OK)
            return st;
    }
    const size_t need = smla_decode_workspace_size(&chosen, T, H);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
        return SMLA_EWORKSPACE;

    // ---- launch ------------------------------------------------------------------------
    smla::DecodeParams p{};  // zero: every field not set below (the paged mode among them)
    p.q = static_cast<const uint8_t *>(q);
    p.q_st = q_stride_t;
    p.q_sh = q_stride_h;
    p.kv_a = static_cast<const uint8_t *>(kv_a);
    p.kv_b = static_cast<const uint8_t *>(kv_b);
    p.split_col = kv_b != nullptr ? split_col : W;
    p.indices = indices;
    p.lens = lens;
    p.T = T;
    p.H = H;
    p.W = W;
    p.scale_log2 = (float)((double)bmm1_scale * 1.4426950408889634);
    p.bmm2 = bmm2_scale;
    p.sinks = sinks;
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    p.lse_log2 = (flags & SMLA_LSE_LOG2) ? 1 : 0;
    p.splits = chosen.splits;
    p.groups = plan_groups(H, &chosen);
    p.gw = plan_heads(&chosen);
    p.merge = chosen.merge;
    p.ws_o = nullptr;
    p.ws_ml = nullptr;
    p.counters = nullptr;
    p.status = nullptr;
    p.wait_polls = g_wait_polls.load(std::memory_order_relaxed);
    p.wait_extra = g_wait_extra.load(std::memory_order_relaxed);
    {
        int cus = 0;
        if (current_cu_count(&cus) != hipSuccess)
            return SMLA_EHIP;
        p.spec_idx = (int64_t)T * p.groups * p.splits >= cus ? 1 : 0;
    }
    if (need > 0) {
        const WsLayout w = ws_layout(&chosen, T, H);
        uint8_t *base = static_cast<uint8_t *>(workspace);
        p.status = reinterpret_cast<int32_t *>(base + w.status);
        p.counters = reinterpret_cast<int32_t *>(base + w.counters);
        p.ws_o = reinterpret_cast<float *>(base + w.partials);
        p.ws_ml = reinterpret_cast<float *>(base + w.ml);
    }
    if (need > 0 && clear_header) {
        const WsLayout w = ws_layout(&chosen, T, H);
        hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(256), 0, stream,
                           static_cast<int32_t *>(workspace), (int)(w.partials / 4));
        if (hipGetLastError() != hipSuccess)
            return SMLA_EHIP;
    }
    const hipError_t e = smla::launch_decode(p, chosen.tiles, row_bytes, qk_dim,
                                             (flags & SMLA_P_ONE_TERM) == 0, chunk_local, stream);
    return e == hipSuccess ? SMLA_OK : SMLA_EHIP;
}

}  // namespace smla

extern "C" {

smla_status sparse_mla_decode(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                              const void *kv_a, int64_t rows_a,
                              const void *kv_b, int64_t rows_b, int32_t split_col,
                              int32_t row_bytes, int32_t qk_dim,
                              const int32_t *indices, const int32_t *lens,
                              int32_t T, int32_t H, int32_t W,
                              float bmm1_scale, float bmm2_scale, const float *sinks,
                              void *out, float *lse, uint32_t flags,
                              const smla_plan *plan, void *workspace, size_t workspace_bytes,
                              hipStream_t stream)
{
    return smla::decode_impl(q, q_stride_t, q_stride_h, kv_a, rows_a, kv_b, rows_b, split_col,
                             row_bytes, qk_dim, indices, lens, T, H, W, bmm1_scale, bmm2_scale,
                             sinks, out, lse, flags, plan, workspace, workspace_bytes, false,
                             stream);
}

smla_status smla_paged_decode_plan(int32_t B, int32_t q_len, int32_t H, int32_t max_pages,
                                   int32_t page_size, uint32_t flags, smla_plan *plan)
{
    if (plan == nullptr || B < 0 || q_len < 1 || H <= 0 || H % 16 != 0 || max_pages < 1 ||
        page_size < 1 || (int64_t)max_pages * page_size > 0x7FFFFFFF)
        return SMLA_EINVAL;
    if (flags & ~(SMLA_LSE_LOG2 | SMLA_P_ONE_TERM))
        return SMLA_EINVAL;
    int cus = 0;
    if (current_cu_count(&cus) != hipSuccess)
        return SMLA_EHIP;
    const int32_t W = max_pages * page_size;
    plan->tiles = 2;
    plan->splits = default_splits(B * q_len, head_groups(H, 2), W, cus, 2);
    if (plan->splits > kMaxSplits)
        return SMLA_EUNSUPPORTED;
    plan->chunk = kChunk;
    plan->heads = 0;
    // the spread merge when the grid fits the compute units (every workgroup resident): its
    // merge reads are spread over all the ranges instead of one range reading the others'
    plan->merge = SMLA_MERGE_LAST;
    if (plan->splits >= 2 && plan->splits <= kMaxSpreadSplits &&
        (int64_t)B * q_len * head_groups(H, 2) * plan->splits <= cus)
        plan->merge = SMLA_MERGE_SPREAD;
    return SMLA_OK;
}

smla_status paged_mla_decode(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                             const void *cache, int64_t num_pages, int32_t page_size,
                             int64_t page_stride, const int32_t *block_table, int32_t max_pages,
                             const int32_t *lengths, int32_t B, int32_t q_len, int32_t H,
                             float bmm1_scale, float bmm2_scale, void *out, float *lse,
                             uint32_t flags, const smla_plan *plan, void *workspace,
                             size_t workspace_bytes, hipStream_t stream)
{
    if (B < 0 || q_len < 1 || H <= 0 || H % 16 != 0 || max_pages < 1 || page_size < 1 ||
        num_pages < 1 || (int64_t)max_pages * page_size > 0x7FFFFFFF ||
        (int64_t)B * q_len > 0x7FFFFFFF)
        return SMLA_EINVAL;
    if (flags & ~(SMLA_LSE_LOG2 | SMLA_P_ONE_TERM))
        return SMLA_EINVAL;
    if (!isfinite(bmm1_scale) || !isfinite(bmm2_scale))
        return SMLA_EINVAL;
    if (page_stride < (int64_t)page_size * 576 || (page_stride & 15))
        return SMLA_EINVAL;
    smla_plan chosen;
    if (plan != nullptr) {
        if (!plan_ok(plan, H))
            return SMLA_EINVAL;
        chosen = *plan;
    } else {
        const smla_status st = smla_paged_decode_plan(B, q_len, H, max_pages, page_size, flags,
                                                      &chosen);
        if (st != SMLA_OK)
            return st;
    }
    if (chosen.tiles != 2)
        return SMLA_EUNSUPPORTED;  // the paged mode is built into the 64-head kernel
    const int32_t W = max_pages * page_size;
    if ((W + chosen.splits - 1) / chosen.splits > smla::G64_MAX_RANGE)
        return SMLA_EUNSUPPORTED;
    const int32_t T = B * q_len;
    if (T == 0)
        return SMLA_OK;
    {
        const smla_status st = spread_ok(&chosen, T, H);
        if (st != SMLA_OK)
            return st;
    }
    if (q == nullptr || cache == nullptr || block_table == nullptr || lengths == nullptr ||
        out == nullptr)
        return SMLA_EINVAL;
    if (!aligned16(q) || (q_stride_t & 15) || (q_stride_h & 15) || q_stride_t < 0 ||
        q_stride_h < 0 || !aligned16(cache) || !aligned16(out) || !aligned4(block_table) ||
        !aligned4(lengths) || (lse != nullptr && !aligned4(lse)))
        return SMLA_EINVAL;
    const size_t need = smla_decode_workspace_size(&chosen, T, H);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
        return SMLA_EWORKSPACE;

    smla::DecodeParams p{};
    p.q = static_cast<const uint8_t *>(q);
    p.q_st = q_stride_t;
    p.q_sh = q_stride_h;
    p.kv_a = static_cast<const uint8_t *>(cache);
    p.kv_b = nullptr;
    p.split_col = W;
    p.indices = nullptr;
    p.lens = lengths;
    p.T = T;
    p.H = H;
    p.W = W;
    p.scale_log2 = (float)((double)bmm1_scale * 1.4426950408889634);
    p.bmm2 = bmm2_scale;
    p.sinks = nullptr;
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    p.lse_log2 = (flags & SMLA_LSE_LOG2) ? 1 : 0;
    p.splits = chosen.splits;
    p.groups = plan_groups(H, &chosen);
    p.gw = plan_heads(&chosen);
    p.merge = chosen.merge;
    p.wait_polls = g_wait_polls.load(std::memory_order_relaxed);
    p.wait_extra = g_wait_extra.load(std::memory_order_relaxed);
    p.paged = 1;
    p.block_table = block_table;
    p.max_pages = max_pages;
    p.page_size = page_size;
    p.q_len = q_len;
    p.page_stride = page_stride;
    if (need > 0) {
        const WsLayout w = ws_layout(&chosen, T, H);
        uint8_t *base = static_cast<uint8_t *>(workspace);
        p.status = reinterpret_cast<int32_t *>(base + w.status);
        p.counters = reinterpret_cast<int32_t *>(base + w.counters);
        p.ws_o = reinterpret_cast<float *>(base + w.partials);
        p.ws_ml = reinterpret_cast<float *>(base + w.ml);
    }
    const hipError_t e = smla::launch_decode_g64(p, 576, 576, (flags & SMLA_P_ONE_TERM) == 0,
                                                 false, stream);
    return e == hipSuccess ? SMLA_OK : SMLA_EHIP;
}

smla_status mla_value(const void *partials, const float *lse2, int32_t S, int32_t T, int32_t H,
                      const void *w_uv, int64_t w_stride_h, int64_t w_stride_v, const void *gate,
                      const int32_t *totals, int32_t rows_per_request, void *out, uint32_t flags,
                      hipStream_t stream)
{
    if (S < 1 || S > 64 || T < 0 || H < 1 || rows_per_request < 1 || flags != 0)
        return SMLA_EINVAL;
    if (w_stride_h < 0 || w_stride_v < 0 || (w_stride_h & 7) || (w_stride_v & 7))
        return SMLA_EINVAL;
    if (T == 0)  // empty tensors may have null data pointers
        return SMLA_OK;
    if (partials == nullptr || lse2 == nullptr || w_uv == nullptr || gate == nullptr ||
        out == nullptr)
        return SMLA_EINVAL;
    if (!aligned16(partials) || !aligned16(w_uv) || !aligned4(lse2) ||
        ((uintptr_t)gate & 1u) || ((uintptr_t)out & 1u) || (totals != nullptr && !aligned4(totals)))
        return SMLA_EINVAL;
    smla::ValueParams p;
    p.partials = static_cast<const uint16_t *>(partials);
    p.lse2 = lse2;
    p.S = S;
    p.T = T;
    p.H = H;
    p.w_uv = static_cast<const uint16_t *>(w_uv);
    p.w_sh = w_stride_h;
    p.w_sv = w_stride_v;
    p.gate = static_cast<const uint16_t *>(gate);
    p.totals = totals;
    p.rows_per_request = rows_per_request;
    p.out = static_cast<uint16_t *>(out);
    return smla::launch_mla_value(p, stream) == hipSuccess ? SMLA_OK : SMLA_EHIP;
}

smla_status smla_testing_set_merge_wait(int32_t max_polls, int32_t unreachable)
{
    if (max_polls < 0 || (unreachable != 0 && unreachable != 1))
        return SMLA_EINVAL;
    g_wait_polls.store(max_polls == 0 ? kDefaultWaitPolls : max_polls, std::memory_order_relaxed);
    g_wait_extra.store(unreachable, std::memory_order_relaxed);
    return SMLA_OK;
}

smla_status lse_merge(const void *partials, const float *lse2, int32_t S, int32_t T, int32_t H,
                      int32_t D, void *out, float *lse_out, uint32_t flags, hipStream_t stream)
{
    if (S < 1 || T < 0 || H < 1 || D < 1)
        return SMLA_EINVAL;
    if (flags & ~SMLA_LSE_LOG2)
        return SMLA_EINVAL;
    if (S > 64 || D % 8 != 0)
        return SMLA_EUNSUPPORTED;
    if (T == 0)  // empty tensors may have null data pointers
        return SMLA_OK;
    if (partials == nullptr || lse2 == nullptr || out == nullptr)
        return SMLA_EINVAL;
    if (!aligned16(partials) || !aligned16(out) || !aligned4(lse2) ||
        (lse_out != nullptr && !aligned4(lse_out)))
        return SMLA_EINVAL;
    smla::LseMergeParams p;
    p.partials = static_cast<const uint16_t *>(partials);
    p.lse2 = lse2;
    p.S = S;
    p.T = T;
    p.H = H;
    p.D = D;
    p.out = static_cast<uint16_t *>(out);
    p.lse_out = lse_out;
    p.lse_log2 = (flags & SMLA_LSE_LOG2) ? 1 : 0;
    return smla::launch_lse_merge(p, stream) == hipSuccess ? SMLA_OK : SMLA_EHIP;
}

}  // extern "C"
