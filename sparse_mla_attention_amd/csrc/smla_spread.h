// The spread split merge of the 64-head decode kernel (plan merge = SMLA_MERGE_SPREAD).
//
// Method (the attn_sparse page's merge method and module docstring, "Precision"): the S range
// partials of a (token, head group) merge in FP32, in range order, with weights 2^(m_s - M),
// M = max_s m_s, and L = sum_s 2^(m_s - M) l_s; the sink (if any) and the normalization follow
// as in a one-range call.  Every operation is the last-arriver merge's, in the same order, so
// the two merges give the same bits.
//
// Decomposition.  Before calling spread_merge, every range has stored its whole partial (FP32
// accumulators in register order, then (m, l) per head) for the group's real heads (padding
// heads past H are neither stored nor read) with device-scope stores and waited for them to
// complete.  Range s then writes the output columns of 32-column tiles [16 s / S, 16 (s + 1) /
// S) of the group's heads (512 / S columns when S divides 16):
//   1. arrival: one atomic add on the (token, head group)'s arrival counter, then a bounded
//      wait until all S ranges have arrived (the grid holds at most one workgroup per compute
//      unit, so every range is resident);
//   2. one round of loads: (m, l) of every range and head into LDS, and this range's column
//      slice of every range's partial, 16 bytes per load, all issued before any is used (the
//      slice, whole 32-column tiles, is a contiguous run of each partial);
//   3. each thread holds positions of one head: it computes that head's M, L, weights and
//      normalization from LDS, sums its positions over the ranges in range order, scales,
//      rounds to BF16 into the LDS output tile;
//   4. coalesced row stores of the slice, the LSE (range 0), and the departure count: the last
//      range to leave resets both counters.
// A range whose wait gives up counts itself in the status word, writes NaN for its columns
// (and LSE) and leaves the counters as they are.
//
// Partial layout (per range, HG heads = H2 tiles of 32): position p (16 bytes) = ((tile * H2 +
// h2) * 4 + j) * 64 + lane holds accumulator registers 4 j .. 4 j + 3 of the 32x32 P.V tile
// `tile` (columns 32 tile ..) for head tile h2, lane `lane`: head 32 h2 + lane % 32, columns
// 32 tile + 8 j + 4 (lane / 32) + 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace dev {

template <int HG, int S>
__device__ __attribute__((always_inline)) inline void spread_merge_s(
    const DecodeParams &a, uint8_t *lds, int *misc, int t, int hg, int64_t tg, int split,
    int tid, float anchor, float log2_anchor)
{
    constexpr int NT = 512;
    constexpr int H2 = HG / 32;
    constexpr int SC1 = 16;                        // device-scope (write-through) accesses
    constexpr int TPOS = 256 * H2;                 // 16-byte positions of one 32-column tile
    constexpr int MAXT = (16 + S - 1) / S;         // most tiles of one range's slice
    constexpr int PP = MAXT * TPOS / NT;           // positions per thread
    static_assert(TPOS % NT == 0 || NT % TPOS == 0, "positions split evenly over the threads");
    static_assert(TPOS >= NT, "one head per thread needs a tile's positions to cover the threads");
    const int tile0 = 16 * split / S;              // this range's tiles [tile0, tile0 + ntiles)
    const int ntiles = 16 * (split + 1) / S - tile0;
    const int lane = tid & 63;
    const int heads_here = min(a.gw, a.H - hg * a.gw);  // real heads of the group
    // positions tid + NT i share lane and head tile: one head per thread
    const int h2 = (tid >> 8) % H2;
    const int hl = lane & 31;
    const int hloc = 32 * h2 + hl;                 // head within the group
    const int head = hg * a.gw + hloc;             // (a real head only if hloc < heads_here)
    const bool active = hloc < heads_here;
    int *ctr = a.counters + 2 * tg;                // [0] arrivals, [1] departures

    // ---- 1. arrival and bounded wait ---------------------------------------------------
    if (tid == 0) {
        __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int need = S + a.wait_extra;
        int ready = 0;
        for (int spin = 0;; spin++) {
            if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need) {
                ready = 1;
                break;
            }
            if (spin >= a.wait_polls)
                break;
            __builtin_amdgcn_s_sleep(1);
        }
        *misc = ready;
        if (!ready)
            __hip_atomic_fetch_add(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const bool failed = *misc == 0;

    // ---- 2. one round of loads ------------------------------------------------------------
    // (m, l) of every range and head: [S][HG] float2 past the output tile
    float2 *gl = reinterpret_cast<float2 *>(lds + HG * 1024);
    constexpr int NML = (S * HG + NT - 1) / NT;
    float2 ml[NML];
#pragma unroll
    for (int k = 0; k < NML; k++) {
        const int i = tid + NT * k;
        ml[k] = float2{0.0f, 0.0f};
        if (i < S * HG && i % HG < heads_here) {
            const float *m = a.ws_ml + ((tg * S + i / HG) * HG + i % HG) * 2;
            ml[k] = float2{load_device(m), load_device(m + 1)};
        }
    }
    // this range's slice of every range's partial: positions pbase + tid + NT i, i below
    // ntiles * TPOS / NT
    const int pbase = tile0 * TPOS;
    const int npp = ntiles * TPOS / NT;            // this range's positions per thread
    v4i v[PP][S];
#pragma unroll
    for (int r = 0; r < S; r++) {
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(a.ws_o + (tg * S + r) * (HG * 512), 0,
                                                          HG * 512 * 4, 0x00020000);
#pragma unroll
        for (int i = 0; i < PP; i++) {
            v[i][r] = v4i{0, 0, 0, 0};
            if (active && i < npp)
                v[i][r] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, (pbase + tid + NT * i) * 16, 0, SC1);
        }
    }
#pragma unroll
    for (int k = 0; k < NML; k++) {
        const int i = tid + NT * k;
        if (i < S * HG)
            gl[i] = ml[k];
    }
    lds_barrier();  // orders LDS only: the partial loads stay in flight

    // ---- 3. this thread's head: M, L, weights, normalization; sums -----------------------
    float big_g = -INFINITY;
#pragma unroll
    for (int r = 0; r < S; r++)
        big_g = fmaxf(big_g, gl[r * HG + hloc].x);
    float l_new = 0.0f;
    float wr[S];
#pragma unroll
    for (int r = 0; r < S; r++) {
        const float2 x = gl[r * HG + hloc];
        wr[r] = x.x == -INFINITY ? 0.0f : exp2f(x.x - big_g);
        l_new += wr[r] * x.y;
    }
    const bool any = big_g != -INFINITY;
    float big_m = big_g, big_l = l_new, wgt = 1.0f;
    if (a.sinks != nullptr && hloc < heads_here) {
        const float sk = a.sinks[head] * LOG2E;
        big_m = fmaxf(big_g, sk);
        wgt = any ? exp2f(big_g - big_m) : 0.0f;
        big_l = wgt * l_new + anchor * exp2f(sk - big_m);
    }
    const float inv = failed ? __int_as_float(0x7FC00000) : any ? a.bmm2 * wgt / big_l : 0.0f;
    uint8_t *tile = lds;                           // BF16 [HG][1024 bytes]
    if (active) {
#pragma unroll
        for (int i = 0; i < PP; i++) {
            if (i >= npp)
                break;
            const int p = pbase + tid + NT * i;
            const int j = (p >> 6) & 3, ptile = p / (256 * H2);
            float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int r = 0; r < S; r++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    sum[e] += wr[r] * __int_as_float(v[i][r][e]);
            const int col = 32 * ptile + 8 * j + 4 * (lane >> 5);
            uint2 pk;
            pk.x = bf16x2(sum[0] * inv, sum[1] * inv);
            pk.y = bf16x2(sum[2] * inv, sum[3] * inv);
            *reinterpret_cast<uint2 *>(tile + tile_off(hloc, 2 * col)) = pk;
        }
    }
    if (split == 0 && (tid & 255) < 32 && (tid >> 8) < H2 && hloc < heads_here &&
        a.lse != nullptr) {
        const float lse2 = failed ? __int_as_float(0x7FC00000)
                           : any  ? big_m - log2_anchor + log2f(big_l)
                                  : -INFINITY;
        a.lse[(int64_t)t * a.H + head] = a.lse_log2 ? lse2 : lse2 * LN2;
    }
    __syncthreads();  // the tile is complete and every wave's loads have been used

    // ---- 4. row stores of the slice, departure ---------------------------------------------
    const int parts = 4 * ntiles;                  // 16-byte parts of a row in the slice
    for (int x = tid; x < heads_here * parts; x += NT) {
        const int row = x / parts, part = 4 * tile0 + x % parts;
        const v4i o = lds_load<v4i>(tile, tile_off(row, 16 * part));
        __builtin_nontemporal_store(
            o, reinterpret_cast<v4i *>(a.out + ((int64_t)t * a.H + hg * a.gw + row) * 512 +
                                       8 * part));
    }
    if (tid == 0 && !failed) {
        const int left = __hip_atomic_fetch_add(ctr + 1, 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        if (left == S - 1) {                       // the last to leave: every range has read
            __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// The spread merge of range `split` of (token t, head group hg); S = a.splits in 2 .. 16
// (checked on the host).  LDS: the BF16 output tile [HG][1024] at lds, the (m, l) of the
// ranges [S][HG] float2 after it; `misc` one int of LDS.  `anchor` is the recipe's P anchor
// (the sink's weight and the LSE are in its units).
template <int HG>
__device__ __attribute__((always_inline)) inline void spread_merge(
    const DecodeParams &a, uint8_t *lds, int *misc, int t, int hg, int64_t tg, int split,
    int tid, float anchor, float log2_anchor)
{
#define SMLA_SPREAD_CASE(n)                                                                    \
    case n: spread_merge_s<HG, n>(a, lds, misc, t, hg, tg, split, tid, anchor, log2_anchor); break;
    switch (a.splits) {
        SMLA_SPREAD_CASE(2) SMLA_SPREAD_CASE(3) SMLA_SPREAD_CASE(4) SMLA_SPREAD_CASE(5)
        SMLA_SPREAD_CASE(6) SMLA_SPREAD_CASE(7) SMLA_SPREAD_CASE(8) SMLA_SPREAD_CASE(9)
        SMLA_SPREAD_CASE(10) SMLA_SPREAD_CASE(11) SMLA_SPREAD_CASE(12) SMLA_SPREAD_CASE(13)
        SMLA_SPREAD_CASE(14) SMLA_SPREAD_CASE(15)
    default: spread_merge_s<HG, 16>(a, lds, misc, t, hg, tg, split, tid, anchor, log2_anchor); break;
    }
#undef SMLA_SPREAD_CASE
}

}  // namespace dev
}  // namespace smla
