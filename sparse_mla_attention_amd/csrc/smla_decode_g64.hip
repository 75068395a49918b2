// Sparse MLA decode for gfx950 (MI355X), 64 heads per workgroup with rows gathered straight
// into LDS.
//
// Method (vLLM API pages): the formula is the sparse_mla_cute page's "What this module
// computes"; the E4M3-P recipe, the contiguous key split and the split merge are the
// attn_sparse page's module docstring and its SparseDcpDecode.kernel / merge methods.  The
// arithmetic is that of the 32-head kernel (smla_decode.hip), operation for operation: the
// same QK instruction chains, the same running maxima and rescale factors, E4M3 P (two-term
// by default) at 448 of the running maximum, the same accumulator rescales, the same order of
// the FP32 sums of the unquantized P and the same fused split merge, so under one split plan
// the two kernels agree bit for bit.
//
// Why this decomposition.  The 32-head kernel pays a chunk's fixed costs (row-load issue,
// index reads, score exchange, barriers) once per 32 heads, and its scattered row loads into
// registers cap the gather near 9 bytes per clock per CU.  Here one workgroup serves 64 heads,
// and the rows go from memory to LDS without passing through registers
// (global_load_lds_dwordx4: measured at 6 TB/s from HBM and ~9 TB/s when the two head groups
// of a token meet in the XCD's L2).  Two roles share each SIMD, as in the 32-head kernel, so
// one role's vector work overlaps the other's matrix work:
//   QK waves (0..3): wave w takes head tile w (16 heads) over all 64 keys of a chunk:
//     S^T tiles of 16 keys x 16 heads on v_mfma_scale_f32_16x16x128_f8f6f4 (K read from the
//     slot, Q fragments held in registers, the rope step on two 16x16x32 FP8 instructions),
//     then the softmax of its heads over the whole chunk (no exchange of maxima): running
//     maximum, rescale factor, E4M3 P (two-term by default) and the factor into a P buffer.
//   P.V waves (4..7): wave 4 + j owns output columns 128 j .. 128 j + 127 of all 64 heads:
//     O^T *= alpha (per head), then O^T (32 columns x 32 heads) += V^T (ds_read_b64_tr_b8 from
//     the slot) P^T on
//     v_mfma_scale_f32_32x32x64_f8f6f4, 4 column tiles x 2 head tiles (x 2 with two-term P).
//     It also gathers its own column slice of every chunk (and a quarter of the rope rows).
// Slot (one gathered chunk): four slices of 8 KB, slice j holding latent pieces 8 j .. 8 j + 7
//   of the 64 rows (row pitch 128 bytes, piece q of row k at position q ^ f(k), f(k) =
//   2 ((k >> 1) & 3) + ((k >> 3) & 1), which keeps the QK reads of 16 rows and the transposed
//   V reads of 8 rows x 2 pieces on distinct banks), then 4 KB of rope rows (pitch 64 bytes,
//   rope piece q at position q ^ ((k >> 2) & 3)).  Each load instruction fills 1 KB of a slot
//   (lane l -> 16 bytes at l * 16), so a lane fetches whichever row piece the layout puts
//   there; masked columns fetch a static zero row.  The 64-bit source row address of every
//   column of the range is staged in LDS once.
// Iteration c (one LDS-only barrier): the QK waves compute QK and softmax of chunk c (P into
//   buffer c & 1); each P.V wave computes P.V of chunk c-1 from its slice of slot c-1 and P
//   buffer (c-1) & 1, then refills that slice with chunk c+2 (the loads of a slice are issued
//   from inline assembly after the wave's own reads of it, and waited for with explicit
//   counts before the barrier that publishes the chunk).  Three slots hold chunks c-1 .. c+1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_device.h"
#include "smla_internal.h"
#include "smla_spread.h"

namespace smla {
namespace {

using namespace dev;

constexpr int CHUNK = 64;                          // columns per chunk
constexpr int NT = 512;                            // threads per workgroup (8 waves)
constexpr int HG = 64;                             // heads per workgroup
constexpr int SLOTS = 3;                           // gathered chunks in LDS
constexpr int SLICE = CHUNK * 128;                 // one 128-column slice of a slot
constexpr int NCT = 4;                             // 32-column P.V tiles per P.V wave

// Masked columns gather this row, so their bytes are zero (0 * anything stays finite); it is as
// long as the longest row (656 bytes).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row_g64[656];

// Position swizzle of the 8 pieces of a latent row within its slice.
__device__ inline int fsw(int k) { return (((k >> 1) & 3) << 1) | ((k >> 3) & 1); }

// Rope position swizzle of the 8 BF16 rope pieces of a 656-byte row.
__device__ inline int rsw(int k) { return (k >> 1) & 7; }

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Eight E4M3 values (bytes of w0, then w1), each times its scale, rounded to BF16 (exact when
// the scales are powers of two).
__device__ inline v8bf e4m3x8_bf16(int w0, int w1, v4f s0, v4f s1)
{
    const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
    const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
    const v2f c = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
    const v2f d = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
    v8bf r;
    r[0] = (__bf16)(a[0] * s0[0]);
    r[1] = (__bf16)(a[1] * s0[1]);
    r[2] = (__bf16)(b[0] * s0[2]);
    r[3] = (__bf16)(b[1] * s0[3]);
    r[4] = (__bf16)(c[0] * s1[0]);
    r[5] = (__bf16)(c[1] * s1[1]);
    r[6] = (__bf16)(d[0] * s1[2]);
    r[7] = (__bf16)(d[1] * s1[3]);
    return r;
}

__device__ inline v8bf as_bf16x8(v4i x) { return __builtin_bit_cast(v8bf, x); }

// LDS carve-up (byte offsets); TAIL: 576-byte QK on E4M3 rows (an E4M3 rope region per slot);
// DS: 656-byte fp8_ds_mla rows (a BF16 rope region of 64 rows x 128 bytes per slot, and the
// chunks' [4 blocks][64 keys] FP32 scale tables in a ring of four past the slots, so that the
// refill of a slot leaves the scales of the chunk it held for the P.V products that follow).
template <bool TAIL, bool DS>
struct LdsG {
    static constexpr int LAT = 4 * SLICE;                      // latent region of a slot
    static constexpr int DROPE = LAT;                          // DS: [64][128 bytes] rope
    static constexpr int SLOTB = LAT + (DS ? CHUNK * 128 : TAIL ? CHUNK * 64 : 0);
    static constexpr int V = 0;                                // [SLOTS] slots
    static constexpr int DSR = SLOTS * SLOTB;                  // DS: [4][4][64] float scales
    static constexpr int DSRB = 4 * CHUNK * 4;                 // DS: one chunk's table
    static constexpr int P = DSR + (DS ? 4 * DSRB : 0);        // [2 buf][2 term][64][64 keys]
    static constexpr int PTERM = HG * 64;
    static constexpr int PBUF = 2 * PTERM;
    static constexpr int SCL = P + 2 * PBUF;                   // [2 buf][64] float: alpha
    static constexpr int FIN = SCL + 2 * HG * 4;               // [4 key quarters][64] l, [64] m
    static constexpr int ADDR = FIN + 6 * HG * 4;              // [G64_MAX_RANGE] row addresses
    static constexpr int MISC = ADDR + G64_MAX_RANGE * 8;      // ticket, spare, wait outcome
    static constexpr int TOTAL = MISC + 16;
    static constexpr int OUT_TILE = HG * 1024;                 // BF16 [64][512], after the loop
    static_assert(OUT_TILE <= P, "output tile must fit in the slots");
    static_assert(OUT_TILE + 16 * HG * 8 <= P, "(m, l) of 16 ranges must fit past the tile");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// One LDS-direct load of 4 bytes per lane: lane l's bytes from `src` go to LDS byte m0 + 4 l.
__device__ inline void lds_dma4(uint64_t src, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(src), "s"(m0));
}

// One LDS-direct load: each lane's 16 bytes from `src` go to LDS byte m0 + 16 * lane.  Issued
// from inline assembly so that the compiler's wait counting does not see it (it would wait for
// every outstanding load before any LDS read); the kernel waits with explicit counts.  M0 is
// written here and used by nothing else in this kernel.
__device__ inline void lds_dma16(uint64_t src, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0));
}

// The same load at device scope (sc1: misses in the non-coherent caches), for the split
// exchange's partials written by another compute unit.
__device__ inline void lds_dma16_dev(uint64_t src, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off sc1"
                 :
                 : "v"(src), "s"(m0)
                 : "m0");
}

// LDS byte offset where the two-range spread merge lands the other range's half partial
// (64 KB, past the BF16 output tile).
constexpr int PAIR_LZ = 64 * 1024;

template <int N>
__device__ inline void wait_dma()
{
    asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory");
}

// Which 16-byte pieces lane group g of a QK wave holds (the same for Q and K, so the products
// are unchanged): latent pieces 8 s + qk_pg(g) and 8 s + 4 + qk_pg(g) of step s, rope piece
// 32 + qk_pr(g).  The two lane groups that share an LDS pass (g = 2h, 2h + 1) then read
// disjoint bank sets under the slot swizzles, so the K reads run without bank conflicts.
__device__ inline int qk_pg(int g) { return ((g & 1) << 1) | (g >> 1); }
__device__ inline int qk_pr(int g) { return g ^ ((g & 1) << 1); }

// LDS byte address (M0 operand) of a pointer into the workgroup's LDS.
__device__ inline uint32_t lds_addr(const uint8_t *p)
{
    return (uint32_t)(uintptr_t)(const SMLA_LDS(uint8_t) *)p;
}

// CLA: the chunk-local recipe (the sparse_mla_cute page, "How."): every key range is one
// 128-column window of the token's columns, [128 s, 128 s + 128) for range s, whose P is
// anchored at 256 of the window's own maximum (one softmax over both 64-column chunks, no
// running maximum); the ranges then merge as split partials.  Otherwise the attn_sparse
// page's recipe: contiguous ranges of ceil(n / splits) columns, P at 448 of the running
// maximum.
template <int RB, int QK, bool TWO, bool DIST, bool CLA, bool PAIR, bool SPI>
__global__ void __launch_bounds__(NT, 1) decode_g64_kernel(DecodeParams a)
{
    // DS: 656-byte fp8_ds_mla rows (E4M3 latent with an FP32 scale per 128 elements, BF16
    // rope): the QK products of each 128-element block are scaled per key, the rope product
    // runs in BF16, and the P.V waves dequantize their 128 columns of V to BF16
    constexpr bool DS = RB == 656;
    constexpr bool TAIL = QK == 576 && !DS;        // a fifth, 64-byte E4M3 QK step (rope)
    constexpr int NDMA = DS ? 11 : TAIL ? 9 : 8;   // loads per P.V wave and chunk
    constexpr float AN = CLA ? 256.0f : ANCHOR;    // P anchor
    constexpr float LOG2_AN = CLA ? 8.0f : LOG2_ANCHOR;
    using L = LdsG<TAIL, DS>;

    __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];
    static_assert(PAIR_LZ + 64 * 1024 <= L::TOTAL, "two-range spread landing zone");

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const bool qk_wave = wave < 4;
    const int w = wave & 3;                        // QK: head tile; P.V: column slice

    int t, unit;
    unit_of(blockIdx.x, a.T, a.splits * a.groups, &t, &unit);
    const int hg = unit % a.groups;
    const int split = unit / a.groups;

    const int32_t *idx_row = a.indices + (int64_t)t * a.W;
    // SPI: the indices of every column this range can hold whatever the token's count turns
    // out to be are loaded alongside the count rather than after it: columns [0, (split + 1)
    // ceil(W / splits)), column tid + NT k in raw_s[k], when they are at most SPEC per thread
    // (sparse mode).  Used for grids that fill the device (it saves a dependent load there;
    // measured slower for small grids, which take the instantiation without it).
    constexpr int SPEC = 4;
    const int spec_hi = SPI ? min(a.W, (split + 1) * ((a.W + a.splits - 1) / a.splits)) : 0;
    const bool spec = SPI && !a.paged && spec_hi <= SPEC * NT;
    int raw_s[SPEC];
    if constexpr (SPI) {
#pragma unroll
        for (int k = 0; k < SPEC; k++) {
            const int c = tid + NT * k;
            raw_s[k] = spec && c < spec_hi ? idx_row[c] : -1;
        }
    }
    // the token's active count: lens[t] (sparse), or its request's context length less the
    // causal offset of its row (paged)
    const int req = a.paged ? t / a.q_len : t;
    int n = a.lens[req];
    if (a.paged)
        n -= a.q_len - 1 - (t - req * a.q_len);
    n = n < 0 ? 0 : (n > a.W ? a.W : n);
    const int per = CLA ? 2 * CHUNK : (n + a.splits - 1) / a.splits;
    const int first = min(n, split * per);
    // the host keeps every range within the staging buffer; the clamp only keeps LDS accesses
    // in bounds
    const int mine = min(min(n - first, per), G64_MAX_RANGE);
    const int nch = (mine + CHUNK - 1) / CHUNK;


    const uint64_t *addr = reinterpret_cast<const uint64_t *>(lds + L::ADDR);
    float *fin = reinterpret_cast<float *>(lds + L::FIN);  // [4][64] l, [64] m
    float *scl = reinterpret_cast<float *>(lds + L::SCL);  // [2][64] alpha per chunk
    const uint64_t zero = (uint64_t)(uintptr_t)g_zero_row_g64;

    // ---- source address of every column of the range: its row, or the zero row when the
    // column is masked (index -1) or lies past the range (tail of the last chunk)
    {
        const uint8_t *pool_a = a.kv_a, *pool_b = a.kv_b != nullptr ? a.kv_b : a.kv_a;
        const int split_col = a.kv_b != nullptr ? a.split_col : a.W;
        uint64_t *ad = reinterpret_cast<uint64_t *>(lds + L::ADDR);
        if (spec) {
            // [first, first + mine) lies within the loaded columns; the tail of the last
            // chunk reads the zero row
#pragma unroll
            for (int k = 0; k < SPEC; k++) {
                const int c = tid + NT * k;
                const int i = c - first;
                if (i >= 0 && i < mine)
                    ad[i] = raw_s[k] < 0 ? zero
                                         : (uint64_t)(uintptr_t)((c >= split_col ? pool_b : pool_a) +
                                                                 (int64_t)raw_s[k] * RB);
            }
            for (int i = mine + tid; i < nch * CHUNK; i += NT)
                ad[i] = zero;
        } else
        for (int i = tid; i < nch * CHUNK; i += NT) {
            uint64_t src = zero;
            if (i < mine) {
                if (a.paged) {
                    const int k = first + i;
                    const int page = a.block_table[(int64_t)req * a.max_pages + k / a.page_size];
                    src = (uint64_t)(uintptr_t)(pool_a + (int64_t)page * a.page_stride +
                                                (int64_t)(k % a.page_size) * RB);
                } else {
                    const int raw = idx_row[first + i];
                    if (raw >= 0)
                        src = (uint64_t)(uintptr_t)((first + i >= split_col ? pool_b : pool_a) +
                                                    (int64_t)raw * RB);
                }
            }
            ad[i] = src;
        }
    }
    __syncthreads();                               // the only full fence before the loop

    // ---- epilogue (every wave; `acc` holds the P.V waves' accumulators) ---------------------
    // acc[ct][h2]: O^T tile of columns 32 (4 w + ct) + .. x heads 32 h2 + ..; lane l holds head
    // 32 h2 + l % 32, columns 8 (rr / 4) + 4 (l / 32) + rr % 4 of the tile in register rr.
    auto epilogue = [&](v16f(&acc)[NCT][2]) __attribute__((always_inline)) {
        lds_barrier();
        const int hl = lane & 31, u = lane >> 5;
        float g_h[2], l_h[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            const int head = 32 * h2 + hl;
            g_h[h2] = fin[4 * HG + head];
            l_h[h2] = ((fin[head] + fin[HG + head]) + fin[2 * HG + head]) + fin[3 * HG + head];
        }
        const int64_t tg = (int64_t)t * a.groups + hg;
        // A range's partial: its FP32 accumulators as they stand (at 448 of the range's running
        // maximum m, not normalized) and (m, l) per head.  Byte offset of accumulator registers
        // 4 j .. 4 j + 3 of tile (ct, h2) of P.V wave w: 16 bytes per lane, one 1 KB run per (tile,
        // j) across the wave, so every store and load of the exchange is one 16-byte access per lane.
        auto part_off = [&](int ct, int h2, int j) {
            return ((((NCT * w + ct) * 2 + h2) * 4 + j) * 64 + lane) * 16;
        };
        constexpr int SC1 = 16;  // cache policy of device-scope (write-through) accesses
        auto part_rsrc = [&](int64_t unit) {
            return __builtin_amdgcn_make_buffer_rsrc(a.ws_o + unit * (HG * 512), 0, HG * 512 * 4,
                                                     0x00020000);
        };
        // two-range spread merge: range s writes output columns 256 s .. 256 s + 255, the column
        // tiles of P.V waves 2 s and 2 s + 1 (`merging`); the other two P.V waves store theirs
        const bool pair = PAIR && a.splits == 2;
        const bool merging = !qk_wave && (w >> 1) == split;
        // the FP32 merge of two ranges' values in range order, x0 from range 0 (the last-arriver
        // merge's operations: both two-range merges give the same bits)
        auto merge2 = [](float w0, float x0, float w1, float x1) {
            float sum = 0.0f;
            sum += w0 * x0;
            sum += w1 * x1;
            return sum;
        };
        bool failed = false;
        if (pair) {
            // Each range stores only the half of its partial that the other range merges (the
            // column tiles of the other pair of P.V waves) and its (m, l), arrives, and waits
            // (bounded) for the other range.  The other range's half for this range's columns
            // then comes into LDS in one round of LDS-direct loads issued by all eight waves,
            // and the P.V waves of this half merge it with their own accumulators in registers:
            // the last-arriver merge's FP32 operations in the same order (range 0's term first),
            // so the two merges give the same bits.
            const int64_t ui = tg * 2 + split, uo = tg * 2 + (1 - split);
            const int heads_here = min(a.gw, a.H - hg * a.gw);
            int *misc = reinterpret_cast<int *>(lds + L::MISC);
            int *ctr = a.counters + 2 * tg;        // [0] arrivals, [1] departures
            if (!qk_wave && !merging) {
                // (the accumulator stores went out right after the chunk loop)
                if (w == 2 * (1 - split) && u == 0) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++) {
                        if (32 * h2 + hl >= heads_here)
                            continue;
                        store_device(a.ws_ml + (ui * HG + 32 * h2 + hl) * 2 + 0, g_h[h2]);
                        store_device(a.ws_ml + (ui * HG + 32 * h2 + hl) * 2 + 1, l_h[h2]);
                    }
                }
                __builtin_amdgcn_s_waitcnt(0);     // this wave's stores have completed
            }
            __syncthreads();
            if (tid == 0) {
                __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const int need = 2 + a.wait_extra;
                int ready = 0;
                for (int spin = 0;; spin++) {
                    if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                        need) {
                        ready = 1;
                        break;
                    }
                    if (spin >= a.wait_polls)
                        break;
                    __builtin_amdgcn_s_sleep(1);
                }
                misc[2] = ready;
                if (!ready)
                    __hip_atomic_fetch_add(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            failed = misc[2] == 0;
            // the other range's (m, l) of this lane's heads, and its half for this range's
            // columns: positions 4096 split .. 4096 split + 4095 of its block (64 runs of 1 KB,
            // run k = (tile * 2 + h2) * 4 + j) into LDS at PAIR_LZ + 1024 k, eight runs a wave;
            // runs of padding heads are not loaded
            float og[2], ol[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                const int64_t m = (uo * HG + 32 * h2 + hl) * 2;
                og[h2] = 32 * h2 + hl < heads_here ? load_device(a.ws_ml + m) : -INFINITY;
                ol[h2] = 32 * h2 + hl < heads_here ? load_device(a.ws_ml + m + 1) : 0.0f;
            }
            {
                const uint64_t src = (uint64_t)(uintptr_t)(a.ws_o + uo * (HG * 512)) +
                                     (uint64_t)(4096 * split + 64 * 8 * wave + lane) * 16;
                const uint32_t dst = lds_addr(lds) + PAIR_LZ + 8192 * wave;
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const int h2k = ((8 * wave + k) >> 2) & 1;
                    if (32 * h2k + hl < heads_here)
                        lds_dma16_dev(src + 1024 * k, dst + 1024 * k);
                }
                wait_dma<0>();
            }
            lds_barrier();
            float w_s[2][2];  // [range][h2]: weight 2^(m_s - M) of the range's accumulators
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                const float gr[2] = {split == 0 ? g_h[h2] : og[h2], split == 1 ? g_h[h2] : og[h2]};
                const float lr[2] = {split == 0 ? l_h[h2] : ol[h2], split == 1 ? l_h[h2] : ol[h2]};
                g_h[h2] = fmaxf(fmaxf(-INFINITY, gr[0]), gr[1]);
                l_h[h2] = 0.0f;
#pragma unroll
                for (int r = 0; r < 2; r++) {
                    w_s[r][h2] = gr[r] == -INFINITY ? 0.0f : exp2f(gr[r] - g_h[h2]);
                    l_h[h2] += w_s[r][h2] * lr[r];
                }
            }
            if (merging) {
                // run of tile (4 w + ct), head tile h2, registers 4 j .. 4 j + 3: k = ((4 (w & 1)
                // + ct) * 2 + h2) * 4 + j of the landing zone
#pragma unroll
                for (int ct = 0; ct < NCT; ct++) {
                    v4i x[2][4];
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            x[h2][j] = lds_load<v4i>(
                                lds, PAIR_LZ + (((4 * (w & 1) + ct) * 2 + h2) * 4 + j) * 1024 +
                                         16 * lane);
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                        for (int rr = 0; rr < 16; rr++) {
                            const float xo = __int_as_float(x[h2][rr >> 2][rr & 3]);
                            const float xs = acc[ct][h2][rr];
                            // range order: range 0's term first
                            const float x0 = split == 0 ? xs : xo;
                            const float x1 = split == 1 ? xs : xo;
                            acc[ct][h2][rr] = merge2(w_s[0][h2], x0, w_s[1][h2], x1);
                        }
                    // one column tile's reads at a time (they would not fit in registers
                    // beside the accumulators all at once)
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else if (DIST && !PAIR && a.splits > 1) {
            // Spread merge: every range stores its whole partial (the group's real heads only:
            // padding heads past H are never merged), then merges its own column slice of all
            // of them and writes it (smla_spread.h).
            const int64_t ui = tg * a.splits + split;
            const int heads_here = min(a.gw, a.H - hg * a.gw);
            if (!qk_wave) {
                const auto rs = part_rsrc(ui);
#pragma unroll
                for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++) {
                        if (32 * h2 + hl >= heads_here)
                            continue;
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                v4i{__float_as_int(acc[ct][h2][4 * j]),
                                    __float_as_int(acc[ct][h2][4 * j + 1]),
                                    __float_as_int(acc[ct][h2][4 * j + 2]),
                                    __float_as_int(acc[ct][h2][4 * j + 3])},
                                rs, part_off(ct, h2, j), 0, SC1);
                    }
            }
            if (wave == 4 && u == 0) {
#pragma unroll
                for (int h2 = 0; h2 < 2; h2++) {
                    if (32 * h2 + hl >= heads_here)
                        continue;
                    store_device(a.ws_ml + (ui * HG + 32 * h2 + hl) * 2 + 0, g_h[h2]);
                    store_device(a.ws_ml + (ui * HG + 32 * h2 + hl) * 2 + 1, l_h[h2]);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
            __syncthreads();
            spread_merge<HG>(a, lds, reinterpret_cast<int *>(lds + L::MISC) + 2, t, hg, tg, split,
                             tid, AN, LOG2_AN);
            return;
        } else if (!DIST && a.splits > 1) {
            // Split merge.  Each range takes an arrival ticket first.  Every range but the last
            // writes its partial (FP32 accumulators in register order, then (m, l) per head)
            // with device-scope (write-through) stores, waits for them to complete and bumps
            // the ready count; the last range waits until the ready count shows every other
            // partial, then merges all of them in range order, its own from registers.  The
            // writers are running when the last range waits (they hold earlier tickets and
            // wait on nothing), so the wait ends; it is also bounded: a range that gives up
            // counts itself in the workspace's status word, writes NaN for its heads and
            // leaves the counters as they are.
            int *misc = reinterpret_cast<int *>(lds + L::MISC);  // ticket, spare, wait outcome
            int *ctr = a.counters + 2 * tg;         // [0] arrival ticket, [1] ready count
            if (tid == 0)
                misc[0] = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (misc[0] != a.splits - 1) {
                const int64_t ui = tg * a.splits + split;
                if (!qk_wave) {
                    const auto rs = part_rsrc(ui);
#pragma unroll
                    for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                        for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                __builtin_amdgcn_raw_buffer_store_b128(
                                    v4i{__float_as_int(acc[ct][h2][4 * j]),
                                        __float_as_int(acc[ct][h2][4 * j + 1]),
                                        __float_as_int(acc[ct][h2][4 * j + 2]),
                                        __float_as_int(acc[ct][h2][4 * j + 3])},
                                    rs, part_off(ct, h2, j), 0, SC1);
                }
                if (wave == 4 && u == 0) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++) {
                        store_device(a.ws_ml + (ui * HG + 32 * h2 + hl) * 2 + 0, g_h[h2]);
                        store_device(a.ws_ml + (ui * HG + 32 * h2 + hl) * 2 + 1, l_h[h2]);
                    }
                }
                __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
                __syncthreads();
                if (tid == 0)
                    __hip_atomic_fetch_add(ctr + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
            if (tid == 0) {
                const int need = a.splits - 1 + a.wait_extra;
                int ready = 0;
                for (int spin = 0;; spin++) {
                    if (__hip_atomic_load(ctr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >=
                        need) {
                        ready = 1;
                        break;
                    }
                    if (spin >= a.wait_polls)
                        break;
                    __builtin_amdgcn_s_sleep(1);
                }
                misc[2] = ready;
                if (!ready)
                    __hip_atomic_fetch_add(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            __syncthreads();
            // A range that gave up writes NaN rows and LSEs (final part); what it merges then is
            // never used, and every workspace address it reads is in bounds either way.
            failed = misc[2] == 0;
            // Merge in range order, own partial from registers, the others' from the workspace
            // (FP32 throughout: the result does not depend on which range arrived last).
            float own_g[2], own_l[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                own_g[h2] = g_h[h2];
                own_l[h2] = l_h[h2];
            }
            if (a.splits == 2) {
                // Two ranges: the other range's (m, l) and its first column tile come in one
                // round trip, and each column tile's loads go out before the previous one is
                // summed.
                const int other = 1 - split;
                const int64_t uo = tg * 2 + other;
                float og[2], ol[2];
                v4i cur[2][4], nxt[2][4];
                if (!qk_wave) {
                    const auto rs = part_rsrc(uo);
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            cur[h2][j] = __builtin_amdgcn_raw_buffer_load_b128(
                                rs, part_off(0, h2, j), 0, SC1);
                }
#pragma unroll
                for (int h2 = 0; h2 < 2; h2++) {
                    const int64_t m = (uo * HG + 32 * h2 + hl) * 2;
                    og[h2] = load_device(a.ws_ml + m);
                    ol[h2] = load_device(a.ws_ml + m + 1);
                }
                float w_s[2][2];  // [range][h2]: weight 2^(m_s - M) of the range's accumulators
#pragma unroll
                for (int h2 = 0; h2 < 2; h2++) {
                    const float gr[2] = {split == 0 ? own_g[h2] : og[h2],
                                         split == 1 ? own_g[h2] : og[h2]};
                    const float lr[2] = {split == 0 ? own_l[h2] : ol[h2],
                                         split == 1 ? own_l[h2] : ol[h2]};
                    g_h[h2] = fmaxf(fmaxf(-INFINITY, gr[0]), gr[1]);
                    l_h[h2] = 0.0f;
#pragma unroll
                    for (int r = 0; r < 2; r++) {
                        w_s[r][h2] = gr[r] == -INFINITY ? 0.0f : exp2f(gr[r] - g_h[h2]);
                        l_h[h2] += w_s[r][h2] * lr[r];
                    }
                }
                if (!qk_wave) {
                    const auto rs = part_rsrc(uo);
#pragma unroll
                    for (int ct = 0; ct < NCT; ct++) {
                        if (ct + 1 < NCT) {
#pragma unroll
                            for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                                for (int j = 0; j < 4; j++)
                                    nxt[h2][j] = __builtin_amdgcn_raw_buffer_load_b128(
                                        rs, part_off(ct + 1, h2, j), 0, SC1);
                        }
#pragma unroll
                        for (int h2 = 0; h2 < 2; h2++) {
#pragma unroll
                            for (int rr = 0; rr < 16; rr++) {
                                const float xo = __int_as_float(cur[h2][rr >> 2][rr & 3]);
                                const float xs = acc[ct][h2][rr];
                                const float x0 = split == 0 ? xs : xo;
                                const float x1 = split == 1 ? xs : xo;
                                acc[ct][h2][rr] = merge2(w_s[0][h2], x0, w_s[1][h2], x1);
                            }
                        }
                        if (ct + 1 < NCT) {
#pragma unroll
                            for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                                for (int j = 0; j < 4; j++)
                                    cur[h2][j] = nxt[h2][j];
                        }
                    }
                }
            } else {
#pragma unroll
                for (int h2 = 0; h2 < 2; h2++) {
                    const int head = 32 * h2 + hl;
                    float big_g = -INFINITY;
                    for (int s = 0; s < a.splits; s++) {
                        const float gs =
                            s == split ? own_g[h2]
                                       : load_device(a.ws_ml + ((tg * a.splits + s) * HG + head) * 2);
                        big_g = fmaxf(big_g, gs);
                    }
                    g_h[h2] = big_g;
                    l_h[h2] = 0.0f;
                    for (int s = 0; s < a.splits; s++) {
                        const int64_t us = tg * a.splits + s;
                        const float gs =
                            s == split ? own_g[h2] : load_device(a.ws_ml + (us * HG + head) * 2);
                        const float ls =
                            s == split ? own_l[h2] : load_device(a.ws_ml + (us * HG + head) * 2 + 1);
                        l_h[h2] += (gs == -INFINITY ? 0.0f : exp2f(gs - g_h[h2])) * ls;
                    }
                }
                if (!qk_wave) {
                    // one column tile at a time: its loads of one range are issued together
#pragma unroll
                    for (int ct = 0; ct < NCT; ct++) {
                        v16f sum[2] = {v16f{}, v16f{}};
                        for (int s = 0; s < a.splits; s++) {
                            const int64_t us = tg * a.splits + s;
                            float w_s[2];
#pragma unroll
                            for (int h2 = 0; h2 < 2; h2++) {
                                const float gs =
                                    s == split ? own_g[h2]
                                               : load_device(a.ws_ml + (us * HG + 32 * h2 + hl) * 2);
                                w_s[h2] = gs == -INFINITY ? 0.0f : exp2f(gs - g_h[h2]);
                            }
                            if (s == split) {
#pragma unroll
                                for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                                    for (int rr = 0; rr < 16; rr++)
                                        sum[h2][rr] += w_s[h2] * acc[ct][h2][rr];
                            } else {
                                const auto rs = part_rsrc(us);
                                v4i v[2][4];
#pragma unroll
                                for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                                    for (int j = 0; j < 4; j++)
                                        v[h2][j] = __builtin_amdgcn_raw_buffer_load_b128(
                                            rs, part_off(ct, h2, j), 0, SC1);
#pragma unroll
                                for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                                    for (int rr = 0; rr < 16; rr++)
                                        sum[h2][rr] += w_s[h2] * __int_as_float(v[h2][rr >> 2][rr & 3]);
                            }
                        }
                        acc[ct][0] = sum[0];
                        acc[ct][1] = sum[1];
                    }
                }
            }
            if (tid == 0 && !failed) {  // every range has arrived and been merged: ready for
                                        // the next call
                __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }

        // ---- final: sink, normalization, BF16 tile in LDS, coalesced row stores, LSE ------
        uint8_t *tile = lds;  // [64][1024 bytes], over the slots
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            // real heads are the group's first min(gw, H - hg gw); the index of a padding head
            // may name a real head of another group, so padding is tested on the local index
            const bool real = 32 * h2 + hl < min(a.gw, a.H - hg * a.gw);
            const int head = hg * a.gw + 32 * h2 + hl;
            const bool any = g_h[h2] != -INFINITY;
            float big_m = g_h[h2], big_l = l_h[h2], wgt = 1.0f;
            if (a.sinks != nullptr && real) {
                const float sk = a.sinks[head] * LOG2E;
                big_m = fmaxf(g_h[h2], sk);
                wgt = any ? exp2f(g_h[h2] - big_m) : 0.0f;
                big_l = wgt * l_h[h2] + AN * exp2f(sk - big_m);
            }
            const float inv = failed ? __int_as_float(0x7FC00000) : any ? a.bmm2 * wgt / big_l : 0.0f;
            if (!qk_wave && (!pair || merging)) {
#pragma unroll
                for (int ct = 0; ct < NCT; ct++) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int col = 32 * (NCT * w + ct) + 8 * i + 4 * u;
                        uint2 pk;
                        pk.x = bf16x2(acc[ct][h2][4 * i] * inv, acc[ct][h2][4 * i + 1] * inv);
                        pk.y = bf16x2(acc[ct][h2][4 * i + 2] * inv, acc[ct][h2][4 * i + 3] * inv);
                        *reinterpret_cast<uint2 *>(tile + tile_off((32 * h2 + hl), 2 * col)) = pk;
                    }
                }
            }
            if (wave == 4 && u == 0 && real && a.lse != nullptr && (!pair || split == 0)) {
                const float lse2 = failed ? __int_as_float(0x7FC00000)
                                   : any  ? big_m - LOG2_AN + log2f(big_l)
                                          : -INFINITY;
                a.lse[(int64_t)t * a.H + head] = a.lse_log2 ? lse2 : lse2 * LN2;
            }
        }
        lds_barrier();
        const int heads_here = min(a.gw, a.H - hg * a.gw);
        // row parts (16 bytes) written: all 64, or this range's 32 under the two-range spread
        const int np = pair ? 32 : 64, p0 = pair ? 32 * split : 0;
        for (int x = tid; x < heads_here * np; x += NT) {
            const int row = x / np, part = p0 + x % np;
            const v4i v = lds_load<v4i>(tile, tile_off(row, 16 * part));
            // streaming store: the output is not read again by this kernel
            __builtin_nontemporal_store(
                v, reinterpret_cast<v4i *>(a.out + ((int64_t)t * a.H + hg * a.gw + row) * 512 +
                                           8 * part));
        }
        if (pair && tid == 0 && !failed) {
            int *ctr = a.counters + 2 * ((int64_t)t * a.groups + hg);
            const int left = __hip_atomic_fetch_add(ctr + 1, 1, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT);
            if (left == 1) {  // the last to leave: both ranges have read the arrival count
                __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(ctr + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };

    if (qk_wave) {
        // =================================== QK waves =======================================
        const int r = lane & 15, g = lane >> 4;    // row r of a 16-key tile, lane group g
        const int head = 16 * w + r;               // this lane's head within the group

        const int pg = qk_pg(g), pr = qk_pr(g);
        // Q fragments, B operand of QK: lane (n, g) holds head 16 w + n.
        v8i qf[4];
        v4i qt = v4i{0, 0, 0, 0};
        v8bf qrope[DS ? 2 : 1];                    // DS: the rope of q in BF16
        {
            // a padding head computes with the group's first head's q: its scores reach no
            // output, and no instruction between here and the first product waits for these
            // loads
            const int gh = hg * a.gw + (head < min(a.gw, a.H - hg * a.gw) ? head : 0);
            const uint8_t *qp = a.q + (int64_t)t * a.q_st + (int64_t)gh * a.q_sh;
#pragma unroll
            for (int s = 0; s < 4; s++)
                qf[s] = join(gload(qp + 16 * (8 * s + pg)), gload(qp + 16 * (8 * s + 4 + pg)));
            if (TAIL)
                qt = gload(qp + 16 * (32 + pr));
            if constexpr (DS) {
                // rope elements 8 (4 q2 + g) .. + 7 of this lane's head, in BF16 (exact)
                const v4f one = v4f{1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
                for (int q2 = 0; q2 < 2; q2++) {
                    const uint2 w = *reinterpret_cast<const uint2 *>(qp + 512 + 8 * (4 * q2 + g));
                    qrope[q2] = e4m3x8_bf16((int)w.x, (int)w.y, one, one);
                }
            }
        }

        // per-lane LDS offsets (loop invariant): pieces pg and 4 + pg of slice s of row 16 kt + r
        // at kb0 / kb1 + s * SLICE + kt * 2048; rope piece 32 + pr at rb + kt * 1024
        const int kb0 = r * 128 + 16 * (pg ^ fsw(r));
        const int kb1 = r * 128 + 16 * ((4 + pg) ^ fsw(r));
        const int rb = L::LAT + r * 64 + 16 * (pr ^ ((r >> 2) & 3));
        int rbd[2] = {0, 0};                       // DS: rope pieces 4 q2 + g of row 16 kt + r
        if constexpr (DS) {
#pragma unroll
            for (int q2 = 0; q2 < 2; q2++)
                rbd[q2] = L::DROPE + r * 128 + 16 * ((4 * q2 + g) ^ rsw(r));
        }
        int pw[4];                                 // P bytes of key tile kt in a P buffer
#pragma unroll
        for (int kt = 0; kt < 4; kt++)
            pw[kt] = head * 64 + 16 * (kt ^ psw(head)) + 4 * g;

        float m_run = -INFINITY, l_lane[4] = {0.0f, 0.0f, 0.0f, 0.0f};

        // QK of chunk x: the masked base-2 scores of this lane's head (keys 16 kt + 4 g + i) and
        // their maximum over this lane's keys.
        auto qk_scores = [&](int x, v4f(&sc)[4], float &mx) {
            // the K reads and products of the QK waves go ahead of the P.V waves' work on
            // the same SIMD; the softmax then runs at normal priority
            __builtin_amdgcn_s_setprio(3);
            const uint8_t *slot = lds + (x % SLOTS) * L::SLOTB;
            const uint8_t *ab = reinterpret_cast<const uint8_t *>(addr) + x * CHUNK * 8;
            const uint64_t mk = __ballot(lds_load<uint64_t>(ab, lane * 8) != zero);
            if constexpr (DS) {
                // the rope product in BF16, then each 128-element latent block's product
                // scaled per key by the block's FP32 scale (keys 16 kt + 4 g + i of this lane)
#pragma unroll
                for (int kt = 0; kt < 4; kt++) {
                    sc[kt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int q2 = 0; q2 < 2; q2++)
                        sc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(lds_load<v4i>(slot + kt * 2048, rbd[q2])), qrope[q2],
                            sc[kt], 0, 0, 0);
                }
#pragma unroll
                for (int s = 0; s < 4; s++) {
                    v8i av[4];
                    v4f sv[4], pr4[4];
#pragma unroll
                    for (int kt = 0; kt < 4; kt++) {
                        av[kt] = join(lds_load<v4i>(slot + s * SLICE + kt * 2048, kb0),
                                      lds_load<v4i>(slot + s * SLICE + kt * 2048, kb1));
                        sv[kt] = lds_load<v4f>(lds + L::DSR + (x & 3) * L::DSRB + 256 * s,
                                               4 * (16 * kt + 4 * g));
                    }
#pragma unroll
                    for (int kt = 0; kt < 4; kt++)
                        pr4[kt] = mfma16(av[kt], qf[s], v4f{0.f, 0.f, 0.f, 0.f});
                    mfma_result_pad();             // these products (and the rope's) landed
#pragma unroll
                    for (int kt = 0; kt < 4; kt++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            sc[kt][i] = __builtin_fmaf(sv[kt][i], pr4[kt][i], sc[kt][i]);
                }
            } else {
                // every K fragment of the chunk is read first (in the order the products use
                // them), and the products run step-major over the four independent key-tile
                // chains
                v8i av[4][4];
                v4i rr[4];
#pragma unroll
                for (int s = 0; s < 4; s++)
#pragma unroll
                    for (int kt = 0; kt < 4; kt++)
                        av[s][kt] = join(lds_load<v4i>(slot + s * SLICE + kt * 2048, kb0),
                                         lds_load<v4i>(slot + s * SLICE + kt * 2048, kb1));
                if constexpr (TAIL) {
#pragma unroll
                    for (int kt = 0; kt < 4; kt++)
                        rr[kt] = lds_load<v4i>(slot + kt * 1024, rb);
                }
#pragma unroll
                for (int kt = 0; kt < 4; kt++)
                    sc[kt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; s++)
#pragma unroll
                    for (int kt = 0; kt < 4; kt++)
                        sc[kt] = mfma16(av[s][kt], qf[s], sc[kt]);
                if constexpr (TAIL) {
#pragma unroll
                    for (int q2 = 0; q2 < 2; q2++)
#pragma unroll
                        for (int kt = 0; kt < 4; kt++)
                            sc[kt] = mfma16k32(v2i{rr[kt][2 * q2], rr[kt][2 * q2 + 1]},
                                               v2i{qt[2 * q2], qt[2 * q2 + 1]}, sc[kt]);
                }
                // the scheduler keeps this order: every K read of the chunk, then the products
                __builtin_amdgcn_sched_group_barrier(0x100, TAIL ? 36 : 32, 0);  // LDS reads
                __builtin_amdgcn_sched_group_barrier(0x008, TAIL ? 24 : 16, 0);  // MFMA
            }
            // active-column bits of this lane's keys 16 kt + 4 g + i: bit 16 (kt & 1) + i of
            // word kt >> 1
            const uint64_t bits = mk >> (4 * g);
            const uint32_t word[2] = {(uint32_t)bits, (uint32_t)(bits >> 32)};
            mfma_result_pad();
            __builtin_amdgcn_s_setprio(0);
            mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 4; kt++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    // all ones for an active column, else zero; a masked score becomes -inf
                    const int on = (int)(word[kt >> 1] << (31 - (16 * (kt & 1) + i))) >> 31;
                    const float v = sc[kt][i] * a.scale_log2;
                    sc[kt][i] = __uint_as_float((__float_as_uint(v) & (uint32_t)on) |
                                                (0xFF800000u & ~(uint32_t)on));
                    mx = fmaxf(mx, sc[kt][i]);
                }
            }
        };

        // a head's maximum over the four lane groups (rows of 16 lanes) that hold its keys
        auto head_max = [&](float mx) {
            {
                const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx),
                                                                  __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
                const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                                  __float_as_uint(mx), false, false);
                mx = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
            }
            return mx;
        };

        // P of chunk x from its scores at fb = m - log2(anchor): E4M3 (two-term by default)
        // into the P buffer, the rescale factor alpha of the accumulators beside it; this
        // lane's sums of the unquantized P are rescaled by alpha and extended.
        auto emit_p = [&](int x, const v4f(&sc)[4], float fb, float alpha) {
            uint8_t *pbase = lds + L::P + (x & 1) * L::PBUF;
#pragma unroll
            for (int kt = 0; kt < 4; kt++) {
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    p[i] = __builtin_amdgcn_exp2f(sc[kt][i] - fb);  // exp2(-inf) = 0
                const float lsum = ((p[0] + p[1]) + p[2]) + p[3];
                l_lane[kt] = __builtin_fmaf(l_lane[kt], alpha, lsum);
                int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hi, true);
                *reinterpret_cast<int *>(pbase + pw[kt]) = hi;
                if constexpr (TWO) {
                    const v2f h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
                    const v2f h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
                    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[0] - h01[0]),
                                                             16.0f * (p[1] - h01[1]), 0, false);
                    lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[2] - h23[0]),
                                                         16.0f * (p[3] - h23[1]), lo, true);
                    *reinterpret_cast<int *>(pbase + L::PTERM + pw[kt]) = lo;
                }
            }
            if (g == 0)
                scl[(x & 1) * HG + head] = alpha;
        };

        // QK and softmax of chunk x (the attn_sparse page's recipe): the chunk maximum over all
        // 64 keys, the running maximum m, the rescale factor alpha = 2^(m_old - m) of
        // everything accumulated so far, P = 2^(s2 - m + log2 448) <= 448.
        auto qk_softmax = [&](int x) {
            v4f sc[4];
            float mx;
            qk_scores(x, sc, mx);
            mx = head_max(mx);
            const float m_new = fmaxf(m_run, mx);
            // alpha = 1 while the range has no active column yet (m_new = -inf), 0 on the first
            // chunk that has one (nothing accumulated)
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            const float fb = m_new == -INFINITY ? 0.0f : m_new - LOG2_AN;
            emit_p(x, sc, fb, alpha);
        };

        // Every QK wave computes its 16 heads, padding heads included (with the group's first
        // head's q), so that the waves of a workgroup keep one schedule whatever H is.
        if (nch > 0) {
            lds_barrier();                          // the P.V waves issue chunks 0 and 1
            if constexpr (CLA) {
                // the window's one or two chunks: the scores of each as it lands, then one
                // softmax at the window's maximum (P at 256 of it, no rescale) once the last
                // has been scored; the P.V waves take both chunks after that
                v4f s0[4], s1[4];
                float mx0 = -INFINITY, mx1 = -INFINITY;
                for (int c = 0; c <= nch; c++) {
                    lds_barrier();                  // chunk c landed
                    if (c == 0)
                        qk_scores(0, s0, mx0);
                    else if (c < nch)
                        qk_scores(1, s1, mx1);
                    if (c == nch - 1) {
                        m_run = head_max(fmaxf(mx0, mx1));
                        const float fb = m_run == -INFINITY ? 0.0f : m_run - LOG2_AN;
                        emit_p(0, s0, fb, 1.0f);
                        if (nch > 1)
                            emit_p(1, s1, fb, 1.0f);
                    }
                }
            } else {
                for (int c = 0; c <= nch; c++) {
                    lds_barrier();                  // chunk c landed; P buffer c & 1 free
                    if (c < nch)
                        qk_softmax(c);
                }
            }
        }

        // ---- per-head results: l per key quarter and the running maximum ------------------------
#pragma unroll
        for (int kt = 0; kt < 4; kt++) {
            float lt = l_lane[kt];
            lt += __shfl_xor(lt, 16);
            lt += __shfl_xor(lt, 32);
            if (g == 0) {
                fin[kt * HG + head] = lt;
                if (kt == 0)
                    fin[4 * HG + head] = m_run;
            }
        }
        v16f none[NCT][2];
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
                none[ct][h2] = v16f{};
        epilogue(none);
    } else {
        // =================================== P.V waves ======================================
        const int hl = lane & 31, u = lane >> 5;   // head of the B / C columns, key block
        v16f acc[NCT][2];

        // transposed V reads of column tile ct (pieces 2 ct + (q4 & 1) of slice w), read rho:
        // lane (q4, i16) reads key 32 (q4 >> 1) + 8 rho + (i16 >> 1), half i16 & 1, at
        // position piece ^ fsw(key); fsw's low bit is rho & 1, its upper bits (i16 >> 2) & 3
        const int q4 = lane >> 4, i16 = lane & 15;
        const int vrow = (32 * (q4 >> 1) + (i16 >> 1)) * 128 + 8 * (i16 & 1) + w * SLICE;
        int voff[NCT][2];                          // [column tile][rho & 1]
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
            for (int rp = 0; rp < 2; rp++)
                voff[ct][rp] = vrow + 16 * ((2 * ct + (q4 & 1)) ^ ((((i16 >> 2) & 3) << 1) | rp));
        const int p_rd0 = hl * 64 + 16 * ((2 * u) ^ psw(hl));
        const int p_rd1 = hl * 64 + 16 * ((2 * u + 1) ^ psw(hl));

        // the loads of this wave per chunk: slice instruction m (0..7) fills slice granules
        // 64 m + lane: key 8 m + lane / 8 at position lane % 8, holding latent piece
        // 8 w + ((lane % 8) ^ fsw(key)); the rope instruction fills rope granules 64 w + lane:
        // key 16 w + lane / 4, rope piece 32 + ((lane % 4) ^ ((key >> 2) & 3))
        const int skey8 = 8 * (lane >> 3);         // address entry of key lane / 8 (+ 64 m)
        int soff[2];                               // piece offset by the parity of m
#pragma unroll
        for (int mp = 0; mp < 2; mp++)
            soff[mp] = 16 * (8 * w + ((lane & 7) ^ ((((lane >> 4) & 3) << 1) | mp)));
        const int rkey = 16 * w + (lane >> 2);
        const int roff = 16 * (32 + ((lane & 3) ^ ((rkey >> 2) & 3)));
        const uint32_t lds0 = lds_addr(lds);

        auto issue = [&](int x) {
            const uint32_t sb = lds0 + (x % SLOTS) * L::SLOTB;
            const uint8_t *ab = reinterpret_cast<const uint8_t *>(addr) + x * CHUNK * 8;
            uint64_t src[NDMA];
#pragma unroll
            for (int m = 0; m < 8; m++)
                src[m] = lds_load<uint64_t>(ab + 64 * m, skey8) + (uint32_t)soff[m & 1];
            if constexpr (TAIL)
                src[8] = lds_load<uint64_t>(ab, rkey * 8) + (uint32_t)roff;
            if constexpr (DS) {
                // scale w of key `lane` (4 bytes), and rope instructions 2 w, 2 w + 1: key
                // 8 i + lane / 8 at position lane % 8, holding rope piece (lane % 8) ^ rsw(key)
                src[8] = lds_load<uint64_t>(ab, lane * 8) + (uint32_t)(512 + 4 * w);
#pragma unroll
                for (int i2 = 0; i2 < 2; i2++) {
                    const int key = 8 * (2 * w + i2) + (lane >> 3);
                    src[9 + i2] = lds_load<uint64_t>(ab, key * 8) +
                                  (uint32_t)(528 + 16 * ((lane & 7) ^ rsw(key)));
                }
            }
#pragma unroll
            for (int m = 0; m < 8; m++)
                lds_dma16(src[m], sb + w * SLICE + 1024 * m);
            if constexpr (TAIL)
                lds_dma16(src[8], sb + L::LAT + 1024 * w);
            if constexpr (DS) {
                lds_dma4(src[8], lds0 + L::DSR + (x & 3) * L::DSRB + 256 * w);
#pragma unroll
                for (int i2 = 0; i2 < 2; i2++)
                    lds_dma16(src[9 + i2], sb + L::DROPE + 1024 * (2 * w + i2));
            }
        };

        // P.V of chunk x over this wave's 4 column tiles and both 32-head tiles, in two
        // steps: every V^T and P fragment into registers (after which the slot may be
        // refilled), then the products
        struct Frags {
            v8i vt[NCT];
            v8i bh[2], bl[2];
            float alpha[2];
            int dsr;                               // DS: LDS offset of the chunk's scale table
            int pb;                                // DS: LDS offset of the chunk's P buffer
        };
        auto pv_read = [&](int x, Frags &f) {
            const uint8_t *vs = lds + (x % SLOTS) * L::SLOTB;
            const uint8_t *pbuf = lds + L::P + (x & 1) * L::PBUF;
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                f.alpha[h2] = scl[(x & 1) * HG + 32 * h2 + hl];
                if constexpr (!DS) {
                    f.bh[h2] = join(lds_load<v4i>(pbuf + 2048 * h2, p_rd0),
                                    lds_load<v4i>(pbuf + 2048 * h2, p_rd1));
                    f.bl[h2] = f.bh[h2];
                    if constexpr (TWO)
                        f.bl[h2] = join(lds_load<v4i>(pbuf + L::PTERM + 2048 * h2, p_rd0),
                                        lds_load<v4i>(pbuf + L::PTERM + 2048 * h2, p_rd1));
                }
            }
            // DS: the P fragments are read by the products themselves (the QK waves write the
            // other P buffer meanwhile)
            f.pb = L::P + (x & 1) * L::PBUF;
#pragma unroll
            for (int ct = 0; ct < NCT; ct++) {
#pragma unroll
                for (int rho = 0; rho < 4; rho++) {
                    const v2i y = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (SMLA_LDS(v2i) *)(vs + rho * 1024 + voff[ct][rho & 1]));
                    f.vt[ct][2 * rho] = y[0];
                    f.vt[ct][2 * rho + 1] = y[1];
                }
            }
            if constexpr (DS)
                f.dsr = L::DSR + (x & 3) * L::DSRB + 256 * w + 4 * 32 * u;
        };
        // the accumulators rescaled to the chunk's running maximum, then its products
        auto pv_mma = [&](const Frags &f) {
            mfma_result_pad();                     // the previous chunk's products have landed
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                for (int h2 = 0; h2 < 2; h2++)
                    acc[ct][h2] *= f.alpha[h2];
            if constexpr (DS) {
                // BF16 products over 16 keys at a time: step k takes bytes 8 k .. 8 k + 7 of
                // each lane's V^T and P fragments (keys 32 u + 8 k + 0..7, the same keys on
                // both sides), V times its key's block scale, P exact (E4M3 is a subset of
                // BF16; the second term times 2^-4, still exact)
                const v4f one = v4f{1.0f, 1.0f, 1.0f, 1.0f};
                const v4f sixteenth = v4f{0.0625f, 0.0625f, 0.0625f, 0.0625f};
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    // P bytes 8 k .. 8 k + 7 of this lane's fragment: 8 (k & 1) into the 16-byte
                    // piece at p_rd0 (k < 2) or p_rd1
                    const int po = (k < 2 ? p_rd0 : p_rd1) + 8 * (k & 1);
                    v8bf ph[2], pl[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++) {
                        const v2i hb = lds_load<v2i>(lds + f.pb + 2048 * h2, po);
                        ph[h2] = e4m3x8_bf16(hb[0], hb[1], one, one);
                        if constexpr (TWO) {
                            const v2i lb = lds_load<v2i>(lds + f.pb + L::PTERM + 2048 * h2, po);
                            pl[h2] = e4m3x8_bf16(lb[0], lb[1], sixteenth, sixteenth);
                        }
                    }
                    // block w's scales of keys 32 u + 8 k + 0..7 (the ring keeps this chunk's
                    // table while the slot is refilled)
                    const v4f s0 = lds_load<v4f>(lds + f.dsr, 32 * k);
                    const v4f s1 = lds_load<v4f>(lds + f.dsr, 32 * k + 16);
#pragma unroll
                    for (int ct = 0; ct < NCT; ct++) {
                        const v8bf vb = e4m3x8_bf16(f.vt[ct][2 * k], f.vt[ct][2 * k + 1], s0, s1);
#pragma unroll
                        for (int h2 = 0; h2 < 2; h2++) {
                            acc[ct][h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                vb, ph[h2], acc[ct][h2], 0, 0, 0);
                            if constexpr (TWO)
                                acc[ct][h2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                    vb, pl[h2], acc[ct][h2], 0, 0, 0);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int ct = 0; ct < NCT; ct++) {
#pragma unroll
                    for (int h2 = 0; h2 < 2; h2++) {
                        acc[ct][h2] = mfma32(f.vt[ct], f.bh[h2], acc[ct][h2], 127);
                        if constexpr (TWO)  // the second term's 2^-4
                            acc[ct][h2] = mfma32(f.vt[ct], f.bl[h2], acc[ct][h2], 127 - 4);
                    }
                }
            }
        };

#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
                acc[ct][h2] = v16f{};
        if (nch > 0) {
            // every slot is free, so the first two chunks go out before the barrier that the
            // QK waves reach once their Q loads are issued
            issue(0);
            if (nch > 1)
                issue(1);
            lds_barrier();
            if (nch > 1)
                wait_dma<NDMA>();                   // chunk 0
            else
                wait_dma<0>();
            for (int c = 0; c <= nch; c++) {
                lds_barrier();                      // chunk c landed; P of chunk c-1 visible
                if constexpr (CLA) {
                    // a window has at most two chunks, both in their slots from the start;
                    // their P is ready once the QK waves have scored the last of them
                    if (c == nch) {
                        for (int x = 0; x < nch; x++) {
                            Frags f;
                            pv_read(x, f);
                            pv_mma(f);
                        }
                    }
                } else {
                    // The loads of chunk c+2 go out before the products of chunk c-1: the QK
                    // waves' products of chunk c then reach the matrix units first, and these
                    // run during the QK waves' softmax.
                    Frags f;
                    if (c > 0)
                        pv_read(c - 1, f);
                    if (c + 2 < nch) {
                        // the wave's own reads of the slice it refills have completed
                        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                        issue(c + 2);
                    }
                    __builtin_amdgcn_sched_barrier(0);  // the products stay after the loads
                    if (c > 0)
                        pv_mma(f);
                }
                if (c + 2 < nch)
                    wait_dma<NDMA>();               // chunk c+1
                else
                    wait_dma<0>();
            }
        }
        mfma_result_pad();                          // the last products have landed
        // two-range spread merge: the half of the partial that the other range merges goes
        // out now; its (m, l) follows once the epilogue's barrier has published them
        if (PAIR && a.splits == 2 && (w >> 1) != split) {
            const int heads_here = min(a.gw, a.H - hg * a.gw);
            const int64_t ui = ((int64_t)t * a.groups + hg) * 2 + split;
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(a.ws_o + ui * (HG * 512), 0,
                                                              HG * 512 * 4, 0x00020000);
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                for (int h2 = 0; h2 < 2; h2++) {
                    if (32 * h2 + (lane & 31) >= heads_here)
                        continue;
#pragma unroll
                    for (int j = 0; j < 4; j++)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            v4i{__float_as_int(acc[ct][h2][4 * j]),
                                __float_as_int(acc[ct][h2][4 * j + 1]),
                                __float_as_int(acc[ct][h2][4 * j + 2]),
                                __float_as_int(acc[ct][h2][4 * j + 3])},
                            rs, ((((NCT * w + ct) * 2 + h2) * 4 + j) * 64 + lane) * 16, 0, 16);
                }
        }
        epilogue(acc);
    }
}

template <int RB, int QK, bool TWO, bool CLA>
hipError_t launch_g64_one(const DecodeParams &p, hipStream_t stream)
{
    const unsigned blocks = (unsigned)p.T * (unsigned)p.groups * (unsigned)p.splits;
    // the spread merge's ranges wait for each other: its grid is at most one workgroup per
    // compute unit (checked on the host), so every workgroup is resident at once
    // grids that fill the device load their index rows speculatively (SPI)
    bool spi = false;
    if constexpr (!CLA)
        spi = p.spec_idx != 0 && p.paged == 0;
    if (p.merge == 1 && p.splits == 2) {
        if constexpr (!CLA) {
            if (spi) {
                hipLaunchKernelGGL((decode_g64_kernel<RB, QK, TWO, true, CLA, true, true>),
                                   dim3(blocks), dim3(NT), 0, stream, p);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((decode_g64_kernel<RB, QK, TWO, true, CLA, true, false>), dim3(blocks),
                           dim3(NT), 0, stream, p);
    } else if (p.merge == 1 && p.splits > 1) {
        hipLaunchKernelGGL((decode_g64_kernel<RB, QK, TWO, true, CLA, false, false>),
                           dim3(blocks), dim3(NT), 0, stream, p);
    } else {
        if constexpr (!CLA) {
            if (spi) {
                hipLaunchKernelGGL((decode_g64_kernel<RB, QK, TWO, false, CLA, false, true>),
                                   dim3(blocks), dim3(NT), 0, stream, p);
                return hipGetLastError();
            }
        }
        hipLaunchKernelGGL((decode_g64_kernel<RB, QK, TWO, false, CLA, false, false>),
                           dim3(blocks), dim3(NT), 0, stream, p);
    }
    return hipGetLastError();
}

template <bool TWO, bool CLA>
hipError_t launch_g64_shape(const DecodeParams &p, int row_bytes, int qk_dim, hipStream_t stream)
{
    if (row_bytes == 576 && qk_dim == 576)
        return launch_g64_one<576, 576, TWO, CLA>(p, stream);
    if (row_bytes == 576 && qk_dim == 512)
        return launch_g64_one<576, 512, TWO, CLA>(p, stream);
    if (row_bytes == 512 && qk_dim == 512)
        return launch_g64_one<512, 512, TWO, CLA>(p, stream);
    if (row_bytes == 656 && qk_dim == 576)
        return launch_g64_one<656, 576, TWO, CLA>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_g64(const DecodeParams &p, int row_bytes, int qk_dim, bool two_term,
                             bool chunk_local, hipStream_t stream)
{
    // the chunk-local recipe quantizes P as one E4M3 term
    if (chunk_local)
        return launch_g64_shape<false, true>(p, row_bytes, qk_dim, stream);
    return two_term ? launch_g64_shape<true, false>(p, row_bytes, qk_dim, stream)
                    : launch_g64_shape<false, false>(p, row_bytes, qk_dim, stream);
}

}  // namespace smla
