// Sparse MLA decode for gfx950 (MI355X): per-token row gather, QK^T and P.V on the
// block-scaled FP8 matrix instructions, online softmax with P quantized to E4M3, and a fused
// merge of split partials.
//
// Method (vLLM API pages): the formula is the sparse_mla_cute page's "What this module
// computes"; the E4M3-P recipe, the contiguous key split and the split merge are the
// attn_sparse page's module docstring and its SparseDcpDecode.kernel / merge methods.
//
// Work decomposition.  A workgroup of 8 waves takes one token t, one group of 32 heads (the
// last group zero-padded) and one of S contiguous key ranges of the token's clamped count
// (range s = [min(n, s per), + min(n - first, per)), per = ceil(n / S)), processed in chunks of
// 64 columns.  Workgroups of the same token are placed on the same XCD (workgroups are
// dispatched to the 8 XCDs round-robin), so the head groups of a token share its gathered rows
// in that XCD's L2 and the split partials of a token are merged through the same L2.
//
// Two roles, one wave of each per SIMD, so that one role's matrix work overlaps the other's
// vector and LDS work:
//   QK waves (0..3): wave w owns keys 16 w .. 16 w + 15 of every chunk.  Lane (r, g) = (lane
//     % 16, lane / 16) loads row 16 w + r of the chunk straight into registers, 16-byte pieces
//     8 s + 4 j + g (s < 4, j < 2) and the rope piece 32 + g: each load instruction reads 64
//     contiguous bytes of 16 rows.  Those registers are the A operand of QK on
//     v_mfma_scale_f32_16x16x128_f8f6f4 (16 keys x 16 heads x 128 bytes; the Q fragments, the
//     B operand, are loaded once with the same byte permutation; the rope step runs on two
//     16x16x32 FP8 instructions), so K never goes through LDS; the 512 latent bytes are
//     written to an LDS slot for P.V.  Rows are loaded two chunks ahead of their QK (three
//     register stages, issued from inline assembly with explicit waits); masked columns read
//     a zero row.  The base-2 scores s2 = S bmm1 log2(e) (-inf for masked keys) go to LDS in
//     lane order, with this wave's 16-key maximum per head.
//   P.V waves (4..7): wave 4 + j owns latent columns 128 j .. 128 j + 127 and, for the
//     softmax, the keys 16 j .. 16 j + 15 of every chunk (the same lanes as the QK wave that
//     computed their scores).  Softmax (the attn_sparse page's recipe): chunk maximum over the
//     four key quarters, running maximum m, alpha = 2^(m_old - m); P = 2^(s2 - m + log2 448)
//     <= 448, rounded to E4M3 by v_cvt_pk_fp8_f32 (two-term default: P = hi + lo/16, lo =
//     E4M3(16 (P - hi))); FP32 sums of the unquantized P kept per lane, rescaled by alpha.
//     P.V: O^T *= alpha (per head), then
//     O^T (32 columns x 32 heads) += V^T (32 columns x 64 keys, ds_read_b64_tr_b8 from
//     the slot) P^T (64 keys x 32 heads, from the P buffer) on
//     v_mfma_scale_f32_32x32x64_f8f6f4, 4 tiles per chunk (8 instructions with two-term P).
//     One of these waves also loads the row indices, eight chunks at a time and at least
//     eight chunks ahead, into an LDS ring for the QK waves.
//   Software pipeline: iteration c runs, in the QK waves, the row loads of chunk c+3 and QK
//   (scores, maxima, V slot) of chunk c+1, and in the P.V waves the softmax of chunk c and
//   P.V of chunk c-1, with a single workgroup barrier per iteration; three V slots hold
//   chunks c-1 .. c+1.
//
// Epilogue: one range (S = 1): merge with the sink, BF16 output through an LDS tile (coalesced
// row stores) and the LSE.  S > 1: every range writes its partial (its FP32 accumulators in
// register order, so reads and writes coalesce) and (m, l); the last range to finish (atomic
// ticket per token and head group) merges all partials in range order, weights 2^(m_s - M),
// writes the output and resets the ticket.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

using namespace dev;

constexpr int CHUNK = 64;                          // columns per chunk
constexpr int NT = 512;                            // threads per workgroup (8 waves)
constexpr int HG = 32;                             // heads per workgroup
constexpr int VSLOTS = 3;                          // V slots in LDS: chunks c-1 .. c+1
constexpr int NCT = 4;                             // 32-column P.V tiles per P.V wave
constexpr int IRING = 16;                          // chunks of row indices held in LDS
constexpr int IBLK = 8;                            // chunks of indices loaded per refill

// Masked columns gather this row, so their bytes are zero (0 * anything stays finite).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[576];

// LDS carve-up (byte offsets).
struct Lds {
    static constexpr int VSLOT = CHUNK * 512;                  // latent bytes of one chunk
    static constexpr int V = 0;                                // [VSLOTS][64 keys][512]
    static constexpr int SC = VSLOTS * VSLOT;                  // [2 buf][4 waves][64 lanes][8]
    static constexpr int P = SC + 2 * 4 * 64 * 8 * 4;          // [2 buf][2 term][32][64]
    static constexpr int PTERM = HG * 64;
    static constexpr int PBUF = 2 * PTERM;
    static constexpr int SCL = P + 2 * PBUF;                   // [2 buf][32] float: alpha
    static constexpr int MX = SCL + 2 * HG * 4;                // [2 buf][32 heads][4 key quarters]
    static constexpr int FIN = MX + 2 * HG * 4 * 4;            // [4 key quarters][32] l, [32] G, e
    static constexpr int IDX = FIN + 6 * HG * 4;               // [16 chunks][64] int indices
    static constexpr int QR = IDX + IRING * CHUNK * 4;         // [4 QK waves][32][64] q rope
    static constexpr int MISC = QR + 4 * HG * 64;              // ticket
    static constexpr int TOTAL = MISC + 16;
    static constexpr int OUT_TILE = HG * 1024;                 // BF16 [32][512], after the loop
    static_assert(OUT_TILE <= P, "output tile must fit in the V slots");
    static_assert(OUT_TILE + 64 * HG * 8 <= SC, "(m, l) of 64 ranges must fit past the tile");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// V slot of chunk x (x >= -1).
__device__ inline int vslot(int x) { return (x + VSLOTS) % VSLOTS; }

template <int RB, int QK, bool TWO>
__global__ void __launch_bounds__(NT, 1) decode_kernel(DecodeParams a)
{
    constexpr bool TAIL = QK == 576;               // a fifth, 64-byte QK step (rope)
    constexpr int NLD = TAIL ? 9 : 8;              // row loads per S lane and chunk
    using L = Lds;

    __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const bool s_wave = wave < 4;
    const int w = wave & 3;                        // S: key quarter; O: column quarter

    int t, unit;
    unit_of(blockIdx.x, a.T, a.splits * a.groups, &t, &unit);
    const int hg = unit % a.groups;
    const int split = unit / a.groups;

    int n = a.lens[t];
    n = n < 0 ? 0 : (n > a.W ? a.W : n);
    const int per = (n + a.splits - 1) / a.splits;
    const int first = min(n, split * per);
    const int mine = min(n - first, per);
    const int end = first + mine;
    const int nch = (mine + CHUNK - 1) / CHUNK;
    const int32_t *idx_row = a.indices + (int64_t)t * a.W;

    float *fin = reinterpret_cast<float *>(lds + L::FIN);  // [4][32] l, [32] m

    // ---- epilogue (every wave; `acc` holds the P.V waves' accumulators) ---------------------
    // acc[ct]: O^T tile of columns 32 (4 w + ct) + .. x 32 heads; lane l holds head l % 32,
    // columns 8 (r / 4) + 4 (l / 32) + r % 4 of the tile in register r.
    auto epilogue = [&](v16f(&acc)[NCT]) __attribute__((always_inline)) {
        lds_barrier();
        const int hl = lane & 31, u = lane >> 5;
        // head hl of this lane: the running maximum m (g_h) and the sum l at 448 of it
        float g_h = fin[4 * HG + hl];
        float l_h = ((fin[hl] + fin[HG + hl]) + fin[2 * HG + hl]) + fin[3 * HG + hl];
        const int head = hg * HG + hl;
        const int64_t tg = (int64_t)t * a.groups + hg;
        const int tile0 = NCT * w;
        if (a.splits > 1) {
            // Split merge.  Every range writes its partial (FP32 accumulators as they stand, at
            // 448 of the range's running maximum m; then (m, l) per head) with device-scope
            // (write-through) stores, waits for them to complete and only then takes an arrival
            // ticket; the range holding the last ticket therefore sees every other partial
            // complete and merges all of them in range order, its own from registers (FP32 throughout, so the result does not depend on
            // the arrival order).  (With few workgroups this beats taking the ticket first: the
            // stores of all ranges overlap instead of following the ticket round trip.)
            // Partial layout: accumulator registers 4 j .. 4 j + 3 of tile `tile` at byte
            // ((tile * 4 + j) * 64 + lane) * 16, one 16-byte access per lane.
            constexpr int SC1 = 16;  // cache policy of device-scope (write-through) accesses
            auto part_off = [&](int ct, int j) { return (((tile0 + ct) * 4 + j) * 64 + lane) * 16; };
            auto part_rsrc = [&](int64_t unit) {
                return __builtin_amdgcn_make_buffer_rsrc(a.ws_o + unit * (HG * 512), 0,
                                                         HG * 512 * 4, 0x00020000);
            };
            int *ticket = reinterpret_cast<int *>(lds + L::MISC);
            int *ctr = a.counters + 2 * tg;         // [0] arrival ticket
            {
                const int64_t ui = tg * a.splits + split;
                if (!s_wave) {
                    const auto rs = part_rsrc(ui);
#pragma unroll
                    for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                v4i{__float_as_int(acc[ct][4 * j]), __float_as_int(acc[ct][4 * j + 1]),
                                    __float_as_int(acc[ct][4 * j + 2]),
                                    __float_as_int(acc[ct][4 * j + 3])},
                                rs, part_off(ct, j), 0, SC1);
                }
                if (wave == 4 && u == 0) {
                    store_device(a.ws_ml + (ui * HG + hl) * 2 + 0, g_h);
                    store_device(a.ws_ml + (ui * HG + hl) * 2 + 1, l_h);
                }
            }
            __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
            __syncthreads();
            if (tid == 0)
                *ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (*ticket != a.splits - 1)
                return;
            // (m, l) of every range and head, staged in LDS in one round of loads (over the
            // V slots, past the output tile)
            float2 *gl = reinterpret_cast<float2 *>(lds + L::OUT_TILE);  // [splits][32]
            for (int i = tid; i < a.splits * HG; i += NT) {
                const int s = i / HG, h = i % HG;
                const float *m = a.ws_ml + ((tg * a.splits + s) * HG + h) * 2;
                if (s != split)  // this range's own values stay in registers
                    gl[i] = float2{load_device(m), load_device(m + 1)};
            }
            __syncthreads();
            float big_g = -INFINITY;
            for (int s = 0; s < a.splits; s++)
                big_g = fmaxf(big_g, s == split ? g_h : gl[s * HG + hl].x);
            float l_new = 0.0f;
            for (int s = 0; s < a.splits; s++) {
                const float gs = s == split ? g_h : gl[s * HG + hl].x;
                const float ls = s == split ? l_h : gl[s * HG + hl].y;
                l_new += (gs == -INFINITY ? 0.0f : exp2f(gs - big_g)) * ls;
            }
            if (!s_wave) {
                // range order, all four column tiles of one range per round of loads
                v16f sum[NCT];
#pragma unroll
                for (int ct = 0; ct < NCT; ct++)
                    sum[ct] = v16f{};
                for (int s = 0; s < a.splits; s++) {
                    const float gs = s == split ? g_h : gl[s * HG + hl].x;
                    const float wgt = gs == -INFINITY ? 0.0f : exp2f(gs - big_g);
                    if (s == split) {
#pragma unroll
                        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                            for (int r = 0; r < 16; r++)
                                sum[ct][r] += wgt * acc[ct][r];
                    } else {
                        const auto rs = part_rsrc(tg * a.splits + s);
                        v4i v[NCT][4];
#pragma unroll
                        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                v[ct][j] = __builtin_amdgcn_raw_buffer_load_b128(
                                    rs, part_off(ct, j), 0, SC1);
#pragma unroll
                        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                            for (int r = 0; r < 16; r++)
                                sum[ct][r] += wgt * __int_as_float(v[ct][r >> 2][r & 3]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < NCT; ct++)
                    acc[ct] = sum[ct];
            }
            g_h = big_g;
            l_h = l_new;
            if (tid == 0)  // every range has arrived: ready for the next call
                __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        // ---- final: sink, normalization, BF16 tile in LDS, coalesced row stores, LSE ------
        uint8_t *tile = lds;  // [32][1024 bytes], over the V slots
        const bool any = g_h != -INFINITY;
        float big_m = g_h, big_l = l_h, wgt = 1.0f;
        if (a.sinks != nullptr && head < a.H) {
            const float sk = a.sinks[head] * LOG2E;
            big_m = fmaxf(g_h, sk);
            wgt = any ? exp2f(g_h - big_m) : 0.0f;
            big_l = wgt * l_h + ANCHOR * exp2f(sk - big_m);
        }
        const float inv = any ? a.bmm2 * wgt / big_l : 0.0f;
        if (!s_wave) {
#pragma unroll
            for (int ct = 0; ct < NCT; ct++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int col = 32 * (tile0 + ct) + 8 * i + 4 * u;
                    uint2 pk;
                    pk.x = bf16x2(acc[ct][4 * i] * inv, acc[ct][4 * i + 1] * inv);
                    pk.y = bf16x2(acc[ct][4 * i + 2] * inv, acc[ct][4 * i + 3] * inv);
                    *reinterpret_cast<uint2 *>(tile + tile_off(hl, 2 * col)) = pk;
                }
            }
        }
        if (wave == 4 && u == 0 && head < a.H && a.lse != nullptr) {
            const float lse2 = any ? big_m - LOG2_ANCHOR + log2f(big_l) : -INFINITY;
            a.lse[(int64_t)t * a.H + head] = a.lse_log2 ? lse2 : lse2 * LN2;
        }
        lds_barrier();
        const int heads_here = min(HG, a.H - hg * HG);
        for (int x = tid; x < heads_here * 64; x += NT) {
            const int row = x >> 6, part = x & 63;
            const v4i v = lds_load<v4i>(tile, tile_off(row, 16 * part));
            // streaming store: the output is not read again by this kernel
            __builtin_nontemporal_store(
                v, reinterpret_cast<v4i *>(a.out + ((int64_t)t * a.H + hg * HG + row) * 512 +
                                           8 * part));
        }
    };

    if (s_wave) {
        // =================================== QK waves =====================================
        const int r = lane & 15, g = lane >> 4;    // row r of this wave's 16 keys, piece group
        const int key = 16 * w + r;                // this lane's key within a chunk

        // Q fragments, B operand of QK: lane (n, g) holds, for head 16 ht + n and step s, the
        // q pieces 8 s + g and 8 s + 4 + g (the same permutation as the K rows).  The rope
        // pieces (32 + g, two 8-byte halves, one per 16x16x32 step) wait in this wave's own
        // LDS copy and are read per chunk, which keeps the loop within the register budget.
        v8i qf[2][4];
        uint8_t *qr = lds + L::QR + w * HG * 64;
#pragma unroll
        for (int ht = 0; ht < 2; ht++) {
            const int head = hg * HG + 16 * ht + r;
            const bool live = head < a.H;
            const uint8_t *qp = a.q + (int64_t)t * a.q_st + (int64_t)(live ? head : 0) * a.q_sh;
#pragma unroll
            for (int s = 0; s < 4; s++) {
                v4i lo = v4i{0, 0, 0, 0}, hi = v4i{0, 0, 0, 0};
                if (live) {
                    lo = gload(qp + 16 * (8 * s + g));
                    hi = gload(qp + 16 * (8 * s + 4 + g));
                }
                qf[ht][s] = join(lo, hi);
            }
            if constexpr (TAIL) {
                v4i qt = v4i{0, 0, 0, 0};
                if (live)
                    qt = gload(qp + 16 * (32 + g));
                *reinterpret_cast<v4i *>(qr + (16 * ht + r) * 64 + 16 * g) = qt;
            }
        }

        // raw index of this lane's key in chunk x, from the index ring (written by the P.V
        // waves at least one barrier earlier)
        const int *idx_ring = reinterpret_cast<const int *>(lds + L::IDX);
        auto load_raw = [&](int x) { return idx_ring[(x % IRING) * CHUNK + key]; };
        // Issue the row loads of chunk x into `st` (raw: the index, arrived); returns the
        // chunk's mask of active keys (bit k: key 16 w + k of the chunk), wave-uniform.  Lane
        // (r, g) loads pieces 8 s + 4 j + g into st[2 s + j] and the rope piece 32 + g.
        auto issue = [&](int x, int raw, v4i(&st)[NLD]) {
            const int pos = first + x * CHUNK + key;
            const bool valid = pos < end && raw >= 0;
            const uint8_t *pool = (a.kv_b != nullptr && pos >= a.split_col) ? a.kv_b : a.kv_a;
            const uint8_t *row = (valid ? pool + (int64_t)raw * RB : g_zero_row) + 16 * g;
            gload_row_async(st, row);
            return (uint32_t)(__ballot(valid) & 0xFFFFu);
        };

        // Per chunk the QK waves issue NLD row loads, in chunk order, so a chunk's rows have
        // arrived at its QK once the next two chunks' loads (2 NLD) are behind them.
        constexpr int BEHIND = 2 * NLD;

        // QK products of the chunk held in `st` (16 keys x 32 heads as two 16-head tiles)
        auto qk_issue = [&](const v4i(&st)[NLD], v4f &c0, v4f &c1) {
            c0 = v4f{0.f, 0.f, 0.f, 0.f};
            c1 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const v8i av = join(st[2 * s], st[2 * s + 1]);
                c0 = mfma16(av, qf[0][s], c0);
                c1 = mfma16(av, qf[1][s], c1);
            }
            if constexpr (TAIL) {
                const v4i q0 = lds_load<v4i>(qr, r * 64 + 16 * g);
                const v4i q1 = lds_load<v4i>(qr, (16 + r) * 64 + 16 * g);
#pragma unroll
                for (int hh = 0; hh < 2; hh++) {
                    const v2i av = v2i{st[8][2 * hh], st[8][2 * hh + 1]};
                    c0 = mfma16k32(av, v2i{q0[2 * hh], q0[2 * hh + 1]}, c0);
                    c1 = mfma16k32(av, v2i{q1[2 * hh], q1[2 * hh + 1]}, c1);
                }
            }
        };
        // Base-2 scores of chunk x with masked keys at -inf (lane (n, q): head 16 ht + n, keys
        // 16 w + 4 q + i) to the chunk's score buffer, in lane order for the P.V wave that owns
        // the same keys, and this wave's 16-key maximum per head to the chunk's MX buffer.
        auto qk_finish = [&](int x, v4f c0, v4f c1, uint32_t mk) {
            mfma_result_pad();
            v4f s0, s1;
            float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float b = ((mk >> (4 * g + i)) & 1u) ? 0.0f : -INFINITY;
                s0[i] = fmaf(c0[i], a.scale_log2, b);
                s1[i] = fmaf(c1[i], a.scale_log2, b);
                mx0 = fmaxf(mx0, s0[i]);
                mx1 = fmaxf(mx1, s1[i]);
            }
            float *sc = reinterpret_cast<float *>(lds + L::SC) + (x & 1) * (4 * 64 * 8) +
                        (w * 64 + lane) * 8;
            *reinterpret_cast<v4f *>(sc) = s0;
            *reinterpret_cast<v4f *>(sc + 4) = s1;
            mx0 = fmaxf(mx0, __shfl_xor(mx0, 16));
            mx0 = fmaxf(mx0, __shfl_xor(mx0, 32));
            mx1 = fmaxf(mx1, __shfl_xor(mx1, 16));
            mx1 = fmaxf(mx1, __shfl_xor(mx1, 32));
            float *mxb = reinterpret_cast<float *>(lds + L::MX) + (x & 1) * HG * 4;
            if (g < 2)
                mxb[(16 * g + r) * 4 + w] = g == 0 ? mx0 : mx1;
        };
        // latent bytes of the chunk in `st` to its V slot (pieces 8 s + 4 j + g of row key)
        auto write_v = [&](int x, const v4i(&st)[NLD]) {
            uint8_t *vs = lds + L::V + vslot(x) * L::VSLOT + key * 512;
            const int sw = vsw(key);
#pragma unroll
            for (int s = 0; s < 4; s++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    *reinterpret_cast<v4i *>(vs + 16 * ((8 * s + 4 * j + g) ^ sw)) =
                        st[2 * s + j];
        };

        v4i st0[NLD], st1[NLD], st2[NLD];
        uint32_t mk0 = 0, mk1 = 0, mk2 = 0;

        // Iteration c: row loads of chunk c+3 into `ld` (the stage chunk c left), QK, scores
        // and V slot of chunk c+1 from `cur`.
        auto iteration = [&](int c, v4i(&ld)[NLD], uint32_t &mld, v4i(&cur)[NLD],
                             uint32_t mcur) __attribute__((always_inline)) {
            lds_barrier();
            mld = issue(c + 3, load_raw(c + 3), ld);
            wait_vm<BEHIND>(cur);                   // the rows of chunk c+1
            v4f c0, c1;
            qk_issue(cur, c0, c1);
            qk_finish(c + 1, c0, c1, mcur);
            write_v(c + 1, cur);
        };

        auto run_range = [&]() __attribute__((always_inline)) {
            if (nch == 0)
                return;
            lds_barrier();                          // the index ring holds chunks 0 .. 7
            mk0 = issue(0, load_raw(0), st0);
            mk1 = issue(1, load_raw(1), st1);
            mk2 = issue(2, load_raw(2), st2);
            {
                wait_vm<BEHIND>(st0);
                v4f c0, c1;
                qk_issue(st0, c0, c1);
                qk_finish(0, c0, c1, mk0);
            }
            write_v(0, st0);
            for (int c = 0;; c += 3) {
                iteration(c, st0, mk0, st1, mk1);
                if (c + 1 >= nch)
                    break;
                iteration(c + 1, st1, mk1, st2, mk2);
                if (c + 2 >= nch)
                    break;
                iteration(c + 2, st2, mk2, st0, mk0);
                if (c + 3 >= nch)
                    break;
            }
            // every load has landed before the registers it targets can be reused
            wait_vm<0>(st0);
            wait_vm<0>(st1);
            wait_vm<0>(st2);
            lds_barrier();                          // drain: the P.V waves' P.V of chunk nch-1
        };

        run_range();
        v16f none[NCT];
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
            none[ct] = v16f{};
        epilogue(none);
    } else {
        // =================================== P.V waves ====================================
        v16f acc[NCT];
        const int hl = lane & 31, u = lane >> 5;   // head of the B / C columns, key block
        const int q4 = lane >> 4, i16 = lane & 15;
        const int p_off0 = hl * 64 + 16 * ((2 * u) ^ psw(hl));
        const int p_off1 = hl * 64 + 16 * ((2 * u + 1) ^ psw(hl));
        // transposed V reads: lane (q4, i16), read rho: key 32 (q4 >> 1) + 8 rho + (i16 >> 1),
        // half i16 & 1 of piece 2 tile + (q4 & 1); byte offsets within a slot per tile and rho
        int v_off[NCT][4];
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
            for (int rho = 0; rho < 4; rho++) {
                const int k = 32 * (q4 >> 1) + 8 * rho + (i16 >> 1);
                const int piece = 2 * (NCT * w + ct) + (q4 & 1);
                v_off[ct][rho] = k * 512 + 16 * (piece ^ vsw(k)) + 8 * (i16 & 1);
            }

        // ---- softmax state: lane (nh, kq) owns heads nh and 16 + nh, keys 16 w + 4 kq + i --
        const int kq = lane >> 4, nh = lane & 15;
        float m_run[2] = {-INFINITY, -INFINITY}, l_lane[2] = {0.0f, 0.0f};

        // softmax of chunk x (branch-free; the attn_sparse page's recipe): the chunk maximum over
        // the four key quarters, the running maximum m, the rescale factor alpha = 2^(m_old - m)
        // of everything accumulated so far (into LDS beside P, for the accumulators), and
        // P = 2^(s2 - m + log2 448) <= 448 as E4M3 (two-term by default) into the chunk's P
        // buffer; the sums of the unquantized P are rescaled and extended here.
        auto softmax = [&](int x) {
            const uint8_t *mxb = lds + L::MX + (x & 1) * HG * 16;
            const float *sc = reinterpret_cast<const float *>(lds + L::SC) +
                              (x & 1) * (4 * 64 * 8) + (w * 64 + lane) * 8;
            const v4f sv[2] = {*reinterpret_cast<const v4f *>(sc),
                               *reinterpret_cast<const v4f *>(sc + 4)};
            uint8_t *pbase = lds + L::P + (x & 1) * L::PBUF;
#pragma unroll
            for (int ht = 0; ht < 2; ht++) {
                const int head = 16 * ht + nh;
                const v4f m4 = lds_load<v4f>(mxb, head * 16);
                const float m_chunk = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
                const float m_new = fmaxf(m_run[ht], m_chunk);
                const float alpha =
                    m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[ht] - m_new);
                m_run[ht] = m_new;
                const float fb = m_new == -INFINITY ? 0.0f : m_new - LOG2_ANCHOR;
                float p[4];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    p[i] = __builtin_amdgcn_exp2f(sv[ht][i] - fb);  // exp2(-inf) = 0
                const float lsum = ((p[0] + p[1]) + p[2]) + p[3];
                l_lane[ht] = __builtin_fmaf(l_lane[ht], alpha, lsum);
                int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
                hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hi, true);
                const int off = head * 64 + 16 * (w ^ psw(head)) + 4 * kq;
                *reinterpret_cast<int *>(pbase + off) = hi;
                if constexpr (TWO) {
                    const float h0 = __builtin_amdgcn_cvt_f32_fp8(hi, 0);
                    const float h1 = __builtin_amdgcn_cvt_f32_fp8(hi, 1);
                    const float h2 = __builtin_amdgcn_cvt_f32_fp8(hi, 2);
                    const float h3 = __builtin_amdgcn_cvt_f32_fp8(hi, 3);
                    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[0] - h0),
                                                             16.0f * (p[1] - h1), 0, false);
                    lo = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[2] - h2),
                                                         16.0f * (p[3] - h3), lo, true);
                    *reinterpret_cast<int *>(pbase + L::PTERM + off) = lo;
                }
                if (w == 0 && kq == ht)
                    reinterpret_cast<float *>(lds + L::SCL)[(x & 1) * HG + head] = alpha;
            }
        };

        // P.V of chunk x over this wave's 4 column tiles: the accumulators rescaled to the
        // chunk's running maximum, then its products
        auto pv = [&](int x) {
            const uint8_t *vs = lds + L::V + vslot(x) * L::VSLOT;
            const uint8_t *pbuf = lds + L::P + (x & 1) * L::PBUF;
            const float alpha = reinterpret_cast<const float *>(lds + L::SCL)[(x & 1) * HG + hl];
            const v8i bh = join(lds_load<v4i>(pbuf, p_off0), lds_load<v4i>(pbuf, p_off1));
            v8i bl = bh;
            if constexpr (TWO)
                bl = join(lds_load<v4i>(pbuf + L::PTERM, p_off0),
                          lds_load<v4i>(pbuf + L::PTERM, p_off1));
            auto read_vt = [&](int ct) {
                v8i vt;
#pragma unroll
                for (int rho = 0; rho < 4; rho++) {
                    const v2i y = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (SMLA_LDS(v2i) *)(vs + v_off[ct][rho]));
                    vt[2 * rho] = y[0];
                    vt[2 * rho + 1] = y[1];
                }
                return vt;
            };
            v8i vcur = read_vt(0);
            mfma_result_pad();                     // the previous chunk's products have landed
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                acc[ct] *= alpha;
#pragma unroll
            for (int ct = 0; ct < NCT; ct++) {
                v8i vnext = vcur;
                if (ct + 1 < NCT)
                    vnext = read_vt(ct + 1);  // next tile's V^T in flight during these products
                acc[ct] = mfma32(vcur, bh, acc[ct], 127);
                if constexpr (TWO)
                    acc[ct] = mfma32(vcur, bl, acc[ct], 127 - 4);  // the second term's 2^-4
                vcur = vnext;
            }
        };

        // Indices of the QK waves' row loads, in an LDS ring of IRING chunks (slot x % IRING),
        // filled by wave 4 in blocks of IBLK chunks: at iteration c = 0 mod IBLK it stores the
        // block of chunks c + IBLK .. c + 2 IBLK - 1, loaded IBLK iterations earlier, and loads
        // the next block, so no iteration waits on an index load.  The QK waves read chunk x's
        // slot at iteration x - 3, and its previous chunk (x - IRING) was read long before.
        // Addresses are clamped into the token's row.
        int *idx_ring = reinterpret_cast<int *>(lds + L::IDX);
        auto idx_load = [&](int x) { return idx_row[min(first + x * CHUNK + lane, a.W - 1)]; };
        int idx_blk[IBLK];

        // Iteration c: index block refill (every IBLK iterations), softmax of chunk c (its
        // scores and maxima arrived last iteration), then P.V of chunk c-1 (its P and V slot
        // arrived last iteration).
        auto iteration = [&](int c) __attribute__((always_inline)) {
            lds_barrier();
            if (w == 0 && c % IBLK == 0) {
#pragma unroll
                for (int j = 0; j < IBLK; j++) {
                    idx_ring[((c + IBLK + j) % IRING) * CHUNK + lane] = idx_blk[j];
                    idx_blk[j] = idx_load(c + 2 * IBLK + j);
                }
            }
            softmax(c);
            pv(c - 1);
        };

        auto run_range = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                acc[ct] = v16f{};
            if (nch == 0)
                return;
            // chunk -1 (read by P.V in iteration 0): a zero V slot, zero P and alpha 1
            {
                const int ot = tid - 256;
                uint8_t *z = lds + L::V + vslot(-1) * L::VSLOT;
                for (int x = ot; x < L::VSLOT / 16; x += 256)
                    *reinterpret_cast<v4i *>(z + 16 * x) = v4i{0, 0, 0, 0};
                for (int x = ot; x < L::PBUF / 16; x += 256)
                    *reinterpret_cast<v4i *>(lds + L::P + L::PBUF + 16 * x) = v4i{0, 0, 0, 0};
                if (ot < HG)
                    reinterpret_cast<float *>(lds + L::SCL)[HG + ot] = 1.0f;
            }
            if (w == 0) {
#pragma unroll
                for (int x = 0; x < IBLK; x++)
                    idx_ring[x * CHUNK + lane] = idx_load(x);
#pragma unroll
                for (int j = 0; j < IBLK; j++)
                    idx_blk[j] = idx_load(IBLK + j);
            }
            lds_barrier();                          // the index ring holds chunks 0 .. IBLK-1
            for (int c = 0;; c += 3) {
                iteration(c);
                if (c + 1 >= nch)
                    break;
                iteration(c + 1);
                if (c + 2 >= nch)
                    break;
                iteration(c + 2);
                if (c + 3 >= nch)
                    break;
            }
            lds_barrier();
            pv(nch - 1);
        };

        run_range();
        mfma_result_pad();                          // the last products have landed

        // ---- per-head results: l (per wave) and the running maximum --------------------------
#pragma unroll
        for (int ht = 0; ht < 2; ht++) {
            float lt = l_lane[ht];
            lt += __shfl_xor(lt, 16);
            lt += __shfl_xor(lt, 32);
            const int head = 16 * ht + nh;
            if (kq == ht) {
                fin[w * HG + head] = lt;
                if (w == 0)
                    fin[4 * HG + head] = m_run[ht];
            }
        }
        epilogue(acc);
    }
}

template <int RB, int QK, bool TWO>
hipError_t launch_one(const DecodeParams &p, hipStream_t stream)
{
    const unsigned blocks = (unsigned)p.T * (unsigned)p.groups * (unsigned)p.splits;
    hipLaunchKernelGGL((decode_kernel<RB, QK, TWO>), dim3(blocks), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

template <bool TWO>
hipError_t launch_shape(const DecodeParams &p, int row_bytes, int qk_dim, hipStream_t stream)
{
    if (row_bytes == 576 && qk_dim == 576)
        return launch_one<576, 576, TWO>(p, stream);
    if (row_bytes == 576 && qk_dim == 512)
        return launch_one<576, 512, TWO>(p, stream);
    if (row_bytes == 512 && qk_dim == 512)
        return launch_one<512, 512, TWO>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int tiles, int row_bytes, int qk_dim,
                         bool two_term, bool chunk_local, hipStream_t stream)
{
    if (tiles == 2)
        return launch_decode_g64(p, row_bytes, qk_dim, two_term, chunk_local, stream);
    if (tiles != 1 || chunk_local)
        return hipErrorInvalidValue;
    return two_term ? launch_shape<true>(p, row_bytes, qk_dim, stream)
                    : launch_shape<false>(p, row_bytes, qk_dim, stream);
}

}  // namespace smla
