// Sparse MLA decode for gfx950 (MI355X), 64 heads per workgroup with rows gathered straight
// into LDS.
//
// Method (vLLM API pages): the formula is the sparse_mla_cute page's "What this module
// computes"; the E4M3-P recipe, the contiguous key split and the split merge are the
// attn_sparse page's module docstring and its SparseDcpDecode.kernel / merge methods.  The
// arithmetic is that of the 32-head kernel (smla_decode.hip), operation for operation: the
// same QK instruction chains, the same integer-offset softmax frames, E4M3 P (two-term by
// default) at the 448 anchor, the same E8M0 chunk weights on the P.V instruction, the same
// order of the FP32 sums of the unquantized P and the same fused split merge, so under one
// split plan the two kernels agree bit for bit.
//
// Why this decomposition.  The 32-head kernel spends most of a chunk on a serial chain of
// latencies that every 32-head group pays again (row-load issue, index reads, QK, score
// exchange, softmax, P.V, one barrier per 64 columns), and the scattered row loads into
// registers cap the gather near 9 bytes per clock per CU.  Here one workgroup serves 64 heads,
// so each chunk's fixed costs are paid for twice the heads, and the rows go from memory to LDS
// without passing through registers (global_load_lds_dwordx4: measured at 6 TB/s from HBM and
// ~9 TB/s when the two head groups of a token meet in the XCD's L2).
//
// Workgroup: 8 waves (two per SIMD), one token, one group of 64 heads, one key range of the
// attn_sparse split, processed in chunks of 64 columns.
//   Gather: chunk c's rows land in LDS slot c % 3: the 512 latent bytes of key k at
//     k * 512 with 16-byte piece p stored at position p ^ vsw(k), the 64 rope bytes in a rope
//     region at k * 64 with piece 32 + q at position q ^ ((k >> 2) & 3).  Each load
//     instruction fills 1 KB of the slot (lane l -> 16 bytes at l * 16), so a lane fetches
//     whichever row piece the layout puts there; masked columns fetch a static zero row.
//     The loads are issued from inline assembly two chunks ahead and waited for with explicit
//     counts; the indices of the range are staged in LDS once, with masked columns at -1.
//   QK and softmax: wave w takes head tile w % 4 (16 heads) and key half w / 4 (32 keys):
//     S^T tiles of 16 keys x 16 heads on v_mfma_scale_f32_16x16x128_f8f6f4 (K from the slot,
//     Q fragments held in registers, the rope step on two 16x16x32 FP8 instructions); the
//     two key halves of a head exchange their maxima through LDS.
//   P.V: wave w owns output columns 64 w .. 64 w + 63 of all 64 heads:
//     O^T (32 columns x 32 heads) += V^T (ds_read_b64_tr_b8 from the slot) P^T on
//     v_mfma_scale_f32_32x32x64_f8f6f4, 2 column tiles x 2 head tiles (x 2 with two-term P).
//   Iteration c, two LDS-only barriers:
//     A: chunk c has landed, P and scales of chunk c-1 are visible.
//        QK of chunk c (maxima to LDS); V^T of chunk c-1 read into registers.
//     B: maxima visible, slot of chunk c-1 free.
//        Row loads of chunk c+2 into that slot; P.V products of chunk c-1 (matrix core, P
//        from its buffer) overlapping the softmax of chunk c (vector unit), which writes P
//        and scales into the other of the two P buffers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

using namespace dev;

constexpr int CHUNK = 64;                          // columns per chunk
constexpr int NT = 512;                            // threads per workgroup (8 waves)
constexpr int HG = 64;                             // heads per workgroup
constexpr int SLOTS = 3;                           // gathered chunks in LDS: c-1 .. c+1 / c+2

// Masked columns gather this row, so their bytes are zero (0 * anything stays finite).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row_g64[576];

// LDS carve-up (byte offsets); TAIL: 576-byte QK (a rope region per slot).
template <bool TAIL>
struct LdsG {
    static constexpr int LAT = CHUNK * 512;                    // latent bytes of a chunk
    static constexpr int SLOTB = LAT + (TAIL ? CHUNK * 64 : 0);
    static constexpr int V = 0;                                // [SLOTS] slots
    static constexpr int P = SLOTS * SLOTB;                    // [2 buf][2 term][64][64 keys]
    static constexpr int PTERM = HG * 64;
    static constexpr int PBUF = 2 * PTERM;
    static constexpr int ESC = P + 2 * PBUF;                   // [2 buf][64] int: E8M0 byte
    static constexpr int MX = ESC + 2 * HG * 4;                // [2 key halves][64] maxima
    static constexpr int FIN = MX + 2 * HG * 4;                // [4 key quarters][64] l, G, e
    static constexpr int IDX = FIN + 6 * HG * 4;               // [G64_MAX_RANGE] row indices
    static constexpr int MISC = IDX + G64_MAX_RANGE * 4;       // ticket, overflow flag
    static constexpr int TOTAL = MISC + 16;
    static constexpr int OUT_TILE = HG * 1024;                 // BF16 [64][512], after the loop
    static_assert(OUT_TILE <= P, "output tile must fit in the slots");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// One LDS-direct load: each lane's 16 bytes from `src` go to LDS byte m0 + 16 * lane.  Issued
// from inline assembly so that the compiler's wait counting does not see it (it would wait for
// every outstanding load before any LDS read); the kernel waits with explicit counts.  M0 is
// written here and used by nothing else in this kernel.
__device__ inline void lds_dma16(const uint8_t *src, uint32_t m0)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(src), "s"(m0));
}

template <int N>
__device__ inline void wait_dma()
{
    asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory");
}

// LDS byte address (M0 operand) of a pointer into the workgroup's LDS.
__device__ inline uint32_t lds_addr(const uint8_t *p)
{
    return (uint32_t)(uintptr_t)(const SMLA_LDS(uint8_t) *)p;
}

template <int RB, int QK, bool TWO>
__global__ void __launch_bounds__(NT, 1) decode_g64_kernel(DecodeParams a)
{
    constexpr bool TAIL = QK == 576;               // a fifth, 64-byte QK step (rope)
    using L = LdsG<TAIL>;

    __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;        // QK / softmax: row r of 16, lane group g
    const int ht = w & 3, kh = w >> 2;             // head tile (16 heads), key half (32 keys)
    const int hl = lane & 31, u = lane >> 5;       // P.V: head of the B / C columns, key block
    const int q4 = lane >> 4, i16 = lane & 15;     // transposed V reads

    int t, unit;
    unit_of(blockIdx.x, a.T, a.splits * a.groups, &t, &unit);
    const int hg = unit % a.groups;
    const int split = unit / a.groups;

    int n = a.lens[t];
    n = n < 0 ? 0 : (n > a.W ? a.W : n);
    const int per = (n + a.splits - 1) / a.splits;
    const int first = min(n, split * per);
    // the host keeps every range within the index staging buffer; the clamp only keeps LDS
    // accesses in bounds
    const int mine = min(min(n - first, per), G64_MAX_RANGE);
    const int nch = (mine + CHUNK - 1) / CHUNK;
    const int32_t *idx_row = a.indices + (int64_t)t * a.W;

    int *ix = reinterpret_cast<int *>(lds + L::IDX);
    int *flag = reinterpret_cast<int *>(lds + L::MISC) + 1;
    float *fin = reinterpret_cast<float *>(lds + L::FIN);  // [4][64] l, [64] G, [64] e (int)
    float *mxs = reinterpret_cast<float *>(lds + L::MX);   // [2][64]
    int *esc = reinterpret_cast<int *>(lds + L::ESC);

    // ---- Q fragments of head tile ht (B operand of QK): lane (n, g) holds, for head 16 ht + n
    // and step s, the q pieces 8 s + g and 8 s + 4 + g, and the rope piece 32 + g.
    v8i qf[4];
    v4i qt = v4i{0, 0, 0, 0};
    {
        const int head = hg * HG + 16 * ht + r;
        const bool live = head < a.H;
        const uint8_t *qp = a.q + (int64_t)t * a.q_st + (int64_t)(live ? head : 0) * a.q_sh;
        const int keep = live ? -1 : 0;            // padding heads keep zeros
#pragma unroll
        for (int s = 0; s < 4; s++)
            qf[s] = join(gload(qp + 16 * (8 * s + g)) & keep, gload(qp + 16 * (8 * s + 4 + g)) & keep);
        if (TAIL)
            qt = gload(qp + 16 * (32 + g)) & keep;
    }
    // ---- the range's row indices, masked columns (and the tail of the last chunk) at -1
    for (int i = tid; i < nch * CHUNK; i += NT) {
        int v = -1;
        if (i < mine) {
            v = idx_row[first + i];
            v = v < 0 ? -1 : v;
        }
        ix[i] = v;
    }
    if (tid == 0)
        *flag = 0;
    __syncthreads();                               // the only full fence before the loop

    const uint32_t lds0 = lds_addr(lds);
    const uint8_t *pool_a = a.kv_a, *pool_b = a.kv_b != nullptr ? a.kv_b : a.kv_a;
    const int split_col = a.kv_b != nullptr ? a.split_col : a.W;
    const uint64_t zero = (uint64_t)(uintptr_t)g_zero_row_g64;
    // address of 16-byte piece `piece` of the row at key `key` of chunk x
    auto src_of = [&](int x, int key, int piece) {
        const int raw = ix[x * CHUNK + key];
        const int pos = first + x * CHUNK + key;
        // both addresses computed, then selected: a branch here would serialize the index reads
        const uint64_t row = (uint64_t)(uintptr_t)(pos >= split_col ? pool_b : pool_a) +
                             (uint64_t)(uint32_t)max(raw, 0) * RB;
        const uint64_t base = raw < 0 ? zero : row;
        return (const uint8_t *)(base + 16 * piece);
    };
    constexpr int NDMA_HI = TAIL ? 5 : 4;          // loads per chunk of waves 0..3
    constexpr int NDMA_LO = 4;                     // loads per chunk of waves 4..7
    // Row loads of chunk x into its slot: latent instruction j of wave w fills granules
    // 64 (8 j + w) + lane, i.e. key 2 (8 j + w) + lane / 32, position lane % 32; the rope
    // instruction of wave w < 4 fills rope granules 64 w + lane: key 16 w + lane / 4.
    auto issue = [&](int x) {
        const uint32_t sb = lds0 + (x % SLOTS) * L::SLOTB;
        const uint8_t *src[5];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int gi = 64 * (8 * j + w) + lane, key = gi >> 5;
            src[j] = src_of(x, key, (gi & 31) ^ vsw(key));
        }
        if constexpr (TAIL) {
            const int gi = 64 * (w & 3) + lane, key = gi >> 2;
            src[4] = src_of(x, key, 32 + ((gi & 3) ^ ((key >> 2) & 3)));
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
            lds_dma16(src[j], sb + 1024 * (8 * j + w));
        if constexpr (TAIL) {
            if (w < 4)
                lds_dma16(src[4], sb + L::LAT + 1024 * w);
        }
    };
    // wait until this wave's loads of chunk x have landed, `later` chunks issued after it
    auto wait_landed = [&](bool later) {
        if (later) {
            if (w < 4)
                wait_dma<NDMA_HI>();
            else
                wait_dma<NDMA_LO>();
        } else {
            wait_dma<0>();
        }
    };

    // ---- per-wave state -------------------------------------------------------------------
    v16f acc[2][2];                                // O^T tiles: column tile 2 w + ct, heads 32 h2..
    v4f sc[2];                                     // scores of this wave's two key tiles
    float m_run = -INFINITY, frame = -INFINITY, l_lane[2] = {0.0f, 0.0f};
    int ecur = 0;
    bool preset = false, ovf = false;

    // transposed V reads of column tile ct: lane (q4, i16), read rho: key 32 (q4 >> 1) + 8 rho
    // + (i16 >> 1), half i16 & 1 of piece 2 (2 w + ct) + (q4 & 1)
    auto v_off = [&](int ct, int rho) {
        const int k = 32 * (q4 >> 1) + 8 * rho + (i16 >> 1);
        const int piece = 2 * (2 * w + ct) + (q4 & 1);
        return k * 512 + 16 * (piece ^ vsw(k)) + 8 * (i16 & 1);
    };

    // QK of chunk x: base-2 scores with masked keys at -inf into `sc` (lane (n, g): head
    // 16 ht + n, keys 16 (2 kh + kt) + 4 g + i), this wave's 32-key maximum per head to MX.
    auto qk = [&](int x) {
        const uint8_t *slot = lds + (x % SLOTS) * L::SLOTB;
        const uint64_t mk = __ballot(ix[x * CHUNK + lane] >= 0);
        v4f c[2];
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
            c[kt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; s++) {
#pragma unroll
            for (int kt = 0; kt < 2; kt++) {
                const int key = 16 * (2 * kh + kt) + r;
                const int sw = vsw(key);
                const v8i av = join(lds_load<v4i>(slot, key * 512 + 16 * ((8 * s + g) ^ sw)),
                                    lds_load<v4i>(slot, key * 512 + 16 * ((8 * s + 4 + g) ^ sw)));
                c[kt] = mfma16(av, qf[s], c[kt]);
            }
        }
        if constexpr (TAIL) {
#pragma unroll
            for (int kt = 0; kt < 2; kt++) {
                const int key = 16 * (2 * kh + kt) + r;
                const v4i rr = lds_load<v4i>(slot, L::LAT + key * 64 + 16 * (g ^ ((key >> 2) & 3)));
#pragma unroll
                for (int hh = 0; hh < 2; hh++)
                    c[kt] = mfma16k32(v2i{rr[2 * hh], rr[2 * hh + 1]},
                                      v2i{qt[2 * hh], qt[2 * hh + 1]}, c[kt]);
            }
        }
        mfma_result_pad();
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int key = 16 * (2 * kh + kt) + 4 * g + i;
                const float b = ((mk >> key) & 1u) ? 0.0f : -INFINITY;
                sc[kt][i] = fmaf(c[kt][i], a.scale_log2, b);
                mx = fmaxf(mx, sc[kt][i]);
            }
        }
        // maximum over the four lane groups (rows of 16 lanes)
        {
            const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx),
                                                              __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
            const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                              __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
        }
        if (g == 0)
            mxs[kh * HG + 16 * ht + r] = mx;
    };

    // softmax of chunk x (branch-free), from `sc` and both key halves' maxima: frame, P (to the
    // P buffer) and the E8M0 scale.  First pass: G is the running maximum after the first chunk
    // with an active column and e = ceil(m - G) >= 0; an offset beyond FRAME_LIMIT marks the
    // head for the second pass, which fixes G at the head's final maximum before the range
    // starts (e = ceil(m - G) <= 0, at least E_MIN), so no pass ever rescales the accumulators.
    auto softmax = [&](int x) {
        const int head = 16 * ht + r;
        const float m_chunk = fmaxf(mxs[head], mxs[HG + head]);
        const float m_new = fmaxf(m_run, m_chunk);
        const bool fresh = frame == -INFINITY;
        const float diff = fresh || m_new == -INFINITY ? 0.0f : m_new - frame;
        int e = (int)ceilf(fmaxf(diff, (float)E_MIN));
        ovf = ovf || e > FRAME_LIMIT;
        e = min(e, FRAME_LIMIT);                    // first pass after an overflow: unused
        const int shift = fresh ? 0 : ecur - e;
        frame = fresh ? m_new : frame;
        ecur = e;
        m_run = m_new;
        const float fb = frame == -INFINITY ? 0.0f : (frame + (float)e) - LOG2_ANCHOR;
        uint8_t *pbase = lds + L::P + (x & 1) * L::PBUF;
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
            float p[4];
            float lsum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p[i] = __builtin_amdgcn_exp2f(sc[kt][i] - fb);  // exp2(-inf) = 0
                lsum += p[i];
            }
            l_lane[kt] = ldexpf(l_lane[kt], shift) + lsum;
            int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hi, true);
            const int off = head * 64 + 16 * ((2 * kh + kt) ^ psw(head)) + 4 * g;
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
        }
        if (kh == 0 && g == 0)
            esc[(x & 1) * HG + head] = 127 + e;
    };

    // V^T of chunk x, read into registers before the barrier that frees the slot
    v8i vt[2];
    auto pv_read_v = [&](int x) {
        const uint8_t *vs = lds + (x % SLOTS) * L::SLOTB;
#pragma unroll
        for (int ct = 0; ct < 2; ct++) {
#pragma unroll
            for (int rho = 0; rho < 4; rho++) {
                const v2i y = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (SMLA_LDS(v2i) *)(vs + v_off(ct, rho)));
                vt[ct][2 * rho] = y[0];
                vt[ct][2 * rho + 1] = y[1];
            }
        }
    };
    // P.V of chunk x: P^T and the E8M0 scales from the chunk's P buffer, one head tile at a time
    auto pv_mma = [&](int x) {
        const uint8_t *pbuf = lds + L::P + (x & 1) * L::PBUF;
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            const int head = 32 * h2 + hl;
            const int o0 = head * 64 + 16 * ((2 * u) ^ psw(head));
            const int o1 = head * 64 + 16 * ((2 * u + 1) ^ psw(head));
            const int escw = esc[(x & 1) * HG + head];
            const v8i bh = join(lds_load<v4i>(pbuf, o0), lds_load<v4i>(pbuf, o1));
            v8i bl = bh;
            if constexpr (TWO)
                bl = join(lds_load<v4i>(pbuf + L::PTERM, o0), lds_load<v4i>(pbuf + L::PTERM, o1));
#pragma unroll
            for (int ct = 0; ct < 2; ct++) {
                acc[ct][h2] = mfma32(vt[ct], bh, acc[ct][h2], escw);
                if constexpr (TWO)  // the second term's 2^-4
                    acc[ct][h2] = mfma32(vt[ct], bl, acc[ct][h2], escw - 4);
            }
        }
    };

    auto run_range = [&]() __attribute__((always_inline)) {
        frame = preset ? m_run : -INFINITY;
        m_run = -INFINITY;
        l_lane[0] = 0.0f;
        l_lane[1] = 0.0f;
        ecur = 0;
        ovf = false;
#pragma unroll
        for (int ct = 0; ct < 2; ct++)
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
                acc[ct][h2] = v16f{};
        if (nch == 0)
            return;
        lds_barrier();                              // every slot is free
        issue(0);
        if (nch > 1)
            issue(1);
        wait_landed(nch > 1);                       // chunk 0
        for (int c = 0; c < nch; c++) {
            lds_barrier();                          // A: chunk c landed; P of chunk c-1 visible
            qk(c);
            if (c > 0)
                pv_read_v(c - 1);
            lds_barrier();                          // B: maxima visible; slot of chunk c-1 free
            if (c + 2 < nch)
                issue(c + 2);
            if (c > 0)
                pv_mma(c - 1);
            softmax(c);
            if (c + 1 < nch)
                wait_landed(c + 2 < nch);           // chunk c+1
        }
        lds_barrier();                              // P of the last chunk visible
        pv_read_v(nch - 1);
        pv_mma(nch - 1);
    };

    run_range();
    // second pass for the heads whose offset overflowed (rare): restart the range with their
    // frames fixed at their final maxima
    lds_barrier();
    if (__any(ovf) && lane == 0)
        *flag = 1;
    lds_barrier();
    if (*flag != 0) {
        preset = ovf;
        run_range();
    }

    // ---- per-head results: l per key quarter, G and e ---------------------------------------
#pragma unroll
    for (int kt = 0; kt < 2; kt++) {
        float lt = l_lane[kt];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int head = 16 * ht + r;
        if (g == 0) {
            fin[(2 * kh + kt) * HG + head] = lt;
            if (kh == 0 && kt == 0) {
                fin[4 * HG + head] = frame;
                reinterpret_cast<int *>(fin)[5 * HG + head] = ecur;
            }
        }
    }
    mfma_result_pad();
    lds_barrier();

    // ---- epilogue -----------------------------------------------------------------------------
    // acc[ct][h2]: O^T tile of columns 32 (2 w + ct) + .. x heads 32 h2 + ..; lane l holds head
    // 32 h2 + l % 32, columns 8 (rr / 4) + 4 (l / 32) + rr % 4 of the tile in register rr.
    float g_h[2], l_h[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++) {
        const int head = 32 * h2 + hl;
        g_h[h2] = fin[4 * HG + head];
        l_h[h2] = ldexpf(fin[head] + fin[HG + head] + fin[2 * HG + head] + fin[3 * HG + head],
                         reinterpret_cast<const int *>(fin)[5 * HG + head]);
    }
    const int64_t tg = (int64_t)t * a.groups + hg;
    // register-order index of accumulator element rr of tile (ct, h2): one 256-byte run per
    // register and tile, so every store and load instruction of the exchange is one run
    auto part_idx = [&](int ct, int h2, int rr) {
        return (((2 * w + ct) * 2 + h2) * 16 + rr) * 64 + lane;
    };
    if (a.splits > 1) {
        // Partial of this range: FP32 accumulators in register order, then (G, l) per head,
        // with device-scope (write-through) stores; each workgroup waits for its stores to
        // complete before it takes its ticket.
        const int64_t ui = tg * a.splits + split;
        float *po = a.ws_o + ui * (HG * 512);
#pragma unroll
        for (int ct = 0; ct < 2; ct++)
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++)
#pragma unroll
                for (int rr = 0; rr < 16; rr++)
                    store_device(po + part_idx(ct, h2, rr), acc[ct][h2][rr]);
        if (w == 0 && u == 0) {
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                store_device(a.ws_ml + (ui * HG + 32 * h2 + hl) * 2 + 0, g_h[h2]);
                store_device(a.ws_ml + (ui * HG + 32 * h2 + hl) * 2 + 1, l_h[h2]);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
        __syncthreads();
        int *ticket = reinterpret_cast<int *>(lds + L::MISC);
        if (tid == 0)
            *ticket = __hip_atomic_fetch_add(a.counters + tg, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (*ticket != a.splits - 1)
            return;
        // last range: merge every range's partial in range order, its own from registers and the
        // others from the workspace (the same sums whichever range arrives last)
        float own_g[2], own_l[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            own_g[h2] = g_h[h2];
            own_l[h2] = l_h[h2];
            const int head = 32 * h2 + hl;
            float big_g = -INFINITY;
            for (int s = 0; s < a.splits; s++) {
                const float gs = s == split
                                     ? own_g[h2]
                                     : load_device(a.ws_ml + ((tg * a.splits + s) * HG + head) * 2);
                big_g = fmaxf(big_g, gs);
            }
            g_h[h2] = big_g;
            l_h[h2] = 0.0f;
        }
        // weights and sums of the other ranges, in range order
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            const int head = 32 * h2 + hl;
            for (int s = 0; s < a.splits; s++) {
                const int64_t us = tg * a.splits + s;
                const float gs = s == split ? own_g[h2] : load_device(a.ws_ml + (us * HG + head) * 2);
                const float ls = s == split ? own_l[h2] : load_device(a.ws_ml + (us * HG + head) * 2 + 1);
                l_h[h2] += (gs == -INFINITY ? 0.0f : exp2f(gs - g_h[h2])) * ls;
            }
        }
        // one 16-register accumulator tile at a time, so at most 16 loaded values are live
#pragma unroll
        for (int ct = 0; ct < 2; ct++) {
#pragma unroll
            for (int h2 = 0; h2 < 2; h2++) {
                const int head = 32 * h2 + hl;
                v16f sum = v16f{};
                for (int s = 0; s < a.splits; s++) {
                    const int64_t us = tg * a.splits + s;
                    const float gs = s == split ? own_g[h2] : load_device(a.ws_ml + (us * HG + head) * 2);
                    const float w_s = gs == -INFINITY ? 0.0f : exp2f(gs - g_h[h2]);
                    if (s == split) {
#pragma unroll
                        for (int rr = 0; rr < 16; rr++)
                            sum[rr] += w_s * acc[ct][h2][rr];
                    } else {
                        const float *ps = a.ws_o + us * (HG * 512);
                        float v[16];
#pragma unroll
                        for (int rr = 0; rr < 16; rr++)
                            v[rr] = load_device(ps + part_idx(ct, h2, rr));
#pragma unroll
                        for (int rr = 0; rr < 16; rr++)
                            sum[rr] += w_s * v[rr];
                    }
                }
                acc[ct][h2] = sum;
            }
        }
        if (tid == 0)  // every range has arrived: ready for the next call
            __hip_atomic_store(a.counters + tg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- final: sink, normalization, BF16 tile in LDS, coalesced row stores, LSE ----------
    uint8_t *tile = lds;  // [64][1024 bytes], over the slots
#pragma unroll
    for (int h2 = 0; h2 < 2; h2++) {
        const int head = hg * HG + 32 * h2 + hl;
        const bool any = g_h[h2] != -INFINITY;
        float big_m = g_h[h2], big_l = l_h[h2], wgt = 1.0f;
        if (a.sinks != nullptr && head < a.H) {
            const float sk = a.sinks[head] * LOG2E;
            big_m = fmaxf(g_h[h2], sk);
            wgt = any ? exp2f(g_h[h2] - big_m) : 0.0f;
            big_l = wgt * l_h[h2] + ANCHOR * exp2f(sk - big_m);
        }
        const float inv = any ? a.bmm2 * wgt / big_l : 0.0f;
#pragma unroll
        for (int ct = 0; ct < 2; ct++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int col = 32 * (2 * w + ct) + 8 * i + 4 * u;
                uint2 pk;
                pk.x = bf16_bits(acc[ct][h2][4 * i] * inv) |
                       (bf16_bits(acc[ct][h2][4 * i + 1] * inv) << 16);
                pk.y = bf16_bits(acc[ct][h2][4 * i + 2] * inv) |
                       (bf16_bits(acc[ct][h2][4 * i + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(tile + (32 * h2 + hl) * 1024 + 2 * col) = pk;
            }
        }
        if (w == 0 && u == 0 && head < a.H && a.lse != nullptr) {
            const float lse2 = any ? big_m - LOG2_ANCHOR + log2f(big_l) : -INFINITY;
            a.lse[(int64_t)t * a.H + head] = a.lse_log2 ? lse2 : lse2 * LN2;
        }
    }
    lds_barrier();
    const int heads_here = min(HG, a.H - hg * HG);
    for (int x = tid; x < heads_here * 64; x += NT) {
        const int row = x >> 6, part = x & 63;
        const v4i v = lds_load<v4i>(tile, row * 1024 + 16 * part);
        *reinterpret_cast<v4i *>(a.out + ((int64_t)t * a.H + hg * HG + row) * 512 + 8 * part) = v;
    }
}

template <int RB, int QK, bool TWO>
hipError_t launch_g64_one(const DecodeParams &p, hipStream_t stream)
{
    const unsigned blocks = (unsigned)p.T * (unsigned)p.groups * (unsigned)p.splits;
    hipLaunchKernelGGL((decode_g64_kernel<RB, QK, TWO>), dim3(blocks), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

template <bool TWO>
hipError_t launch_g64_shape(const DecodeParams &p, int row_bytes, int qk_dim, hipStream_t stream)
{
    if (row_bytes == 576 && qk_dim == 576)
        return launch_g64_one<576, 576, TWO>(p, stream);
    if (row_bytes == 576 && qk_dim == 512)
        return launch_g64_one<576, 512, TWO>(p, stream);
    if (row_bytes == 512 && qk_dim == 512)
        return launch_g64_one<512, 512, TWO>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_g64(const DecodeParams &p, int row_bytes, int qk_dim, bool two_term,
                             hipStream_t stream)
{
    return two_term ? launch_g64_shape<true>(p, row_bytes, qk_dim, stream)
                    : launch_g64_shape<false>(p, row_bytes, qk_dim, stream);
}

}  // namespace smla
