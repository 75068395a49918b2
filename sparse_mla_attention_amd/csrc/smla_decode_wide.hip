// Sparse MLA decode for gfx950 (MI355X), wide variant: 64 heads per workgroup.
//
// Method (vLLM API pages): the formula is the sparse_mla_cute page's "What this module
// computes"; the E4M3-P recipe, the contiguous key split and the split merge are the
// attn_sparse page's module docstring and its SparseDcpDecode.kernel / merge methods.  The
// arithmetic is that of the 32-head kernel (smla_decode.hip): the same integer-offset softmax
// frames, E4M3 P (two-term by default) at the 448 anchor, E8M0 chunk weights on the P.V
// instruction, FP32 sums of the unquantized P and the same fused split merge.
//
// Why a second decomposition.  A token's gathered rows are read once per head group: at 128
// heads the 32-head kernel streams every row through the L1 caches four times, and the
// scattered 64-byte row pieces cap that stream near 10 TB/s over the chip (measured), so it
// spends ~4x the row bytes' L1 time.  Here a workgroup takes 64 heads (two passes per row at
// 128 heads) and keeps its FP32 output accumulators (64 heads x 512 columns, 128 KB) in the
// register file of four waves, one per SIMD, each allowed 512 registers.
//
// Every wave w (0..3) does all of the work for its own part of each 64-column chunk:
//   keys 16 w .. 16 w + 15: lane (r, g) = (lane % 16, lane / 16) loads row 16 w + r straight
//     into registers (16-byte pieces 8 s + 4 j + g and the rope piece 32 + g; each load
//     instruction reads 64 contiguous bytes of 16 rows), issued from inline assembly three
//     chunks ahead of use together with the row index of the chunk three further on, so no
//     load waits on an index load and the waits are explicit counts;
//   QK of those 16 keys for all 64 heads on v_mfma_scale_f32_16x16x128_f8f6f4 (four 16-head
//     tiles; the K rows are the A operand straight from the load registers, the Q fragments
//     are read from LDS, where Q sits for the whole range; the rope step on 16x16x32 FP8);
//     the base-2 scores stay in registers until the next iteration's softmax, and the wave's
//     16-key maximum per head goes to LDS;
//   the softmax of its 16 keys for all 64 heads (chunk maximum over the four waves' maxima),
//     writing E4M3 P and the per-head E8M0 scale to LDS; the latent bytes of its rows go to an
//     LDS V slot;
//   P.V for latent columns 128 w .. 128 w + 127 over all 64 keys of the chunk and all 64 heads:
//     O^T (32 columns x 32 heads) += V^T (ds_read_b64_tr_b8 from the V slot) P^T on
//     v_mfma_scale_f32_32x32x64_f8f6f4, 4 column tiles x 2 head tiles (x 2 with two-term P).
// Iteration c (one workgroup barrier): the loads of chunk c+3, the softmax of chunk c, the P.V
// of chunk c-1 and the QK of chunk c+1; three V slots hold chunks c-1 .. c+1.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_device.h"
#include "smla_internal.h"

namespace smla {
namespace {

using namespace dev;

constexpr int CHUNK = 64;                          // columns per chunk
constexpr int NW = 4;                              // waves per workgroup, one per SIMD
constexpr int NTW = 64 * NW;                       // threads per workgroup
constexpr int HGW = 64;                            // heads per workgroup
constexpr int NHT = HGW / 16;                      // 16-head QK tiles
constexpr int NH2 = HGW / 32;                      // 32-head P.V tiles
constexpr int NCT = 4;                             // 32-column P.V tiles per wave
constexpr int VSLOTS = 3;                          // V slots: chunks c-1 .. c+1

// Masked columns gather this row, so their bytes are zero (0 * anything stays finite).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row_wide[576];

// Latent q rows in LDS are padded by one 16-byte piece, so the 16 heads of one QK read (same
// piece, consecutive heads) land on 16 distinct bank groups.
constexpr int QL_PITCH = 512 + 16;

// LDS carve-up (byte offsets).
struct LdsW {
    static constexpr int VSLOT = CHUNK * 512;                  // latent bytes of one chunk
    static constexpr int V = 0;                                // [VSLOTS][64 keys][512]
    static constexpr int P = VSLOTS * VSLOT;                   // [2 buf][2 term][64][64]
    static constexpr int PTERM = HGW * 64;
    static constexpr int PBUF = 2 * PTERM;
    static constexpr int ESC = P + 2 * PBUF;                   // [2 buf][64] int: E8M0 byte
    static constexpr int MX = ESC + 2 * HGW * 4;               // [2 buf][64 heads][4 waves]
    static constexpr int FIN = MX + 2 * HGW * NW * 4;          // [4 waves][64] l, [64] G, e
    static constexpr int QR = FIN + (NW + 2) * HGW * 4;        // [64 heads][64] q rope
    static constexpr int QL = QR + HGW * 64;                   // [64 heads][512 + 16] q latent
    static constexpr int MISC = QL + HGW * QL_PITCH;           // ticket, overflow flag
    static constexpr int TOTAL = MISC + 16;
    static constexpr int OUT_TILE = HGW * 1024;                // BF16 [64][512], after the loop
    static_assert(OUT_TILE <= P, "output tile must fit in the V slots");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

__device__ inline int vslot_w(int x) { return (x + VSLOTS) % VSLOTS; }


// One row index, loaded like the rows (inline assembly, waited for with explicit counts).
__device__ inline void gload_idx_async(int &dst, const int32_t *p)
{
    asm volatile("global_load_dword %0, %1, off" : "=&v"(dst) : "v"(p));
}

template <int N>
__device__ inline void wait_vm_idx(int &x)
{
    asm volatile("s_waitcnt vmcnt(%1)" : "+v"(x) : "i"(N));
}

template <int RB, int QK, bool TWO>
__global__ void __launch_bounds__(NTW, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
decode_wide_kernel(DecodeParams a)
{
    constexpr bool TAIL = QK == 576;               // a fifth, 64-byte QK step (rope)
    constexpr int NLD = TAIL ? 9 : 8;              // row loads per lane and chunk
    constexpr int GRP = NLD + 1;                   // loads per chunk group: rows + one index
    using L = LdsW;

    __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;        // QK / softmax: row r of 16, lane group g
    const int key = 16 * w + r;                    // this lane's key within a chunk
    const int hl = lane & 31, u = lane >> 5;       // P.V: head of the B / C columns, key block

    int t, unit;
    unit_of(blockIdx.x, a.T, a.splits * a.groups, &t, &unit);
    const int hg = unit % a.groups;
    const int split = unit / a.groups;

    const int n_raw = a.lens[t];

    // Q of the 64 heads goes to LDS (latent rows at QL_PITCH, rope rows at 64 bytes):
    // lane (r, g) loads pieces 8 s + g and 8 s + 4 + g of head 16 ht + r, and rope piece 32 + g.
    v4i qv[NHT][8];
    v4i qt[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ht++) {
        const int head = hg * HGW + 16 * ht + r;
        const bool live = head < a.H;
        const uint8_t *qp = a.q + (int64_t)t * a.q_st + (int64_t)(live ? head : 0) * a.q_sh;
        // padding heads load head 0's row (in bounds) and keep zeros
        const int keep = live ? -1 : 0;
#pragma unroll
        for (int s = 0; s < 4; s++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                qv[ht][2 * s + j] = gload(qp + 16 * (8 * s + 4 * j + g)) & keep;
        qt[ht] = v4i{0, 0, 0, 0};
        if (TAIL)
            qt[ht] = gload(qp + 16 * (32 + g)) & keep;
    }

    const int n = n_raw < 0 ? 0 : (n_raw > a.W ? a.W : n_raw);
    const int per = (n + a.splits - 1) / a.splits;
    // one range: it starts at column 0 whatever the count, so the index loads need not wait
    const int first = a.splits == 1 ? 0 : min(n, split * per);
    const int mine = a.splits == 1 ? n : min(n - first, per);
    const int end = first + mine;
    const int nch = (mine + CHUNK - 1) / CHUNK;
    const int32_t *idx_row = a.indices + (int64_t)t * a.W;
    // index of this lane's key in chunk x (address clamped into the token's row)
    auto idx_addr = [&](int x) { return idx_row + min(first + x * CHUNK + key, a.W - 1); };

    int *flag = reinterpret_cast<int *>(lds + L::MISC) + 1;
    float *fin = reinterpret_cast<float *>(lds + L::FIN);  // [4][64] l, [64] G, [64] e (int)
    uint8_t *qr = lds + L::QR;

    int ix0 = *idx_addr(0), ix1 = *idx_addr(1), ix2 = *idx_addr(2);
    // Everything loaded so far has landed before the first asynchronous load is issued, so the
    // compiler's own wait counting never has to look past those loads.
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int ht = 0; ht < NHT; ht++) {
#pragma unroll
        for (int s = 0; s < 4; s++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                *reinterpret_cast<v4i *>(lds + L::QL + (16 * ht + r) * QL_PITCH +
                                         16 * (8 * s + 4 * j + g)) = qv[ht][2 * s + j];
        if (TAIL)
            *reinterpret_cast<v4i *>(qr + (16 * ht + r) * 64 + 16 * g) = qt[ht];
    }
    if (tid == 0)
        *flag = 0;

    // ---- per-wave state ------------------------------------------------------------------
    v16f acc[NCT][NH2];                            // O^T tiles: columns 32 (4 w + ct) .. x heads
    v4f sc[NHT];                                   // scores of the chunk whose softmax is next
    float m_run[NHT], frame[NHT], l_lane[NHT];
    int ecur[NHT];
    bool preset[NHT], ovf[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ht++) {
        m_run[ht] = -INFINITY;
        preset[ht] = false;
    }

    // transposed V reads: lane (q4, i16), read rho: key 32 (q4 >> 1) + 8 rho + (i16 >> 1),
    // half i16 & 1 of piece 2 tile + (q4 & 1)
    const int q4 = lane >> 4, i16 = lane & 15;
    auto v_off = [&](int ct, int rho) {
        const int k = 32 * (q4 >> 1) + 8 * rho + (i16 >> 1);
        const int piece = 2 * (NCT * w + ct) + (q4 & 1);
        return k * 512 + 16 * (piece ^ vsw(k)) + 8 * (i16 & 1);
    };

    // Issue the row loads of chunk x into `st` (raw: its index, arrived); returns the chunk's
    // mask of active keys (bit k: key 16 w + k), wave-uniform.
    auto issue = [&](int x, int raw, v4i(&st)[NLD]) {
        const int pos = first + x * CHUNK + key;
        const bool valid = pos < end && raw >= 0;
        const uint8_t *pool = (a.kv_b != nullptr && pos >= a.split_col) ? a.kv_b : a.kv_a;
        const uint8_t *row = (valid ? pool + (int64_t)raw * RB : g_zero_row_wide) + 16 * g;
        gload_row_async_acc(st, row);
        return (uint32_t)(__ballot(valid) & 0xFFFFu);
    };

    // QK of the chunk in `st` (16 keys x 64 heads): base-2 scores with masked keys at -inf
    // into `sc` (lane (n, g): head 16 ht + n, keys 16 w + 4 g + i), the wave's 16-key maximum
    // per head to the chunk's MX buffer, and the latent bytes to the chunk's V slot.
    auto qk = [&](int x, const v4i(&st)[NLD], uint32_t mk) {
        const uint8_t *qlb = lds + L::QL + r * QL_PITCH + 16 * g;  // this lane's q pieces
        v4f c[NHT];
#pragma unroll
        for (int ht = 0; ht < NHT; ht++)
            c[ht] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const v8i av = join(st[2 * s], st[2 * s + 1]);
#pragma unroll
            for (int ht = 0; ht < NHT; ht++) {
                const int ho = (16 * ht) * QL_PITCH;
                const v8i bq = join(lds_load<v4i>(qlb, ho + 16 * (8 * s)),
                                    lds_load<v4i>(qlb, ho + 16 * (8 * s + 4)));
                c[ht] = mfma16(av, bq, c[ht]);
            }
        }
        if constexpr (TAIL) {
#pragma unroll
            for (int ht = 0; ht < NHT; ht++) {
                const v4i q0 = lds_load<v4i>(qr, (16 * ht + r) * 64 + 16 * g);
#pragma unroll
                for (int hh = 0; hh < 2; hh++)
                    c[ht] = mfma16k32(v2i{st[8][2 * hh], st[8][2 * hh + 1]},
                                      v2i{q0[2 * hh], q0[2 * hh + 1]}, c[ht]);
            }
        }
        // latent bytes to the V slot while the products finish
        uint8_t *vs = lds + L::V + vslot_w(x) * L::VSLOT + key * 512;
        const int sw = vsw(key);
#pragma unroll
        for (int s = 0; s < 4; s++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                *reinterpret_cast<v4i *>(vs + 16 * ((8 * s + 4 * j + g) ^ sw)) = st[2 * s + j];
        mfma_result_pad();
        float *mxb = reinterpret_cast<float *>(lds + L::MX) + (x & 1) * HGW * NW;
#pragma unroll
        for (int ht = 0; ht < NHT; ht++) {
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float b = ((mk >> (4 * g + i)) & 1u) ? 0.0f : -INFINITY;
                sc[ht][i] = fmaf(c[ht][i], a.scale_log2, b);
                mx = fmaxf(mx, sc[ht][i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (g == ht)
                mxb[(16 * ht + r) * NW + w] = mx;
        }
    };

    // softmax of chunk x (branch-free), from the scores in `sc` and the four waves' maxima:
    // frame, P (to the chunk's P buffer) and E8M0 scales.  First pass: G is the running maximum
    // after the first chunk with an active column and e = ceil(m - G) >= 0; an offset beyond
    // FRAME_LIMIT marks the head for the second pass, which fixes G at the head's final maximum
    // before the range starts (e = ceil(m - G) <= 0, at least E_MIN), so no pass ever rescales
    // the accumulators.
    auto softmax = [&](int x) {
        const uint8_t *mxb = lds + L::MX + (x & 1) * HGW * NW * 4;
        uint8_t *pbase = lds + L::P + (x & 1) * L::PBUF;
#pragma unroll
        for (int ht = 0; ht < NHT; ht++) {
            const int head = 16 * ht + r;
            const v4f m4 = lds_load<v4f>(mxb, head * 16);
            const float m_chunk = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
            const float m_new = fmaxf(m_run[ht], m_chunk);
            const bool fresh = frame[ht] == -INFINITY;
            const float diff = fresh || m_new == -INFINITY ? 0.0f : m_new - frame[ht];
            int e = (int)ceilf(fmaxf(diff, (float)E_MIN));
            ovf[ht] = ovf[ht] || e > FRAME_LIMIT;
            e = min(e, FRAME_LIMIT);                // first pass after an overflow: unused
            const int shift = fresh ? 0 : ecur[ht] - e;
            frame[ht] = fresh ? m_new : frame[ht];
            ecur[ht] = e;
            m_run[ht] = m_new;
            const float fb = frame[ht] == -INFINITY ? 0.0f : (frame[ht] + (float)e) - LOG2_ANCHOR;
            float p[4];
            float lsum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p[i] = __builtin_amdgcn_exp2f(sc[ht][i] - fb);  // exp2(-inf) = 0
                lsum += p[i];
            }
            l_lane[ht] = ldexpf(l_lane[ht], shift) + lsum;
            int hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            hi = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], hi, true);
            const int off = head * 64 + 16 * (w ^ psw(head)) + 4 * g;
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
            if (w == 0 && g == ht)
                reinterpret_cast<int *>(lds + L::ESC)[(x & 1) * HGW + head] = 127 + e;
        }
    };

    // P.V of chunk x over this wave's 4 column tiles and both 32-head tiles
    auto pv = [&](int x) {
        const uint8_t *vs = lds + L::V + vslot_w(x) * L::VSLOT;
        const uint8_t *pbuf = lds + L::P + (x & 1) * L::PBUF;
        v8i bh[NH2], bl[NH2];
        int escw[NH2];
#pragma unroll
        for (int h2 = 0; h2 < NH2; h2++) {
            const int head = 32 * h2 + hl;
            const int o0 = head * 64 + 16 * ((2 * u) ^ psw(head));
            const int o1 = head * 64 + 16 * ((2 * u + 1) ^ psw(head));
            escw[h2] = reinterpret_cast<const int *>(lds + L::ESC)[(x & 1) * HGW + head];
            bh[h2] = join(lds_load<v4i>(pbuf, o0), lds_load<v4i>(pbuf, o1));
            bl[h2] = bh[h2];
            if constexpr (TWO)
                bl[h2] = join(lds_load<v4i>(pbuf + L::PTERM, o0),
                              lds_load<v4i>(pbuf + L::PTERM, o1));
        }
        auto read_vt = [&](int ct) {
            v8i vt;
#pragma unroll
            for (int rho = 0; rho < 4; rho++) {
                const v2i y = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (SMLA_LDS(v2i) *)(vs + v_off(ct, rho)));
                vt[2 * rho] = y[0];
                vt[2 * rho + 1] = y[1];
            }
            return vt;
        };
        v8i vcur = read_vt(0);
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
            v8i vnext = vcur;
            if (ct + 1 < NCT)
                vnext = read_vt(ct + 1);  // next tile's V^T in flight during these products
#pragma unroll
            for (int h2 = 0; h2 < NH2; h2++)
                acc[ct][h2] = mfma32(vcur, bh[h2], acc[ct][h2], escw[h2]);
            if constexpr (TWO) {
#pragma unroll
                for (int h2 = 0; h2 < NH2; h2++)  // the second term's 2^-4
                    acc[ct][h2] = mfma32(vcur, bl[h2], acc[ct][h2], escw[h2] - 4);
            }
            vcur = vnext;
        }
    };

    v4i st0[NLD], st1[NLD], st2[NLD];
    uint32_t mk0 = 0, mk1 = 0, mk2 = 0;

    // Per chunk x every lane issues one group of loads, in chunk order: the NLD row loads of
    // chunk x, then the index of chunk x + 3.  Iteration c issues the group of chunk c+3 into
    // the stage chunk c left (its index arrived with the group of chunk c), softmaxes chunk c,
    // runs P.V of chunk c-1 and QK of chunk c+1 (whose rows arrived once at most the index of
    // its own group and the two later groups are in flight).
    auto iteration = [&](int c, v4i(&ld)[NLD], int &ixl, uint32_t &mld, v4i(&cur)[NLD],
                         uint32_t mcur) __attribute__((always_inline)) {
        lds_barrier();
        wait_vm_idx<2 * GRP>(ixl);               // the index of chunk c+3
        mld = issue(c + 3, ixl, ld);
        gload_idx_async(ixl, idx_addr(c + 6));
        softmax(c);
        if (c > 0)
            pv(c - 1);
        wait_vm_acc<2 * GRP + 1>(cur);                // the rows of chunk c+1
        if (c + 1 < nch)
            qk(c + 1, cur, mcur);
    };

    auto run_range = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ht = 0; ht < NHT; ht++) {
            frame[ht] = preset[ht] ? m_run[ht] : -INFINITY;
            m_run[ht] = -INFINITY;
            l_lane[ht] = 0.0f;
            ecur[ht] = 0;
            ovf[ht] = false;
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
            for (int h2 = 0; h2 < NH2; h2++)
                acc[ct][h2] = v16f{};
        if (nch == 0)
            return;
        lds_barrier();                            // q rope and every LDS buffer are free
        mk0 = issue(0, ix0, st0);
        gload_idx_async(ix0, idx_addr(3));
        mk1 = issue(1, ix1, st1);
        gload_idx_async(ix1, idx_addr(4));
        mk2 = issue(2, ix2, st2);
        gload_idx_async(ix2, idx_addr(5));
        wait_vm_acc<2 * GRP + 1>(st0);                // the rows of chunk 0
        qk(0, st0, mk0);
        for (int c = 0;; c += 3) {
            iteration(c, st0, ix0, mk0, st1, mk1);
            if (c + 1 >= nch)
                break;
            iteration(c + 1, st1, ix1, mk1, st2, mk2);
            if (c + 2 >= nch)
                break;
            iteration(c + 2, st2, ix2, mk2, st0, mk0);
            if (c + 3 >= nch)
                break;
        }
        // every load has landed before the registers it targets can be reused
        wait_vm_acc<0>(st0);
        wait_vm_acc<0>(st1);
        wait_vm_acc<0>(st2);
        wait_vm_idx<0>(ix0);
        wait_vm_idx<0>(ix1);
        wait_vm_idx<0>(ix2);
        lds_barrier();                            // P and V slot of the last chunk
        pv(nch - 1);
    };

    run_range();
    // second pass for the heads whose offset overflowed (rare): restart the range with their
    // frames fixed at their final maxima
    lds_barrier();
    {
        bool any_ovf = false;
#pragma unroll
        for (int ht = 0; ht < NHT; ht++)
            any_ovf = any_ovf || ovf[ht];
        if (__any(any_ovf) && lane == 0)
            *flag = 1;
    }
    lds_barrier();
    if (*flag != 0) {
#pragma unroll
        for (int ht = 0; ht < NHT; ht++)
            preset[ht] = ovf[ht];
        ix0 = *idx_addr(0);
        ix1 = *idx_addr(1);
        ix2 = *idx_addr(2);
        __builtin_amdgcn_s_waitcnt(0);
        run_range();
    }

    // ---- per-head results: l (per wave), G and e ------------------------------------------
#pragma unroll
    for (int ht = 0; ht < NHT; ht++) {
        float lt = l_lane[ht];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        const int head = 16 * ht + r;
        if (g == ht) {
            fin[w * HGW + head] = lt;
            if (w == 0) {
                fin[NW * HGW + head] = frame[ht];
                reinterpret_cast<int *>(fin)[(NW + 1) * HGW + head] = ecur[ht];
            }
        }
    }
    mfma_result_pad();
    lds_barrier();

    // ---- epilogue ---------------------------------------------------------------------------
    // acc[ct][h2]: O^T tile of columns 32 (4 w + ct) + .. x heads 32 h2 + ..; lane l holds
    // head 32 h2 + l % 32, columns 8 (r / 4) + 4 (l / 32) + r % 4 of the tile in register r.
    float g_h[NH2], l_h[NH2];
#pragma unroll
    for (int h2 = 0; h2 < NH2; h2++) {
        const int head = 32 * h2 + hl;
        float ls = 0.0f;
#pragma unroll
        for (int v = 0; v < NW; v++)
            ls += fin[v * HGW + head];
        g_h[h2] = fin[NW * HGW + head];
        l_h[h2] = ldexpf(ls, reinterpret_cast<const int *>(fin)[(NW + 1) * HGW + head]);
    }
    const int64_t tg = (int64_t)t * a.groups + hg;
    // register-order index of accumulator element r of tile (ct, h2): one 256-byte run per
    // register and tile, so every store and load instruction of the exchange is one run
    auto part_idx = [&](int ct, int h2, int rr) {
        return (((w * NCT + ct) * NH2 + h2) * 16 + rr) * 64 + lane;
    };
    if (a.splits > 1) {
        // Partial of this range: FP32 accumulators in register order, then (G, l) per head,
        // with device-scope (write-through) stores; each workgroup waits for its stores to
        // complete before it takes its ticket.
        const int64_t ui = tg * a.splits + split;
        float *po = a.ws_o + ui * (HGW * 512);
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
#pragma unroll
            for (int h2 = 0; h2 < NH2; h2++)
#pragma unroll
                for (int rr = 0; rr < 16; rr++)
                    store_device(po + part_idx(ct, h2, rr), acc[ct][h2][rr]);
        if (w == 0 && u == 0) {
#pragma unroll
            for (int h2 = 0; h2 < NH2; h2++) {
                store_device(a.ws_ml + (ui * HGW + 32 * h2 + hl) * 2 + 0, g_h[h2]);
                store_device(a.ws_ml + (ui * HGW + 32 * h2 + hl) * 2 + 1, l_h[h2]);
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
        // last range: merge every range's partial in range order (its own included, read back
        // from the workspace, so the result does not depend on arrival order)
#pragma unroll
        for (int h2 = 0; h2 < NH2; h2++) {
            const int head = 32 * h2 + hl;
            float big_g = -INFINITY;
            for (int s = 0; s < a.splits; s++)
                big_g = fmaxf(big_g, load_device(a.ws_ml + ((tg * a.splits + s) * HGW + head) * 2));
            g_h[h2] = big_g;
            l_h[h2] = 0.0f;
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                acc[ct][h2] = v16f{};
        }
        for (int s = 0; s < a.splits; s++) {
            const int64_t us = tg * a.splits + s;
            const float *ps = a.ws_o + us * (HGW * 512);
#pragma unroll
            for (int h2 = 0; h2 < NH2; h2++) {
                const int head = 32 * h2 + hl;
                const float gs = load_device(a.ws_ml + (us * HGW + head) * 2);
                const float ls = load_device(a.ws_ml + (us * HGW + head) * 2 + 1);
                const float wgt = gs == -INFINITY ? 0.0f : exp2f(gs - g_h[h2]);
                l_h[h2] += wgt * ls;
#pragma unroll
                for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                    for (int rr = 0; rr < 16; rr++)
                        acc[ct][h2][rr] += wgt * load_device(ps + part_idx(ct, h2, rr));
            }
        }
        if (tid == 0)  // every range has arrived: ready for the next call
            __hip_atomic_store(a.counters + tg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- final: sink, normalization, BF16 tile in LDS, coalesced row stores, LSE ----------
    uint8_t *tile = lds;  // [64][1024 bytes], over the V slots
#pragma unroll
    for (int h2 = 0; h2 < NH2; h2++) {
        const int head = hg * HGW + 32 * h2 + hl;
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
        for (int ct = 0; ct < NCT; ct++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int col = 32 * (NCT * w + ct) + 8 * i + 4 * u;
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
    const int heads_here = min(HGW, a.H - hg * HGW);
    for (int x = tid; x < heads_here * 64; x += NTW) {
        const int row = x >> 6, part = x & 63;
        const v4i v = lds_load<v4i>(tile, row * 1024 + 16 * part);
        *reinterpret_cast<v4i *>(a.out + ((int64_t)t * a.H + hg * HGW + row) * 512 + 8 * part) = v;
    }
}

template <int RB, int QK, bool TWO>
hipError_t launch_wide_one(const DecodeParams &p, hipStream_t stream)
{
    const unsigned blocks = (unsigned)p.T * (unsigned)p.groups * (unsigned)p.splits;
    hipLaunchKernelGGL((decode_wide_kernel<RB, QK, TWO>), dim3(blocks), dim3(NTW), 0, stream, p);
    return hipGetLastError();
}

// The wide kernel serves the 576-byte rows of the 128-head shapes (512 latent + 64 rope bytes,
// QK over all 576); the other row shapes run on the 32-head kernel.
template <bool TWO>
hipError_t launch_wide_shape(const DecodeParams &p, int row_bytes, int qk_dim, hipStream_t stream)
{
    if (row_bytes == 576 && qk_dim == 576)
        return launch_wide_one<576, 576, TWO>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_wide(const DecodeParams &p, int row_bytes, int qk_dim, bool two_term,
                              hipStream_t stream)
{
    return two_term ? launch_wide_shape<true>(p, row_bytes, qk_dim, stream)
                    : launch_wide_shape<false>(p, row_bytes, qk_dim, stream);
}

}  // namespace smla
