// Sparse MLA decode for gfx950 (MI355X): index-driven row gather into LDS, QK^T and P.V on
// the block-scaled FP8 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4, online softmax with
// P quantized to E4M3, and a fused merge of split partials.
//
// Method (vLLM API pages): the formula is the sparse_mla_cute page's "What this module
// computes"; the E4M3-P recipe, the contiguous key split and the split merge are the
// attn_sparse page's module docstring and its SparseDcpDecode.kernel / merge methods.
//
// Work decomposition.  A workgroup (4 waves) takes one token t, one group of HT 32-head tiles
// and one of S contiguous key ranges of the token's clamped count (range s = [min(n, s per),
// + min(n - first, per)), per = ceil(n / S)).  The range is processed in chunks of 64 columns.
// Workgroups of the same token are placed on the same XCD (workgroups are dispatched to the 8
// XCDs round-robin), so the head groups of a token share the gathered rows in that XCD's L2 and
// the split partials of a token are merged through the same L2.
//
// Per chunk c (64 keys) and workgroup:
//   gather: the chunk's rows land in one of three LDS slots with 16-byte direct-to-LDS loads
//     (global_load_lds_dwordx4, issued two chunks ahead; masked columns load a zero row).  A
//     row-major slot layout keeps every load instruction on ~2 whole rows (coalesced); the
//     16-byte pieces of row r sit at XOR-permuted positions p ^ sw(r) so the 32-row operand
//     reads of QK and the transposed 8-row reads of P.V spread over the LDS banks.
//   QK: task (head tile, key tile of 32): S = K Q^T with A = 32 key rows (LDS), B = the 32
//     heads' Q fragments (VGPRs, loaded once), 9 steps of 64 bytes for 576-byte scores.  Lane
//     (h, u) of the accumulator holds keys 8i + 4u + j (reg 4i + j) of head h.
//   softmax: base-2 scores s2 = S * bmm1 log2(e) + (0 or -inf for masked keys), chunk max over
//     the 64 keys, running max m.  P is anchored at F = G + e, e = ceil(m - G) (G: the running
//     max after the first chunk that has one): P = 2^(s2 - F + log2 448) <= 448, rounded to
//     E4M3 by v_cvt_pk_fp8_f32 (two-term default: P = hi + lo/16, lo = E4M3(16 (P - hi))).
//     The accumulator stays in frame G and the chunk's P.V enters with weight 2^e, applied
//     exactly by the instruction's per-lane E8M0 B scale, so the accumulator is never
//     rescaled (only when e would exceed FRAME_LIMIT does the frame move, a rare path).  FP32
//     sums of the unquantized P are kept per lane in frame F.
//   P.V by columns: wave w owns latent columns [128 w, 128 w + 128) for every head of the
//     group: O^T (32 columns x 32 heads) += V^T (32 columns x 64 keys, read with
//     ds_read_b64_tr_b8 from the slot) P^T (64 keys x 32 heads, read from the P buffer in LDS).
//     The V^T fragments are read once per chunk and reused for every head tile.
//   The chunk loop is software-pipelined: iteration c runs QK(c), then the softmax of chunk c
//   next to P.V of chunk c-1 (MFMA and VALU work of one wave overlap), with two barriers.
//
// Epilogue: one range (S = 1): merge with the sink, BF16 output through an LDS tile (coalesced
// row stores) and the LSE.  S > 1: every range writes its FP32 partial (in register order, so
// reads and writes coalesce) and (G, l); the last range to finish (atomic ticket per token and
// head group) merges all partials in range order, weights 2^(G_s - M), writes the output and
// resets the ticket.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define SMLA_LDS(T) __attribute__((address_space(3))) T

constexpr int CHUNK = 64;                          // columns per gathered chunk
constexpr int SLOTS = 3;                           // KV slots in LDS
constexpr int RING = 4;                            // index / table ring entries
constexpr int NT = 256;                            // threads per workgroup (4 waves)
constexpr float ANCHOR = 448.0f;                   // P anchor: E4M3's largest finite value
constexpr float LOG2_ANCHOR = 8.807354922057604f;  // log2(448)
constexpr float LN2 = 0.6931471805599453f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr int FRAME_LIMIT = 64;                    // largest frame offset e applied by scale

// Masked columns gather this row, so their V bytes are zero (0 * anything stays finite).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[576];

template <int RB>
struct Geom {
    static constexpr int PIECES = RB / 16;          // 16-byte pieces of a row
    static constexpr int SLOT = CHUNK * RB;         // one chunk slot
    static constexpr int GI = CHUNK * PIECES / NT;  // gather loads per thread and chunk
    static_assert(CHUNK * PIECES % NT == 0, "gather pieces must tile the workgroup");
    // XOR applied to the piece index of row r.  576-byte rows (16 banks apart): 2 bits, keeps
    // a piece inside its 64-byte group.  512-byte rows (all on the same banks): 4 bits.
    __device__ static constexpr int sw(int r)
    {
        return RB == 576 ? ((r >> 2) & 3)
                         : (((r & 3) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1));
    }
};

// LDS carve-up (byte offsets).
template <int HT, int RB>
struct Lds {
    static constexpr int HG = 32 * HT;
    static constexpr int KV = 0;                               // [SLOTS][64 rows][RB]
    static constexpr int P = SLOTS * Geom<RB>::SLOT;           // [2 buf][2 term][HG][64]
    static constexpr int PTERM = HG * 64;
    static constexpr int PBUF = 2 * PTERM;
    static constexpr int ESC = P + 2 * PBUF;                   // [2 buf][32] words (byte ht)
    static constexpr int REB = ESC + 2 * 32 * 4;               // [2 buf][HT][32] int
    static constexpr int MX = REB + 2 * HT * 32 * 4;           // [2 kt][HG] float
    static constexpr int BIAS = MX + 2 * HG * 4;               // [RING][64] float
    static constexpr int ROWS = BIAS + RING * CHUNK * 4;       // [RING][64] pointer
    static constexpr int RAW = ROWS + RING * CHUNK * 8;        // [RING][64] int
    static constexpr int FIN = RAW + RING * CHUNK * 4;         // [4][HG]: l kt0, l kt1, G, e
    static constexpr int MISC = FIN + 4 * HG * 4;              // ticket
    static constexpr int TOTAL = MISC + 16;
    static constexpr int OUT_TILE = HG * 1024;                 // BF16 [HG][512], after the loop
    static_assert(OUT_TILE <= ESC, "output tile must fit in the KV and P regions");
    static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

__device__ inline v8i join(v4i x, v4i y)
{
    return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

template <typename T>
__device__ inline T lds_load(const uint8_t *base, int off)
{
    return *reinterpret_cast<const T *>(base + off);
}

__device__ inline uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const SMLA_LDS(uint8_t) *)p;
}

// D += A B on 32x32x64 FP8 with E8M0 scale 2^0 on A and the per-lane B scale byte OPB of sb
// (lane l scales column l % 32 of its own k half; here both halves carry the same byte).
template <int OPB>
__device__ inline v16f mfma_b(v8i a, v8i b, v16f c, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, OPB, sb);
}

__device__ inline v16f mfma_b_sel(int op, v8i a, v8i b, v16f c, int sb)
{
    switch (op) {
    case 0: return mfma_b<0>(a, b, c, sb);
    case 1: return mfma_b<1>(a, b, c, sb);
    case 2: return mfma_b<2>(a, b, c, sb);
    default: return mfma_b<3>(a, b, c, sb);
    }
}

__device__ inline v16f mfma_unit(v8i a, v8i b, v16f c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16-byte direct-to-LDS load per lane: lane l's bytes land at LDS address lds_base + 16 l
// (lds_base wave-uniform, in M0).  Inline asm, so that the compiler does not tie LDS reads of
// the other slots to this load's completion; completion is awaited explicitly (vm_wait +
// barrier).  M0 is saved and restored.
__device__ inline void dma16(const void *src, uint32_t lds_base)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %2, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds_base), "v"(src)
                 : "memory");
}

// 4-byte direct-to-LDS load per lane: lane l's word lands at lds_base + 4 l.
__device__ inline void dma4(const void *src, uint32_t lds_base)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %1\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dword %2, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(lds_base), "v"(src)
                 : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ inline void vm_wait()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// BF16 of a finite float, round to nearest even.
__device__ inline uint32_t bf16_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Workgroup b -> (token t, unit u of the token): tokens t = x + 8 k' go to XCD x (b % 8) while
// a multiple of 8 tokens remains; the tail is laid out linearly.
__device__ inline void unit_of(int b, int T, int U, int *t, int *u)
{
    const int tfull = (T / 8) * 8;
    if (b < tfull * U) {
        const int x = b & 7, k = b >> 3;
        *t = x + 8 * (k / U);
        *u = k % U;
    } else {
        const int r = b - tfull * U;
        *t = tfull + r / U;
        *u = r % U;
    }
}

template <int HT, int RB, int QK, bool TWO>
__global__ void __launch_bounds__(NT, 1) decode_kernel(DecodeParams a)
{
    using Gm = Geom<RB>;
    using L = Lds<HT, RB>;
    constexpr int HG = 32 * HT;
    constexpr int NS = QK / 64;                    // 64-byte steps of the score
    constexpr int KTW = HT == 4 ? 2 : 1;           // QK tasks per wave
    constexpr int GI = Gm::GI;

    __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int hl = lane & 31, u = lane >> 5;

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

    // ---- QK task of this wave: head tile qht, key tiles kt0 (and kt0 + 1 when KTW = 2) ----
    const bool has_qk = HT == 1 ? (wave < 2) : true;
    const int qht = HT == 4 ? wave : (HT == 2 ? (wave & 1) : 0);
    const int kt0 = HT == 4 ? 0 : (HT == 2 ? (wave >> 1) : (wave & 1));
    const int qhead = hg * HG + 32 * qht + hl;      // this lane's head for QK and softmax

    // Q fragments (B operand): lane (h, u) holds bytes 64 s + 32 u + [0, 32) of head h.
    v8i qf[NS];
    {
        const bool live = has_qk && qhead < a.H;
        const uint8_t *qp = a.q + (int64_t)t * a.q_st + (int64_t)(live ? qhead : 0) * a.q_sh;
#pragma unroll
        for (int s = 0; s < NS; s++) {
            v8i x = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            if (live)
                x = join(*reinterpret_cast<const v4i *>(qp + 64 * s + 32 * u),
                         *reinterpret_cast<const v4i *>(qp + 64 * s + 32 * u + 16));
            qf[s] = x;
        }
    }

    // ---- tables: row sources and score biases of chunk x from its raw indices -------------
    float *const bias_tab = reinterpret_cast<float *>(lds + L::BIAS);
    const uint8_t **const row_tab = reinterpret_cast<const uint8_t **>(lds + L::ROWS);
    const int32_t *const raw_tab = reinterpret_cast<const int32_t *>(lds + L::RAW);
    auto build = [&](int x, int raw) {  // wave 0, lane = column within the chunk
        const int pos = first + x * CHUNK + lane;
        const bool valid = pos < end && raw >= 0;
        const uint8_t *pool = (a.kv_b != nullptr && pos >= a.split_col) ? a.kv_b : a.kv_a;
        row_tab[(x % RING) * CHUNK + lane] = valid ? pool + (int64_t)raw * RB : g_zero_row;
        bias_tab[(x % RING) * CHUNK + lane] = valid ? 0.0f : -INFINITY;
    };
    // raw indices of chunk x into the ring (wave 0): the address is clamped into the token's
    // index row; values past the range are dropped by build()
    auto dma_raw = [&](int x) {
        const int pos = first + x * CHUNK + lane;
        dma4(idx_row + min(pos, a.W - 1),
             __builtin_amdgcn_readfirstlane(lds_addr(lds + L::RAW + (x % RING) * CHUNK * 4)));
    };
    // gather of chunk x into slot x % 3: 64 * PIECES positions, 64 consecutive per instruction;
    // position s holds piece (s % PIECES) ^ sw(row) of row s / PIECES
    auto gather = [&](int x) {
        const uint8_t *const *rs = row_tab + (x % RING) * CHUNK;
        const uint32_t dst = lds_addr(lds + L::KV + (x % SLOTS) * Gm::SLOT);
#pragma unroll
        for (int it = 0; it < GI; it++) {
            const int s0 = it * NT + wave * 64;
            const int s = s0 + lane;
            const int r = s / Gm::PIECES;
            const int p = (s - r * Gm::PIECES) ^ Gm::sw(r);
            dma16(rs[r] + 16 * p, __builtin_amdgcn_readfirstlane(dst + (uint32_t)s0 * 16u));
        }
    };

    // ---- prologue ---------------------------------------------------------------------
    if (wave == 0) {
#pragma unroll
        for (int x = 0; x < 3; x++) {
            if (x < nch) {
                const int pos = first + x * CHUNK + lane;
                build(x, pos < end ? idx_row[pos] : -1);
            }
        }
    }
    // Q and the indices above are the only compiler-tracked loads before the loop: wait for
    // them here, before any direct-to-LDS load is in flight
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    if (wave == 0 && 3 < nch)
        dma_raw(3);
    if (0 < nch)
        gather(0);
    if (wave == 0 && 4 < nch)
        dma_raw(4);
    if (1 < nch)
        gather(1);

    // ---- lane constants -------------------------------------------------------------------
    // QK A operand: row 32 kt + hl, pieces 4 s + 2 u and 4 s + 2 u + 1 (XOR sw(row)).
    int qk_base[KTW][2];
#pragma unroll
    for (int k = 0; k < KTW; k++) {
        const int r = 32 * (kt0 + k) + hl;
#pragma unroll
        for (int e = 0; e < 2; e++)
            qk_base[k][e] = r * RB + 16 * ((2 * u + e) ^ (RB == 576 ? Gm::sw(r) : 0));
    }
    // P.V A operand (V^T): lane 16 q + i reads, for read j (bytes 8 j .. 8 j + 7 of its k-block
    // g = q >> 1), half (i & 1) of row key(g, j, i >> 1), column piece 8 w + 2 ct + (q & 1).
    // MFMA k index k = 8 j + r of block g is key 32 g + 16 (j & 1) + 4 (j >> 1) + 8 (r >> 2) +
    // (r & 3): the order in which the softmax writes P (lane (h, u) of key tile g owns keys
    // 8 i' + 4 u + j', bytes 16 u + 4 i' + j' of the P row's block g).
    int v_off[4][4];
    {
        const int q = lane >> 4, i = lane & 15;
        const int g = q >> 1, r = i >> 1;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int key = 32 * g + 16 * (j & 1) + 4 * (j >> 1) + 8 * (r >> 2) + (r & 3);
#pragma unroll
            for (int ct = 0; ct < 4; ct++) {
                const int pc = 8 * wave + 2 * ct + (q & 1);
                v_off[j][ct] = key * RB + 16 * (pc ^ Gm::sw(key)) + 8 * (i & 1);
            }
        }
    }
    // P^T B operand: head 32 ht + hl, pieces 2 u and 2 u + 1 of its 64-byte row (XOR (h>>2)&3).
    const int p_sw = (hl >> 2) & 3;
    const int p_off0 = hl * 64 + 16 * ((2 * u) ^ p_sw);
    const int p_off1 = hl * 64 + 16 * ((2 * u + 1) ^ p_sw);

    // ---- state ------------------------------------------------------------------------------
    float m_run = -INFINITY;   // running max of head qhead (base 2)
    float frame = -INFINITY;   // G
    int ecur = 0;              // e of the last chunk: its anchor is F = G + e (kept as an
                               // integer: G + e is rounded in FP32, the offset must not be)
    float l_lane[KTW];         // this lane's share of the unquantized P sum, frame F
#pragma unroll
    for (int k = 0; k < KTW; k++)
        l_lane[k] = 0.0f;
    v16f acc[4][HT];           // O^T tiles: acc[ct][ht] = columns 128 w + 32 ct + .. x heads
#pragma unroll
    for (int ct = 0; ct < 4; ct++)
#pragma unroll
        for (int ht = 0; ht < HT; ht++)
            acc[ct][ht] = v16f{};

    const uint8_t *const kvl = lds + L::KV;

    for (int c = 0; c <= nch && nch > 0; c++) {
        // ---- B1: chunk c has landed; P, scales and frame moves of chunk c-1 are visible ----
        if (c + 1 < nch) {
            if (wave == 0 && c + 4 < nch)
                vm_wait<GI + 1>();
            else
                vm_wait<GI>();
        } else {
            vm_wait<0>();
        }
        __syncthreads();

        const int pb = (c + 1) & 1;  // P buffer of chunk c - 1
        if (c >= 1) {
            // frame moves of chunk c-1 (rare): rescale the accumulators by 2^-dG first
            const int *reb = reinterpret_cast<const int *>(lds + L::REB) + pb * HT * 32;
            int dg[HT];
            bool any = false;
#pragma unroll
            for (int ht = 0; ht < HT; ht++) {
                dg[ht] = reb[ht * 32 + hl];
                any |= dg[ht] != 0;
            }
            if (__any(any)) {
#pragma unroll
                for (int ht = 0; ht < HT; ht++)
#pragma unroll
                    for (int ct = 0; ct < 4; ct++)
#pragma unroll
                        for (int r = 0; r < 16; r++)
                            acc[ct][ht][r] = ldexpf(acc[ct][ht][r], -dg[ht]);
            }
        }

        // ---- QK(c) and the chunk max --------------------------------------------------------
        float s2[KTW][16];
        float mloc = -INFINITY;
        if (c < nch && has_qk) {
            const uint8_t *kvs = kvl + (c % SLOTS) * Gm::SLOT;
            v16f S[KTW];
#pragma unroll
            for (int k = 0; k < KTW; k++) {
                S[k] = v16f{};
#pragma unroll
                for (int s = 0; s < NS; s++) {
                    int o0, o1;
                    if constexpr (RB == 576) {
                        o0 = qk_base[k][0] + 64 * s;
                        o1 = qk_base[k][1] + 64 * s;
                    } else {
                        const int r = 32 * (kt0 + k) + hl;
                        o0 = r * RB + 16 * ((4 * s + 2 * u) ^ Gm::sw(r));
                        o1 = r * RB + 16 * ((4 * s + 2 * u + 1) ^ Gm::sw(r));
                    }
                    const v8i av = join(lds_load<v4i>(kvs, o0), lds_load<v4i>(kvs, o1));
                    S[k] = mfma_unit(av, qf[s], S[k]);
                }
            }
            const uint8_t *bt = reinterpret_cast<const uint8_t *>(bias_tab + (c % RING) * CHUNK);
#pragma unroll
            for (int k = 0; k < KTW; k++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const v4f b4 = lds_load<v4f>(bt, 4 * (32 * (kt0 + k) + 8 * i + 4 * u));
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        s2[k][4 * i + j] = fmaf(S[k][4 * i + j], a.scale_log2, b4[j]);
                        mloc = fmaxf(mloc, s2[k][4 * i + j]);
                    }
                }
            }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        }
        if constexpr (KTW == 1) {
            // the two key tiles of a head tile are in different waves: exchange their maxima
            if (c < nch) {
                float *mx = reinterpret_cast<float *>(lds + L::MX);
                if (has_qk && u == 0)
                    mx[kt0 * HG + 32 * qht + hl] = mloc;
                __syncthreads();
                if (has_qk)
                    mloc = fmaxf(mloc, mx[(kt0 ^ 1) * HG + 32 * qht + hl]);
            }
        }

        // ---- softmax(c): frame, P, sums --------------------------------------------------
        if (c < nch && has_qk) {
            const float m_new = fmaxf(m_run, mloc);
            int e = 0;       // this chunk's anchor offset F - G (after a frame move, if any)
            int dg = 0;      // frame move of this chunk (0 almost always)
            int shift = 0;   // the lane sums go from frame G + ecur to G + e: times 2^shift
            if (frame == -INFINITY) {
                frame = m_new;  // stays -inf until a chunk has an active column
            } else {
                e = (int)ceilf(m_new - frame);  // m_new - frame >= 0, far below 2^31
                shift = ecur - e;
                if (e > FRAME_LIMIT) {
                    dg = e;
                    frame += (float)e;
                    e = 0;
                }
            }
            ecur = e;
            const float fb = frame == -INFINITY ? 0.0f : (frame + (float)e) - LOG2_ANCHOR;
            m_run = m_new;

            uint8_t *pbase = lds + L::P + (c & 1) * L::PBUF;
            const int prow = 32 * qht + hl;
#pragma unroll
            for (int k = 0; k < KTW; k++) {
                float p[16];
                float lsum = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    p[r] = __builtin_amdgcn_exp2f(s2[k][r] - fb);  // exp2(-inf) = 0
                    lsum += p[r];
                }
                l_lane[k] = ldexpf(l_lane[k], shift) + lsum;
                v4i hi, lo;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * i], p[4 * i + 1], 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(p[4 * i + 2], p[4 * i + 3], w, true);
                    hi[i] = w;
                    if constexpr (TWO) {
                        const float h0 = __builtin_amdgcn_cvt_f32_fp8(w, 0);
                        const float h1 = __builtin_amdgcn_cvt_f32_fp8(w, 1);
                        const float h2 = __builtin_amdgcn_cvt_f32_fp8(w, 2);
                        const float h3 = __builtin_amdgcn_cvt_f32_fp8(w, 3);
                        int x = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[4 * i] - h0),
                                                                16.0f * (p[4 * i + 1] - h1), 0,
                                                                false);
                        x = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[4 * i + 2] - h2),
                                                            16.0f * (p[4 * i + 3] - h3), x, true);
                        lo[i] = x;
                    }
                }
                const int kt = kt0 + k;
                const int off = prow * 64 + 16 * ((2 * kt + u) ^ ((prow >> 2) & 3));
                *reinterpret_cast<v4i *>(pbase + off) = hi;
                if constexpr (TWO)
                    *reinterpret_cast<v4i *>(pbase + L::PTERM + off) = lo;
            }
            if (kt0 == 0 && u == 0) {
                uint8_t *esc = lds + L::ESC + (c & 1) * 128;
                esc[hl * 4 + qht] = (uint8_t)(127 + e);
                reinterpret_cast<int *>(lds + L::REB)[(c & 1) * HT * 32 + qht * 32 + hl] = dg;
            }
        }

        // ---- P.V(c-1) -----------------------------------------------------------------------
        if (c >= 1) {
            const uint8_t *kvs = kvl + ((c - 1) % SLOTS) * Gm::SLOT;
            const uint8_t *pbuf = lds + L::P + pb * L::PBUF;
            const int escw = reinterpret_cast<const int *>(lds + L::ESC + pb * 128)[hl];
            const int escl = escw - 0x04040404;  // the second term's 2^-4, per byte
            v8i vt[4];
#pragma unroll
            for (int ct = 0; ct < 4; ct++) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (SMLA_LDS(v2i) *)(kvs + v_off[j][ct]));
                    vt[ct][2 * j] = x[0];
                    vt[ct][2 * j + 1] = x[1];
                }
            }
#pragma unroll
            for (int ht = 0; ht < HT; ht++) {
                const uint8_t *pr = pbuf + ht * 32 * 64;
                const v8i bh = join(lds_load<v4i>(pr, p_off0), lds_load<v4i>(pr, p_off1));
                v8i bl = bh;
                if constexpr (TWO)
                    bl = join(lds_load<v4i>(pr + L::PTERM, p_off0),
                              lds_load<v4i>(pr + L::PTERM, p_off1));
#pragma unroll
                for (int ct = 0; ct < 4; ct++) {
                    acc[ct][ht] = mfma_b_sel(ht, vt[ct], bh, acc[ct][ht], escw);
                    if constexpr (TWO)
                        acc[ct][ht] = mfma_b_sel(ht, vt[ct], bl, acc[ct][ht], escl);
                }
            }
        }

        // ---- B2: P.V(c-1) done everywhere: slot (c-1)%3 and P buffer (c-1)&1 are free -------
        __syncthreads();
        if (wave == 0 && c + 5 < nch)
            dma_raw(c + 5);
        if (c + 2 < nch)
            gather(c + 2);
        if (wave == 0 && c + 3 < nch)
            build(c + 3, raw_tab[((c + 3) % RING) * CHUNK + lane]);
    }

    // ---- epilogue ---------------------------------------------------------------------------
    float *fin = reinterpret_cast<float *>(lds + L::FIN);  // [l kt0][l kt1][G][e int] x HG
    __syncthreads();
    if (has_qk) {
#pragma unroll
        for (int k = 0; k < KTW; k++) {
            const float lt = l_lane[k] + __shfl_xor(l_lane[k], 32);
            if (u == 0)
                fin[(kt0 + k) * HG + 32 * qht + hl] = lt;
        }
        if (kt0 == 0 && u == 0) {
            fin[2 * HG + 32 * qht + hl] = frame;
            reinterpret_cast<int *>(fin)[3 * HG + 32 * qht + hl] = ecur;
        }
    }
    __syncthreads();

    // per head tile: this lane's head, its frame G and sum l in frame G
    float g_h[HT], l_h[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        const int h = 32 * ht + hl;
        g_h[ht] = fin[2 * HG + h];
        const int e_end = reinterpret_cast<const int *>(fin)[3 * HG + h];
        l_h[ht] = ldexpf(fin[h] + fin[HG + h], e_end);
    }

    const int64_t tg = (int64_t)t * a.groups + hg;
    if (a.splits > 1) {
        // partial of this range: FP32 accumulators in register order, then (G, l) per head
        const int64_t ui = tg * a.splits + split;
        float *po = a.ws_o + ui * (HG * 512);
#pragma unroll
        for (int ct = 0; ct < 4; ct++)
#pragma unroll
            for (int ht = 0; ht < HT; ht++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int idx = ((((wave * 4 + ct) * HT + ht) * 4 + i) * 64 + lane) * 4;
                    *reinterpret_cast<v4f *>(po + idx) =
                        v4f{acc[ct][ht][4 * i], acc[ct][ht][4 * i + 1], acc[ct][ht][4 * i + 2],
                            acc[ct][ht][4 * i + 3]};
                }
        if (wave == 0 && u == 0) {
#pragma unroll
            for (int ht = 0; ht < HT; ht++) {
                a.ws_ml[(ui * HG + 32 * ht + hl) * 2 + 0] = g_h[ht];
                a.ws_ml[(ui * HG + 32 * ht + hl) * 2 + 1] = l_h[ht];
            }
        }
        __threadfence();
        __syncthreads();
        int *ticket = reinterpret_cast<int *>(lds + L::MISC);
        if (tid == 0)
            *ticket = atomicAdd(a.counters + tg, 1);
        __syncthreads();
        if (*ticket != a.splits - 1)
            return;
        __threadfence();
        // last range: merge every range's partial in range order (its own included, read back
        // from the workspace, so the result does not depend on which range finishes last)
        float big_g[HT];
#pragma unroll
        for (int ht = 0; ht < HT; ht++) {
            big_g[ht] = -INFINITY;
            for (int s = 0; s < a.splits; s++)
                big_g[ht] = fmaxf(big_g[ht],
                                  a.ws_ml[((tg * a.splits + s) * HG + 32 * ht + hl) * 2]);
            l_h[ht] = 0.0f;
#pragma unroll
            for (int ct = 0; ct < 4; ct++)
                acc[ct][ht] = v16f{};
        }
        for (int s = 0; s < a.splits; s++) {
            const int64_t us = tg * a.splits + s;
            const float *ps = a.ws_o + us * (HG * 512);
#pragma unroll
            for (int ht = 0; ht < HT; ht++) {
                const float gs = a.ws_ml[(us * HG + 32 * ht + hl) * 2];
                const float ls = a.ws_ml[(us * HG + 32 * ht + hl) * 2 + 1];
                const float w = gs == -INFINITY ? 0.0f : exp2f(gs - big_g[ht]);
                l_h[ht] += w * ls;
#pragma unroll
                for (int ct = 0; ct < 4; ct++) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int idx = ((((wave * 4 + ct) * HT + ht) * 4 + i) * 64 + lane) * 4;
                        const v4f x = *reinterpret_cast<const v4f *>(ps + idx);
#pragma unroll
                        for (int j = 0; j < 4; j++)
                            acc[ct][ht][4 * i + j] += w * x[j];
                    }
                }
            }
        }
#pragma unroll
        for (int ht = 0; ht < HT; ht++)
            g_h[ht] = big_g[ht];
        if (tid == 0)
            a.counters[tg] = 0;  // every range has arrived: ready for the next call
    }

    // ---- final: sink, normalization, BF16 tile in LDS, coalesced row stores, LSE ---------
    uint8_t *tile = lds;  // [HG][1024 bytes], over the KV and P regions
#pragma unroll
    for (int ht = 0; ht < HT; ht++) {
        const int head = hg * HG + 32 * ht + hl;
        const bool any = g_h[ht] != -INFINITY;
        float big_m = g_h[ht], big_l = l_h[ht], w = 1.0f;
        if (a.sinks != nullptr && head < a.H) {
            const float sk = a.sinks[head] * LOG2E;
            big_m = fmaxf(g_h[ht], sk);
            w = any ? exp2f(g_h[ht] - big_m) : 0.0f;
            big_l = w * l_h[ht] + ANCHOR * exp2f(sk - big_m);
        }
        const float inv = any ? a.bmm2 * w / big_l : 0.0f;
#pragma unroll
        for (int ct = 0; ct < 4; ct++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int col = 128 * wave + 32 * ct + 8 * i + 4 * u;
                uint2 pk;
                pk.x = bf16_bits(acc[ct][ht][4 * i] * inv) |
                       (bf16_bits(acc[ct][ht][4 * i + 1] * inv) << 16);
                pk.y = bf16_bits(acc[ct][ht][4 * i + 2] * inv) |
                       (bf16_bits(acc[ct][ht][4 * i + 3] * inv) << 16);
                *reinterpret_cast<uint2 *>(tile + (32 * ht + hl) * 1024 + 2 * col) = pk;
            }
        if (wave == 0 && u == 0 && head < a.H && a.lse != nullptr) {
            const float lse2 = any ? big_m - LOG2_ANCHOR + log2f(big_l) : -INFINITY;
            a.lse[(int64_t)t * a.H + head] = a.lse_log2 ? lse2 : lse2 * LN2;
        }
    }
    __syncthreads();
    const int heads_here = min(HG, a.H - hg * HG);
    for (int x = tid; x < heads_here * 64; x += NT) {
        const int row = x >> 6, part = x & 63;
        const v4i v = lds_load<v4i>(tile, row * 1024 + 16 * part);
        *reinterpret_cast<v4i *>(a.out + ((int64_t)t * a.H + hg * HG + row) * 512 + 8 * part) =
            v;
    }
}

template <int HT, int RB, int QK, bool TWO>
hipError_t launch_one(const DecodeParams &p, hipStream_t stream)
{
    const unsigned blocks = (unsigned)p.T * (unsigned)p.groups * (unsigned)p.splits;
    hipLaunchKernelGGL((decode_kernel<HT, RB, QK, TWO>), dim3(blocks), dim3(NT), 0, stream, p);
    return hipGetLastError();
}

template <int RB, int QK, bool TWO>
hipError_t launch_tiles(const DecodeParams &p, int tiles, hipStream_t stream)
{
    switch (tiles) {
    case 1: return launch_one<1, RB, QK, TWO>(p, stream);
    case 2: return launch_one<2, RB, QK, TWO>(p, stream);
    case 4: return launch_one<4, RB, QK, TWO>(p, stream);
    default: return hipErrorInvalidValue;
    }
}

template <bool TWO>
hipError_t launch_shape(const DecodeParams &p, int tiles, int row_bytes, int qk_dim,
                        hipStream_t stream)
{
    if (row_bytes == 576 && qk_dim == 576)
        return launch_tiles<576, 576, TWO>(p, tiles, stream);
    if (row_bytes == 576 && qk_dim == 512)
        return launch_tiles<576, 512, TWO>(p, tiles, stream);
    if (row_bytes == 512 && qk_dim == 512)
        return launch_tiles<512, 512, TWO>(p, tiles, stream);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int tiles, int row_bytes, int qk_dim,
                         bool two_term, hipStream_t stream)
{
    return two_term ? launch_shape<true>(p, tiles, row_bytes, qk_dim, stream)
                    : launch_shape<false>(p, tiles, row_bytes, qk_dim, stream);
}

}  // namespace smla
