// Sparse MLA decode for gfx950 (MI355X): index-driven row gather into LDS, QK^T and P.V on
// the block-scaled FP8 matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4, online softmax with
// P quantized to E4M3, and a fused merge of split partials.
//
// Method (vLLM API pages): the formula is the sparse_mla_cute page's "What this module
// computes"; the E4M3-P recipe, the contiguous key split and the split merge are the
// attn_sparse page's module docstring and its SparseDcpDecode.kernel / merge methods.
//
// Work decomposition.  A workgroup (4 waves) takes one token t, one group of 32 heads (the last
// group zero-padded) and one of S contiguous key ranges of the token's clamped count (range
// s = [min(n, s per), + min(n - first, per)), per = ceil(n / S)), processed in chunks of 64
// columns.  Workgroups of the same token are placed on the same XCD (workgroups are
// dispatched to the 8 XCDs round-robin), so the head groups of a token share its gathered rows
// in that XCD's L2 and the split partials of a token are merged through the same L2.
//
// Per chunk (64 keys):
//   gather: thread tid holds pieces 4 k + tid % 4 of row tid / 4 of the chunk (masked columns
//     read a zero row), loaded with global_load_dwordx4 (64 contiguous bytes of 16 rows per
//     wave instruction) into one of two register stages three chunks ahead and written with
//     ds_write_b128 two chunks ahead.  On MI355X this sustains several times the random-row
//     bandwidth of direct-to-LDS loads.  The XOR permutation sw(row) spreads the
//     32-row operand reads of QK and the transposed 8-row reads of P.V over the LDS banks.
//   QK (waves 0 and 1: key tile kt = wave of 32 keys): S = K Q^T with A = 32 key rows (LDS), B
//     = the 32 heads' Q fragments (VGPRs, loaded once), 9 steps of 64 bytes for 576-byte
//     scores, as two independent accumulation chains.  Lane (h, u) holds keys 8i + 4u + j (reg
//     4i + j) of head h.
//   softmax (waves 0 and 1): s2 = S * bmm1 log2(e) + (0 or -inf for masked keys), chunk max
//     over both key tiles, running max m.  P is anchored at F = G + e, e = ceil(m - G) (G: the
//     running max after the first chunk that has one): P = 2^(s2 - F + log2 448) <= 448,
//     rounded to E4M3 by v_cvt_pk_fp8_f32 (two-term default: P = hi + lo/16, lo = E4M3(16 (P -
//     hi))).  The accumulators stay in frame G and the chunk's P.V enters with weight 2^e,
//     applied exactly by the instruction's per-lane E8M0 B scale, so they are never rescaled
//     (only if e would exceed FRAME_LIMIT does the frame move, a rare path).  FP32 sums of the
//     unquantized P are kept per lane in frame F.
//   P.V by latent columns: O^T (32 columns x 32 heads) += V^T (32 columns x 64 keys, read with
//     ds_read_b64_tr_b8 from the slot) P^T (64 keys x 32 heads, from the P buffer in LDS).
//     Waves 2 and 3 own 256 columns each (16 instructions per chunk) while waves 0 and 1 run
//     QK (9) and the softmax, so the two roles' registers do not add up.
//   Software pipeline: iteration c runs QK(c+1), the softmax of chunk c and P.V of chunk c-1
//   as one straight-line block per wave (MFMA and VALU work interleave), with a single
//   workgroup barrier; four KV slots hold chunks c-1 .. c+2.
//
// Epilogue: one range (S = 1): merge with the sink, BF16 output through an LDS tile (coalesced
// row stores) and the LSE.  S > 1: every range writes its FP32 partial (in register order, so
// reads and writes coalesce) and (G, l); the last range to finish (atomic ticket per token and
// head group) merges all partials in range order, weights 2^(G_s - M), writes the output and
// resets the ticket.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "smla_internal.h"

namespace smla {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v8f __attribute__((ext_vector_type(8)));

#define SMLA_LDS(T) __attribute__((address_space(3))) T
#define SMLA_GLOBAL(T) __attribute__((address_space(1))) T

constexpr int CHUNK = 64;                          // columns per gathered chunk
constexpr int SLOTS = 4;                           // KV slots in LDS: chunks c-1 .. c+2
constexpr int RING = 4;                            // table entries: chunks c+1 .. c+4
constexpr int NT = 256;                            // threads per workgroup (4 waves)
constexpr int HG = 32;                             // heads per workgroup
constexpr float ANCHOR = 448.0f;                   // P anchor: E4M3's largest finite value
constexpr float LOG2_ANCHOR = 8.807354922057604f;  // log2(448)
constexpr float LN2 = 0.6931471805599453f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr int FRAME_LIMIT = 96;                    // largest frame offset e of the first pass
constexpr int E_MIN = -120;                        // smallest offset (preset frames)
constexpr int NCT = 8;                             // 32-column P.V tiles of waves 2 and 3

// Masked columns gather this row, so their V bytes are zero (0 * anything stays finite).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[576];

template <int RB>
struct Geom {
    static constexpr int PIECES = RB / 16;          // 16-byte pieces of a row
    static constexpr int SLOT = CHUNK * RB;         // one chunk slot
    static constexpr int GI = PIECES / 4;           // gather loads per thread and chunk
    static_assert(CHUNK * 4 == NT && PIECES % 4 == 0, "4 threads per row");
    // XOR applied to the piece index of row r.  576-byte rows (16 banks apart): 2 bits, keeps
    // a piece inside its 64-byte group.  512-byte rows (all on the same banks): 4 bits.
    __device__ static constexpr int sw(int r)
    {
        return RB == 576 ? ((r >> 2) & 3)
                         : (((r & 3) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1));
    }
};

// LDS carve-up (byte offsets).
template <int RB>
struct Lds {
    static constexpr int KV = 0;                               // [SLOTS][64 rows][RB]
    static constexpr int P = SLOTS * Geom<RB>::SLOT;           // [2 buf][2 term][32][64]
    static constexpr int PTERM = HG * 64;
    static constexpr int PBUF = 2 * PTERM;
    static constexpr int ESC = P + 2 * PBUF;                   // [2 buf][32] int: E8M0 byte 0
    static constexpr int MX = ESC + 2 * 32 * 4;                // [2 buf][2 kt][32] float
    static constexpr int BIAS = MX + 2 * 2 * 32 * 4;           // [RING][64] float
    static constexpr int ROWS = BIAS + RING * CHUNK * 4;       // [RING][64] pointer
    static constexpr int FIN = ROWS + RING * CHUNK * 8;        // [4][32]: l kt0, l kt1, G, e
    static constexpr int MISC = FIN + 4 * HG * 4;              // ticket, overflow flag
    static constexpr int TOTAL = MISC + 16;
    static constexpr int OUT_TILE = HG * 1024;                 // BF16 [32][512], after the loop
    static_assert(OUT_TILE <= P, "output tile must fit in the KV region");
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

// D += A B on 32x32x64 FP8 with E8M0 scale 2^0 on A and the per-lane B scale byte 0 of sb
// (lane l scales column l % 32 of its own k half; here both halves carry the same byte).
__device__ inline v16f mfma_b(v8i a, v8i b, v16f c, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

__device__ inline v16f mfma_unit(v8i a, v8i b, v16f c)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// BF16 of a finite float, round to nearest even.
__device__ inline uint32_t bf16_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Pad between the last matrix instruction of a chain and the first vector read of its result.
// The block-scaled 32x32x64 FP8 instruction runs 16 passes; a read scheduled 19 wait states
// after it was measured to return the chain's previous partial sum, so reads of a fresh result
// wait behind 24 explicit wait states (the compiler's own padding comes on top).
__device__ inline void mfma_result_pad()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that orders LDS only.  __syncthreads() is a workgroup fence over all
// memory, which makes every wave wait for its outstanding global loads before the barrier: the
// gather's loads in flight across iterations would be drained at every chunk.  The gathered
// rows reach LDS through registers, whose loads the compiler waits for before the LDS store.
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Device-scope (all XCDs) relaxed accesses of the split exchange: coherent without a fence
__device__ inline void store_device(float *p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline float load_device(const float *p)
{
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

template <int RB, int QK, bool TWO>
__global__ void __launch_bounds__(NT, 1) decode_kernel(DecodeParams a)
{
    using Gm = Geom<RB>;
    using L = Lds<RB>;
    constexpr int NS = QK / 64;                    // 64-byte steps of the score
    constexpr int GI = Gm::GI;

    __shared__ __attribute__((aligned(16))) uint8_t lds[L::TOTAL];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int hl = lane & 31, u = lane >> 5;
    const bool qk_wave = wave < 2;                 // waves 0, 1: QK and softmax of key tile
    const int kt = wave & 1;                       // kt = wave; waves 2, 3: P.V of latent
    const int tile0 = NCT * (wave & 1);            // columns [256 (wave - 2), + 256)

    int t, unit;
    unit_of(blockIdx.x, a.T, a.splits * a.groups, &t, &unit);
    const int hg = unit % a.groups;
    const int split = unit / a.groups;
    const int head = hg * HG + hl;                  // this lane's head (P.V columns of O^T)

    int n = a.lens[t];
    n = n < 0 ? 0 : (n > a.W ? a.W : n);
    const int per = (n + a.splits - 1) / a.splits;
    const int first = min(n, split * per);
    const int mine = min(n - first, per);
    const int end = first + mine;
    const int nch = (mine + CHUNK - 1) / CHUNK;
    const int32_t *idx_row = a.indices + (int64_t)t * a.W;

    // Registers shared by the two roles: the P.V accumulators of waves 2 and 3 are, in waves 0
    // and 1, the Q fragments (B operand of QK: lane (h, u) holds bytes 64 s + 32 u + [0, 32) of
    // head h, step s in half s & 1 of acc[s >> 1]).  Each wave needs only one of the two.
    static_assert(NS <= 2 * NCT, "Q fragments must fit in the accumulator registers");
    v16f acc[NCT];             // O^T tiles (waves 2, 3): columns 32 (tile0 + ct) + .. x heads
#pragma unroll
    for (int ct = 0; ct < NCT; ct++)
        acc[ct] = v16f{};
    {
        const bool live = qk_wave && head < a.H;
        const uint8_t *qp = a.q + (int64_t)t * a.q_st + (int64_t)(live ? head : 0) * a.q_sh;
        if (live) {
#pragma unroll
            for (int s = 0; s < NS; s++) {
                const v4f x0 = *reinterpret_cast<const v4f *>(qp + 64 * s + 32 * u);
                const v4f x1 = *reinterpret_cast<const v4f *>(qp + 64 * s + 32 * u + 16);
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    acc[s >> 1][8 * (s & 1) + k] = x0[k];
                    acc[s >> 1][8 * (s & 1) + 4 + k] = x1[k];
                }
            }
        }
    }
    auto qfrag = [&](int s) {  // Q fragment of step s (QK waves)
        const v16f &h = acc[s >> 1];
        const int o = 8 * (s & 1);
        return __builtin_bit_cast(v8i, (v8f){h[o], h[o + 1], h[o + 2], h[o + 3], h[o + 4],
                                             h[o + 5], h[o + 6], h[o + 7]});
    };

    // ---- tables: row sources and score biases of chunk x from its raw indices -------------
    float *const bias_tab = reinterpret_cast<float *>(lds + L::BIAS);
    const uint8_t **const row_tab = reinterpret_cast<const uint8_t **>(lds + L::ROWS);
    auto build = [&](int x, int raw) {  // wave 0, lane = column within the chunk
        const int pos = first + x * CHUNK + lane;
        const bool valid = pos < end && raw >= 0;
        const uint8_t *pool = (a.kv_b != nullptr && pos >= a.split_col) ? a.kv_b : a.kv_a;
        row_tab[(x % RING) * CHUNK + lane] = valid ? pool + (int64_t)raw * RB : g_zero_row;
        bias_tab[(x % RING) * CHUNK + lane] = valid ? 0.0f : -INFINITY;
    };
    // raw index of column `lane` of chunk x (wave 0): the address is clamped into the token's
    // index row; values past the range are dropped by build()
    auto load_raw = [&](int x) { return idx_row[min(first + x * CHUNK + lane, a.W - 1)]; };
    // Gather mapping: thread tid loads row g_row = tid / 4 of the chunk, pieces 4 k + g_q
    // (k < GI, g_q = tid % 4): each wave load instruction reads 64 contiguous bytes of 16 rows,
    // each thread needs one row pointer per chunk, and the ds_write_b128 of a 16-lane group
    // covers 4 rows x 4 pieces on distinct banks.
    const int g_row = tid >> 2, g_q = tid & 3;
    auto g_pos = [&](int k) {  // LDS byte offset of piece 4 k + g_q of row g_row in a slot
        return g_row * RB + 16 * ((4 * k + g_q) ^ Gm::sw(g_row));
    };
    v4i stage_a[GI], stage_b[GI];  // register stages: chunk x lives in stage (x even ? a : b)
    // Loads are issued for every chunk slot of the pipeline, reading the zero row past the
    // range, so that the number of loads in flight is the same on every path and the compiler's
    // wait counts stay partial (a conditional load makes it wait for every load in flight).
    auto gather_load = [&](int x, bool live, v4i(&stage)[GI]) {
        const uint8_t *row = live ? row_tab[(x % RING) * CHUNK + g_row] : g_zero_row;
#pragma unroll
        for (int k = 0; k < GI; k++)
            // global (not flat) loads: flat loads would also hold the LDS counter, and every
            // LDS wait of the chunk's compute would wait for this gather
            stage[k] = *(const SMLA_GLOBAL(v4i) *)(row + 16 * (4 * k + g_q));
    };
    auto gather_store = [&](int x, const v4i(&stage)[GI]) {
        uint8_t *dst = lds + L::KV + (x & (SLOTS - 1)) * Gm::SLOT;
#pragma unroll
        for (int k = 0; k < GI; k++)
            *reinterpret_cast<v4i *>(dst + g_pos(k)) = stage[k];
    };

    // ---- lane constants -------------------------------------------------------------------
    // QK A operand: row 32 kt + hl, pieces 4 s + 2 u and 4 s + 2 u + 1 (XOR sw(row)).
    const int qk_row = 32 * kt + hl;
    const int qk_base0 = qk_row * RB + 16 * ((2 * u) ^ (RB == 576 ? Gm::sw(qk_row) : 0));
    const int qk_base1 = qk_row * RB + 16 * ((2 * u + 1) ^ (RB == 576 ? Gm::sw(qk_row) : 0));
    // P.V A operand (V^T): lane 16 q + i reads, for read j (bytes 8 j .. 8 j + 7 of its k-block
    // g = q >> 1), half (i & 1) of row key(g, j, i >> 1), column piece 2 tile + (q & 1).  MFMA k
    // index 8 j + r of block g is key 32 g + 16 (j & 1) + 4 (j >> 1) + 8 (r >> 2) + (r & 3):
    // the order in which the softmax writes P (lane (h, u) of key tile g owns keys 8 i' + 4 u +
    // j', bytes 16 u + 4 i' + j' of the P row's block g).
    // 576-byte rows: sw(key) < 4 only permutes pieces inside 64-byte groups, so the address of
    // tile `tile` is base[j][tile & 1] + 64 (tile >> 1) (an immediate offset per tile).
    const int vq = lane >> 4, vi = lane & 15;
    const int vg = vq >> 1, vr = vi >> 1;
    auto v_key = [&](int j) {
        return 32 * vg + 16 * (j & 1) + 4 * (j >> 1) + 8 * (vr >> 2) + (vr & 3);
    };
    auto v_addr = [&](int j, int tile) {  // byte offset of lane's read j of 32-column tile
        const int key = v_key(j);
        const int pc = 2 * tile + (vq & 1);
        return key * RB + 16 * (pc ^ Gm::sw(key)) + 8 * (vi & 1);
    };
    int v_base[4][2];
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int par = 0; par < 2; par++)
            v_base[j][par] = v_addr(j, par);  // tiles 0 / 1; tile t adds 64 (t >> 1)
    // P^T B operand: head hl, pieces 2 u and 2 u + 1 of its 64-byte row (XOR (h >> 2) & 3).
    const int p_sw = (hl >> 2) & 3;
    const int p_off0 = hl * 64 + 16 * ((2 * u) ^ p_sw);
    const int p_off1 = hl * 64 + 16 * ((2 * u + 1) ^ p_sw);

    // ---- state ------------------------------------------------------------------------------
    float m_run = -INFINITY;   // running max of head `head` (base 2)
    float frame = -INFINITY;   // G
    int ecur = 0;              // e of the last chunk: its anchor is F = G + e (kept as an
                               // integer: G + e is rounded in FP32, the offset must not be)
    bool preset = false;       // G fixed before the range (second pass)
    bool overflow = false;     // some chunk's offset exceeded FRAME_LIMIT (first pass)
    float l_lane = 0.0f;       // this lane's share of the unquantized P sum, frame F
    v16f s_cur = v16f{};       // base-2 scores of chunk c (this wave's key tile)
    float mloc_cur = -INFINITY;

    // QK of chunk x from its slot (two accumulation chains: even and odd steps), then the
    // base-2 scores with masked keys at -inf and this key tile's maximum per head
    auto qk = [&](int x, float *mloc_out) {
        const uint8_t *kvs = lds + L::KV + (x & (SLOTS - 1)) * Gm::SLOT;
        v16f s0 = v16f{}, s1 = v16f{};
#pragma unroll
        for (int s = 0; s < NS; s++) {
            int o0, o1;
            if constexpr (RB == 576) {
                o0 = qk_base0 + 64 * s;
                o1 = qk_base1 + 64 * s;
            } else {
                o0 = qk_row * RB + 16 * ((4 * s + 2 * u) ^ Gm::sw(qk_row));
                o1 = qk_row * RB + 16 * ((4 * s + 2 * u + 1) ^ Gm::sw(qk_row));
            }
            const v8i av = join(lds_load<v4i>(kvs, o0), lds_load<v4i>(kvs, o1));
            if (s & 1)
                s1 = mfma_unit(av, qfrag(s), s1);
            else
                s0 = mfma_unit(av, qfrag(s), s0);
        }
        mfma_result_pad();
        const v16f sc = s0 + s1;
        const uint8_t *bt = reinterpret_cast<const uint8_t *>(bias_tab + (x % RING) * CHUNK);
        v16f s2;
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const v4f b4 = lds_load<v4f>(bt, 4 * (32 * kt + 8 * i + 4 * u));
#pragma unroll
            for (int j = 0; j < 4; j++) {
                s2[4 * i + j] = fmaf(sc[4 * i + j], a.scale_log2, b4[j]);
                mx = fmaxf(mx, s2[4 * i + j]);
            }
        }
        *mloc_out = fmaxf(mx, __shfl_xor(mx, 32));
        return s2;
    };

    // softmax of chunk x (branch-free): frame, P (written to the chunk's P buffer) and the
    // E8M0 scale byte of each head.  First pass: G is the running max after the first chunk
    // with an active column and e = ceil(m - G) >= 0; an offset beyond FRAME_LIMIT (scores
    // grown by that many binades: the FP32 accumulators could overflow) marks the head for the
    // second pass, which fixes G at the head's final maximum before the range starts (e =
    // ceil(m - G) <= 0, at least E_MIN), so no pass ever rescales the accumulators.
    auto softmax = [&](int x, const v16f &s2, float mloc) {
        const float *mxb = reinterpret_cast<const float *>(lds + L::MX) + (x & 1) * 64;
        const float m_chunk = fmaxf(mloc, mxb[(kt ^ 1) * 32 + hl]);
        const float m_new = fmaxf(m_run, m_chunk);
        const bool fresh = frame == -INFINITY;  // no active column before this chunk
        const float diff = fresh || m_new == -INFINITY ? 0.0f : m_new - frame;
        int e = (int)ceilf(fmaxf(diff, (float)E_MIN));
        overflow = overflow || e > FRAME_LIMIT;
        e = min(e, FRAME_LIMIT);                // first pass after an overflow: result unused
        const int shift = fresh ? 0 : ecur - e;   // lane sum: frame G + ecur -> G + e
        frame = fresh ? m_new : frame;
        ecur = e;
        m_run = m_new;
        const float fb = frame == -INFINITY ? 0.0f : (frame + (float)e) - LOG2_ANCHOR;
        float p[16];
        float lsum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            p[r] = __builtin_amdgcn_exp2f(s2[r] - fb);  // exp2(-inf) = 0
            lsum += p[r];
        }
        l_lane = ldexpf(l_lane, shift) + lsum;
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
                int y = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[4 * i] - h0),
                                                        16.0f * (p[4 * i + 1] - h1), 0, false);
                y = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[4 * i + 2] - h2),
                                                    16.0f * (p[4 * i + 3] - h3), y, true);
                lo[i] = y;
            }
        }
        uint8_t *pbase = lds + L::P + (x & 1) * L::PBUF;
        const int off = hl * 64 + 16 * ((2 * kt + u) ^ ((hl >> 2) & 3));
        *reinterpret_cast<v4i *>(pbase + off) = hi;
        if constexpr (TWO)
            *reinterpret_cast<v4i *>(pbase + L::PTERM + off) = lo;
        if (kt == 0 && u == 0)
            reinterpret_cast<int *>(lds + L::ESC)[(x & 1) * 32 + hl] = 127 + e;
    };

    // P.V of chunk x over this wave's NCT column tiles
    auto pv = [&](int x) {
        const uint8_t *kvs = lds + L::KV + (x & (SLOTS - 1)) * Gm::SLOT;
        const uint8_t *pbuf = lds + L::P + (x & 1) * L::PBUF;
        const int escw = reinterpret_cast<const int *>(lds + L::ESC)[(x & 1) * 32 + hl];
        const int escl = escw - 4;  // the second term's 2^-4
        const v8i bh = join(lds_load<v4i>(pbuf, p_off0), lds_load<v4i>(pbuf, p_off1));
        v8i bl = bh;
        if constexpr (TWO)
            bl = join(lds_load<v4i>(pbuf + L::PTERM, p_off0),
                      lds_load<v4i>(pbuf + L::PTERM, p_off1));
        auto read_vt = [&](int ct) {
            const int tl = tile0 + ct;
            v8i vt;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int off = RB == 576 ? v_base[j][tl & 1] + 64 * (tl >> 1) : v_addr(j, tl);
                const v2i y = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SMLA_LDS(v2i) *)(kvs + off));
                vt[2 * j] = y[0];
                vt[2 * j + 1] = y[1];
            }
            return vt;
        };
        v8i vcur = read_vt(0);
#pragma unroll
        for (int ct = 0; ct < NCT; ct++) {
            v8i vnext = vcur;
            if (ct + 1 < NCT)
                vnext = read_vt(ct + 1);  // next tile's V^T in flight during these products
            acc[ct] = mfma_b(vcur, bh, acc[ct], escw);
            if constexpr (TWO)
                acc[ct] = mfma_b(vcur, bl, acc[ct], escl);
            vcur = vnext;
        }
    };

    // The range: prologue, pipelined loop and drain (run twice when a head overflows).
    auto run_range = [&]() __attribute__((always_inline)) {
    // ---- prologue: tables 0..3, chunks 0 and 1 in their slots, chunk 2 in flight, QK(0) ----
    if (wave == 0) {
#pragma unroll
        for (int x = 0; x < 3; x++) {
            if (x < nch) {
                const int pos = first + x * CHUNK + lane;
                build(x, pos < end ? idx_row[pos] : -1);
            }
        }
    }
    // chunk -1 (read by P.V in iteration 0): a zero slot, zero P and a unit scale, so the
    // pipeline needs no special first iteration
    {
        uint8_t *z = lds + L::KV + (SLOTS - 1) * Gm::SLOT;
        for (int x = tid; x < Gm::SLOT / 16; x += NT)
            *reinterpret_cast<v4i *>(z + 16 * x) = v4i{0, 0, 0, 0};
        for (int x = tid; x < L::PBUF / 16; x += NT)
            *reinterpret_cast<v4i *>(lds + L::P + L::PBUF + 16 * x) = v4i{0, 0, 0, 0};
        if (tid < 32)
            reinterpret_cast<int *>(lds + L::ESC)[32 + tid] = 127;
    }
    lds_barrier();
    gather_load(0, 0 < nch, stage_a);
    gather_store(0, stage_a);
    gather_load(1, 1 < nch, stage_b);
    int raw = load_raw(3);
    gather_load(2, 2 < nch, stage_a);
    lds_barrier();
    if (nch > 0 && qk_wave) {
        s_cur = qk(0, &mloc_cur);
        if (u == 0)
            reinterpret_cast<float *>(lds + L::MX)[kt * 32 + hl] = mloc_cur;
    }
    gather_store(1, stage_b);
    if (wave == 0 && 3 < nch)
        build(3, raw);

    // ---- main loop: iteration c runs QK(c+1), softmax(c), P.V(c-1) --------------------------
    // On entry to iteration c: chunks c and c+1 are in their slots, chunk c+2 is in flight in
    // register stage `st` (loaded one iteration ago), tables are built up to chunk c+3, and P /
    // scales of chunk c-1 and the tile maxima of chunk c are in LDS.  The iteration loads chunk
    // c+3 into stage `ld`, stores chunk c+2 into slot (c+2) % 4 (which held chunk c-2, done) and
    // builds the table of chunk c+4.
    auto iteration = [&](int c, v4i(&st)[GI], v4i(&ld)[GI]) __attribute__((always_inline)) {
        lds_barrier();
        raw = load_raw(c + 4);  // every wave (fixed load count); wave 0 builds the table
        gather_load(c + 3, c + 3 < nch, ld);
        if (qk_wave) {
            float mloc_next;
            const v16f s_next = qk(c + 1, &mloc_next);  // stale slot when c+1 == nch: unused
            softmax(c, s_cur, mloc_cur);
            if (u == 0)
                reinterpret_cast<float *>(lds + L::MX)[((c + 1) & 1) * 64 + kt * 32 + hl] =
                    mloc_next;
            s_cur = s_next;
            mloc_cur = mloc_next;
        } else {
            pv(c - 1);
        }
        gather_store(c + 2, st);  // past the range: zero rows into a slot no chunk reads
        if (wave == 0 && c + 4 < nch)
            build(c + 4, raw);
    };
    for (int c = 0; c < nch; c += 2) {
        iteration(c, stage_a, stage_b);
        if (c + 1 < nch)
            iteration(c + 1, stage_b, stage_a);
    }
    // drain: P.V of the last chunk
    if (nch > 0) {
        lds_barrier();
        if (!qk_wave)
            pv(nch - 1);
    }
    };  // run_range

    int *flag = reinterpret_cast<int *>(lds + L::MISC) + 1;
    if (tid == 0)
        *flag = 0;
    run_range();
    // second pass for the heads whose offset overflowed (rare): restart the range with their
    // frames fixed at their final maxima
    lds_barrier();
    if (qk_wave && __any(overflow) && lane == 0)
        *flag = 1;
    lds_barrier();
    if (*flag != 0) {
        if (qk_wave) {
            preset = overflow;
            frame = preset ? m_run : -INFINITY;
            m_run = -INFINITY;
            ecur = 0;
            l_lane = 0.0f;
            overflow = false;
        } else {
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
                acc[ct] = v16f{};
        }
        lds_barrier();
        run_range();
    }

    // ---- epilogue ---------------------------------------------------------------------------
    float *fin = reinterpret_cast<float *>(lds + L::FIN);  // [l kt0][l kt1][G][e int] x 32
    lds_barrier();
    if (qk_wave) {
        const float lt = l_lane + __shfl_xor(l_lane, 32);
        if (u == 0)
            fin[kt * HG + hl] = lt;
        if (kt == 0 && u == 0) {
            fin[2 * HG + hl] = frame;
            reinterpret_cast<int *>(fin)[3 * HG + hl] = ecur;
        }
    }
    lds_barrier();

    // this lane's head: frame G and the sum l in frame G
    float g_h = fin[2 * HG + hl];
    float l_h = ldexpf(fin[hl] + fin[HG + hl], reinterpret_cast<const int *>(fin)[3 * HG + hl]);

    const int64_t tg = (int64_t)t * a.groups + hg;
    // register-order index of accumulator element r of tile `tile` (one 256-byte run per
    // register and tile: every store and load instruction of the exchange is one coalesced run)
    auto part_idx = [&](int tile, int r) { return (tile * 16 + r) * 64 + lane; };
    if (a.splits > 1) {
        // Partial of this range: FP32 accumulators in register order, then (G, l) per head.
        // The exchange uses device-scope (write-through) stores and loads, and each workgroup
        // waits for its stores to complete before taking its ticket: no cache writeback or
        // invalidation of the whole L2, which the workgroups of other tokens would pay for.
        const int64_t ui = tg * a.splits + split;
        float *po = a.ws_o + ui * (HG * 512);
        if (!qk_wave) {
#pragma unroll
            for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    store_device(po + part_idx(tile0 + ct, r), acc[ct][r]);
        }
        if (wave == 0 && u == 0) {
            store_device(a.ws_ml + (ui * HG + hl) * 2 + 0, g_h);
            store_device(a.ws_ml + (ui * HG + hl) * 2 + 1, l_h);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
        __syncthreads();
        int *ticket = reinterpret_cast<int *>(lds + L::MISC);
        if (tid == 0)
            *ticket = __hip_atomic_fetch_add(a.counters + tg, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        lds_barrier();
        if (*ticket != a.splits - 1)
            return;
        // last range: merge every range's partial in range order (its own included, read back
        // from the workspace, so the result does not depend on which range finishes last)
        float big_g = -INFINITY;
        for (int s = 0; s < a.splits; s++)
            big_g = fmaxf(big_g, load_device(a.ws_ml + ((tg * a.splits + s) * HG + hl) * 2));
        l_h = 0.0f;
#pragma unroll
        for (int ct = 0; ct < NCT; ct++)
            acc[ct] = v16f{};
        // every wave forms the merged sum (wave 0 writes the LSE), waves 2 and 3 the output
        for (int s = 0; s < a.splits; s++) {
            const int64_t us = tg * a.splits + s;
            const float *ps = a.ws_o + us * (HG * 512);
            const float gs = load_device(a.ws_ml + (us * HG + hl) * 2);
            const float ls = load_device(a.ws_ml + (us * HG + hl) * 2 + 1);
            const float w = gs == -INFINITY ? 0.0f : exp2f(gs - big_g);
            l_h += w * ls;
            if (!qk_wave) {
#pragma unroll
                for (int ct = 0; ct < NCT; ct++)
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        acc[ct][r] += w * load_device(ps + part_idx(tile0 + ct, r));
            }
        }
        g_h = big_g;
        if (tid == 0)  // every range has arrived: ready for the next call
            __hip_atomic_store(a.counters + tg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- final: sink, normalization, BF16 tile in LDS, coalesced row stores, LSE ---------
    uint8_t *tile = lds;  // [32][1024 bytes], over the KV region
    {
        const bool any = g_h != -INFINITY;
        float big_m = g_h, big_l = l_h, w = 1.0f;
        if (a.sinks != nullptr && head < a.H) {
            const float sk = a.sinks[head] * LOG2E;
            big_m = fmaxf(g_h, sk);
            w = any ? exp2f(g_h - big_m) : 0.0f;
            big_l = w * l_h + ANCHOR * exp2f(sk - big_m);
        }
        const float inv = any ? a.bmm2 * w / big_l : 0.0f;
        if (!qk_wave) {
#pragma unroll
            for (int ct = 0; ct < NCT; ct++) {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int col = 32 * (tile0 + ct) + 8 * i + 4 * u;
                    uint2 pk;
                    pk.x = bf16_bits(acc[ct][4 * i] * inv) |
                           (bf16_bits(acc[ct][4 * i + 1] * inv) << 16);
                    pk.y = bf16_bits(acc[ct][4 * i + 2] * inv) |
                           (bf16_bits(acc[ct][4 * i + 3] * inv) << 16);
                    *reinterpret_cast<uint2 *>(tile + hl * 1024 + 2 * col) = pk;
                }
            }
        }
        if (wave == 0 && u == 0 && head < a.H && a.lse != nullptr) {
            const float lse2 = any ? big_m - LOG2_ANCHOR + log2f(big_l) : -INFINITY;
            a.lse[(int64_t)t * a.H + head] = a.lse_log2 ? lse2 : lse2 * LN2;
        }
    }
    lds_barrier();
    const int heads_here = min(HG, a.H - hg * HG);
    for (int x = tid; x < heads_here * 64; x += NT) {
        const int row = x >> 6, part = x & 63;
        const v4i v = lds_load<v4i>(tile, row * 1024 + 16 * part);
        *reinterpret_cast<v4i *>(a.out + ((int64_t)t * a.H + hg * HG + row) * 512 + 8 * part) =
            v;
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
                         bool two_term, hipStream_t stream)
{
    if (tiles != 1)
        return hipErrorInvalidValue;
    return two_term ? launch_shape<true>(p, row_bytes, qk_dim, stream)
                    : launch_shape<false>(p, row_bytes, qk_dim, stream);
}

}  // namespace smla
