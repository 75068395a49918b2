// Sparse MLA decode for gfx950 (MI355X): index-driven row gather into LDS, QK^T on FP8 MFMA,
// online softmax with P quantized to E4M3 at 448 of the running maximum, P.V on FP8 MFMA with
// V read transposed from the same LDS tile, and the FP32 merge of split partials.
//
// Method (vLLM API pages): the formula is the sparse_mla_cute page's "What this module
// computes"; the E4M3-P recipe, the contiguous key split and the split merge are the
// attn_sparse page's module docstring and its SparseDcpDecode.kernel / merge methods.
//
// Work decomposition: a workgroup takes one token t, TILES 16-head tiles (one wave each) and
// one key range of the token.  The range is processed in chunks of 128 columns.  A chunk's rows
// are gathered once into LDS with 16-byte direct-to-LDS loads (global_load_lds_dwordx4) and
// feed every wave, so KV bytes are read once per (token, range) whatever the head count.
// Masked columns (negative index, or past the range) load a zero row instead, so their V bytes
// are zero and their scores are forced to -inf.  Two chunk buffers alternate: the gather of
// chunk c+1 is in flight while chunk c is computed.
//
// LDS layout of a chunk buffer: row-major, 128 rows x row_bytes, the 16-byte pieces of row r
// stored in XOR-permuted order (piece p at position p ^ a(r)).  A gather instruction fills 64
// consecutive 16-byte positions, i.e. about two whole rows, so its global reads coalesce into
// whole cache lines; the permutation puts the 16 rows of a QK operand tile and the 8 rows of a
// transposed V read on distinct LDS banks (a(r) = ((r >> 2) ^ ((r >> 4) << 1)) & 3 for
// 576-byte rows, conflict-free; r & 7 for 512-byte rows, at most 2-way).
//
// Per wave and chunk (16 heads x 128 keys):
//   S^T = K Q^T on v_mfma_scale_f32_16x16x128_f8f6f4 (scales 2^0): A = 16 key rows from LDS,
//     B = the wave's Q fragments, kept in VGPRs for the whole kernel.  Lane (h, g) of the
//     accumulator of tile u holds keys 16u + 4g + [0, 4) of head h, so the softmax of head h
//     lives in the 4 lanes h + 16g.  Steps run block-major (consecutive MFMAs feed different
//     tiles) with the next A operand read while the current MFMA runs.
//   softmax: masked scores -> -inf, chunk max (in-lane, then 2 cross-lane steps), running max,
//     alpha = 2^(m_old - m_new), P = 2^(s2 - m_new + log2 448) rounded to E4M3 by
//     v_cvt_pk_fp8_f32 (RNE; P <= 448 by construction, where the conversion is exact RNE),
//     FP32 sums of the unquantized P, accumulators rescaled by alpha.
//   O^T += V^T P^T on the same MFMA: B = P straight from the softmax registers (no LDS round
//     trip: P register u of lane group g holds keys 16u + 4g + [0, 4), and the V^T operand is
//     read with ds_read_b64_tr_b8 from exactly those rows: an 8 x 16 byte block of rows
//     {32j + 4g + [0,4), 32j + 16 + 4g + [0,4)} returned column-wise, 8 keys of one latent
//     column per lane), the V^T operand of tile v+D read while tile v's MFMAs run.
//   Two-term P (default): P = hi + lo/16 with hi = E4M3(P), lo = E4M3(16 (P - hi)); the second
//     product uses the MFMA's E8M0 B scale 2^-4, so it costs one more MFMA per tile and no
//     conversion of V.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

#define SMLA_LDS(T) __attribute__((address_space(3))) T

constexpr int CHUNK = 128;                         // columns per gathered chunk
constexpr float ANCHOR = 448.0f;                   // P anchor: E4M3's largest finite value
constexpr float LOG2_ANCHOR = 8.807354922057604f;  // log2(448)
constexpr float LN2 = 0.6931471805599453f;
constexpr float LOG2E = 1.4426950408889634f;
constexpr int E8M0_ONE = 127;                      // MFMA block scale 2^0
constexpr int E8M0_SIXTEENTH = 123;                // 2^-4, for the second P term

// Masked columns gather this row, so their V bytes are zero (0 * anything stays finite).
__device__ __attribute__((aligned(16))) uint8_t g_zero_row[576];

template <int RB>
struct Geom {
    static constexpr int PIECES = RB / 16;   // 16-byte pieces of a row
    static constexpr int BUF = CHUNK * RB;   // one chunk buffer
    // XOR applied to the piece index of row r (keeps the 128-byte K block of a piece)
    __device__ static constexpr int perm(int r)
    {
        return RB == 576 ? (((r >> 2) ^ ((r >> 4) << 1)) & 3) : (r & 7);
    }
};

__device__ inline v8i join(v4i x, v4i y)
{
    return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

__device__ inline v4i lds16(const uint8_t *base, int off)
{
    return *reinterpret_cast<const v4i *>(base + off);
}

__device__ inline v8i global_read32(const uint8_t *p)
{
    const v4i *v = reinterpret_cast<const v4i *>(p);
    return join(v[0], v[1]);
}

__device__ inline v4f mfma_fp8(v8i a, v8i b, v4f c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, E8M0_ONE, 0,
                                                            E8M0_ONE);
}

__device__ inline v4f mfma_fp8_b_sixteenth(v8i a, v8i b, v4f c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, E8M0_ONE, 0,
                                                            E8M0_SIXTEENTH);
}

// One 16-byte direct-to-LDS load per lane: lane l's 16 bytes land at LDS byte address
// lds_base + 16 l (lds_base wave-uniform, in M0).  Issued as inline asm so that the compiler
// does not tie later LDS reads of the other chunk buffer to this load's completion; the
// kernel waits for it explicitly (s_waitcnt vmcnt(0) + barrier) before reading the buffer.
// M0 is saved and restored around the load.
__device__ inline void dma16(const uint8_t *src, uint32_t lds_base)
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

__device__ inline void wait_all_vm()
{
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

__device__ inline uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const SMLA_LDS(uint8_t) *)p;
}

// BF16 of a finite float, round to nearest even.
__device__ inline uint32_t bf16_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

template <int TILES, int RB, int QK, bool TWO>
__global__ void __launch_bounds__(64 * TILES, 2) decode_kernel(DecodeParams a)
{
    constexpr int NT = 64 * TILES;
    using G = Geom<RB>;
    constexpr int QB = QK / 128;                 // full 128-byte K blocks of the score
    constexpr bool TAIL = (QK % 128) != 0;       // qk_dim 576: a last block of 64 bytes
    constexpr int NQ = QB + (TAIL ? 1 : 0);
    constexpr int IDX_PER_THREAD = (CHUNK + NT - 1) / NT;
    constexpr int GATHER_ITERS = CHUNK * G::PIECES / NT;  // exact for every tile count
    static_assert(CHUNK * G::PIECES % NT == 0, "gather slots must tile the waves");

    __shared__ __attribute__((aligned(16))) uint8_t kvbuf[2][G::BUF];
    // masked indices and gather source rows of three chunks in flight; slot CHUNK is a sink
    // for threads without a column (no branches around the stores)
    __shared__ __attribute__((aligned(16))) int32_t cidx[3][CHUNK + 4];
    __shared__ const uint8_t *rowsrc[3][CHUNK + 1];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int h16 = lane & 15, g = lane >> 4;

    int blk = blockIdx.x;
    const int split = blk % a.splits;
    blk /= a.splits;
    const int grp = blk % a.groups;
    const int t = blk / a.groups;
    const int head = (grp * TILES + wave) * 16 + h16;

    int n = a.lens[t];
    n = n < 0 ? 0 : (n > a.W ? a.W : n);
    const int per = (n + a.splits - 1) / a.splits;
    const int first = min(n, split * per);
    const int mine = min(n - first, per);
    const int end = first + mine;
    const int nchunks = (mine + CHUNK - 1) / CHUNK;
    const int32_t *idx_row = a.indices + (int64_t)t * a.W;
    const uint8_t *zero_row = g_zero_row;

    // Q fragments, B operand of S^T = K Q^T: lane (h16, g) holds bytes 128 b + 32 g + [0, 32).
    v8i qf[NQ];
    {
        const uint8_t *qp = a.q + (int64_t)t * a.q_st + (int64_t)head * a.q_sh;
#pragma unroll
        for (int b = 0; b < QB; b++)
            qf[b] = global_read32(qp + 128 * b + 32 * g);
        if constexpr (TAIL) {
            // bytes 512 + 32 g for g < 2; zero for g >= 2
            const v8i x = global_read32(qp + 512 + 32 * (g & 1));
            qf[QB] = g < 2 ? x : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }

    // The masked index and the gather source row of position pos (only positions < end, which
    // is at most the clamped count <= W, are ever read from the index row).
    auto source_of = [&](int pos, int raw, int32_t *ci, const uint8_t **rs) {
        const int v = (pos < end && raw >= 0) ? raw : -1;
        const uint8_t *pool = (a.kv_b != nullptr && pos >= a.split_col) ? a.kv_b : a.kv_a;
        *ci = v;
        *rs = v >= 0 ? pool + (int64_t)v * RB : zero_row;
    };

    // The gather of chunk c into buffer `buf`: 128 * PIECES 16-byte positions, 64 consecutive
    // ones per wave instruction; position s holds piece (s % PIECES) ^ perm(row) of row
    // s / PIECES.
    auto gather = [&](int c, int buf) {
        const uint8_t *const *rs = rowsrc[c % 3];
        const uint32_t dst = lds_addr(kvbuf[buf]);
#pragma unroll 1
        for (int it = 0; it < GATHER_ITERS; it++) {
            const int s0 = it * NT + wave * 64;
            const int s = s0 + lane;
            const int r = s / G::PIECES;
            const int p = (s - r * G::PIECES) ^ G::perm(r);
            dma16(rs[r] + 16 * p, __builtin_amdgcn_readfirstlane(dst + (uint32_t)s0 * 16u));
        }
    };

    // prologue: indices and sources of chunks 0 and 1, then the gather of chunk 0
#pragma unroll
    for (int c = 0; c < 2; c++) {
        if (c < nchunks) {
            for (int i = tid; i < CHUNK; i += NT) {
                const int pos = first + c * CHUNK + i;
                source_of(pos, pos < end ? idx_row[pos] : -1, &cidx[c][i], &rowsrc[c][i]);
            }
        }
    }
    __syncthreads();
    if (nchunks > 0)
        gather(0, 0);

    float m_run = -INFINITY;  // running max of head h16 (base 2), equal in the 4 lanes h16 + 16g
    float l_run = 0.0f;       // this lane's share of the running sum of unquantized P
    v4f acc[32];              // O^T tiles: acc[v][r] = O[head h16][16 v + 4 g + r]
#pragma unroll
    for (int v = 0; v < 32; v++)
        acc[v] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // Lane constants of the operand reads.  QK: the A row of tile u is 16u + h16; its first
    // piece of block b is (8b + 2g) ^ perm, the second that ^ 1 (byte offset ^ 16).  perm of
    // row 16u + h16 depends on u only through u & 1 for 576-byte rows, not at all for
    // 512-byte rows.  PV: this lane provides half (h16 & 1) of row kv_row(j) = 32j + r0,
    // r0 = 16 (rr >> 2) + 4g + (rr & 3), rr = h16 >> 1, of the 8-row transposed block j; perm
    // of that row does not depend on j.
    // [e][k]: piece k of the pair; the per-step parts (16u RB + 128b) have bit 4 clear, so
    // they add as immediate offsets
    int qk_off[2][2], qk_tail[2][2];
#pragma unroll
    for (int e = 0; e < 2; e++) {
        const int r = 16 * e + h16;  // the A row of tile e; tiles u with u & 1 == e share perm
        qk_off[e][0] = h16 * RB + 16 * ((2 * g) ^ G::perm(r));
        qk_off[e][1] = qk_off[e][0] ^ 16;
        qk_tail[e][0] = h16 * RB + 16 * ((32 + 2 * (g & 1)) ^ G::perm(r));
        qk_tail[e][1] = qk_tail[e][0] ^ 16;
    }
    constexpr int VX = RB == 576 ? 4 : 8;  // pieces spanned by perm
    int v_off[VX];
    {
        const int rr = h16 >> 1;
        const int r0 = 16 * (rr >> 2) + 4 * g + (rr & 3);
#pragma unroll
        for (int x = 0; x < VX; x++)
            v_off[x] = r0 * RB + 16 * (x ^ G::perm(r0)) + 8 * (h16 & 1);
    }

#pragma unroll 1
    for (int c = 0; c < nchunks; c++) {
        const int buf = c & 1;
        // chunk c has landed (each wave waits for its own loads; the barrier publishes them),
        // every wave is done with chunk c-1, and the sources of chunk c+1 are visible
        wait_all_vm();
        __syncthreads();
        // raw indices of chunk c+2, consumed only after this chunk's compute; branch-free: the
        // load address is clamped into the token's row and the value dropped past the range
        int pre[IDX_PER_THREAD];
        int pre_pos[IDX_PER_THREAD];
#pragma unroll
        for (int k = 0; k < IDX_PER_THREAD; k++) {
            pre_pos[k] = first + (c + 2) * CHUNK + tid + k * NT;
            pre[k] = idx_row[min(pre_pos[k], a.W - 1)];
        }
        if (c + 1 < nchunks)
            gather(c + 1, buf ^ 1);

        const uint8_t *kv = kvbuf[buf];
        const int32_t *ci = cidx[c % 3];

        // ---- S^T = K Q^T: 8 tiles of 16 keys ------------------------------------------------
        // Block-major order: consecutive MFMAs feed different tiles, and the A operand of step
        // i+1 is read from LDS while the MFMA of step i runs.  Lane groups 2 and 3 read the
        // tail block's bytes of groups 0 and 1 and multiply them by the zero half of their Q
        // fragment.
        v4f S[8];
#pragma unroll
        for (int u = 0; u < 8; u++)
            S[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        {
            auto a_read = [&](int i) {
                const int b = i >> 3, u = i & 7;
                const int e = u & 1;
                const int imm = (b < QB ? 128 * b : 0) + 16 * u * RB;
                const int *o = b < QB ? qk_off[e] : qk_tail[e];
                return join(lds16(kv + o[0], imm), lds16(kv + o[1], imm));
            };
            constexpr int STEPS = NQ * 8;
            v8i a_cur = a_read(0);
#pragma unroll
            for (int i = 0; i < STEPS; i++) {
                v8i a_next = a_cur;
                if (i + 1 < STEPS)
                    a_next = a_read(i + 1);
                S[i & 7] = mfma_fp8(a_cur, qf[i >> 3], S[i & 7]);
                a_cur = a_next;
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < STEPS - 1; i++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }

        // ---- mask, scale to base 2, chunk max ----------------------------------------------
        float sc[8][4];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const v4i live = *reinterpret_cast<const v4i *>(ci + 16 * u + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; r++) {
                sc[u][r] = live[r] >= 0 ? S[u][r] * a.scale_log2 : -INFINITY;
                mx = fmaxf(mx, sc[u][r]);
            }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        // no active column yet: every score is -inf and so is every P argument (finite bias)
        const float bias = m_new == -INFINITY ? 0.0f : m_new - LOG2_ANCHOR;

        // ---- P = 2^(s2 - m_new + log2 448) as E4M3, FP32 sums of the unquantized P ---------
        int pb[8];
        int pr[8];
        float lsum = 0.0f;
#pragma unroll
        for (int u = 0; u < 8; u++) {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
                p[r] = __builtin_amdgcn_exp2f(sc[u][r] - bias);  // exp2(-inf) = 0
                lsum += p[r];
            }
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
            pb[u] = w;
            if constexpr (TWO) {
                const float h0 = __builtin_amdgcn_cvt_f32_fp8(w, 0);
                const float h1 = __builtin_amdgcn_cvt_f32_fp8(w, 1);
                const float h2 = __builtin_amdgcn_cvt_f32_fp8(w, 2);
                const float h3 = __builtin_amdgcn_cvt_f32_fp8(w, 3);
                int x = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[0] - h0), 16.0f * (p[1] - h1), 0,
                                                        false);
                x = __builtin_amdgcn_cvt_pk_fp8_f32(16.0f * (p[2] - h2), 16.0f * (p[3] - h3), x,
                                                    true);
                pr[u] = x;
            } else {
                pr[u] = 0;
            }
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        // (unconditional: with 16 heads per wave some head's maximum rises in most chunks, and a
        // branch here would let the compiler sink the P math and the PV products past every V
        // read of the chunk)
#pragma unroll
        for (int v = 0; v < 32; v++)
            acc[v] *= alpha;

        // ---- O^T += V^T P^T ----------------------------------------------------------------
        // 32 column tiles (tile v = latent columns 16v .. 16v+15 = piece v of each row); the V^T
        // operand of tile v+D is read while the MFMAs of tile v run (D = 1 at 8 waves per
        // workgroup, where the second wave of each SIMD also hides LDS latency, else 2).
        asm volatile("" ::: "memory");
        {
            constexpr int D = TILES == 8 ? 1 : 2;
            const v8i bp = v8i{pb[0], pb[1], pb[2], pb[3], pb[4], pb[5], pb[6], pb[7]};
            const v8i br = v8i{pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]};
            auto v_read = [&](int v) {
                v8i av;
                const int vb = 16 * (v & ~(VX - 1));
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint8_t *vp = kv + v_off[v & (VX - 1)] + vb + 32 * j * RB;
                    const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SMLA_LDS(v2i) *)vp);
                    av[2 * j] = x[0];
                    av[2 * j + 1] = x[1];
                }
                return av;
            };
            v8i ab[D + 1];
#pragma unroll
            for (int k = 0; k < D; k++)
                ab[k] = v_read(k);
#pragma unroll
            for (int v = 0; v < 32; v++) {
                if (v + D < 32)
                    ab[(v + D) % (D + 1)] = v_read(v + D);
                const v8i a0 = ab[v % (D + 1)];
                acc[v] = mfma_fp8(a0, bp, acc[v]);
                if constexpr (TWO)
                    acc[v] = mfma_fp8_b_sixteenth(a0, br, acc[v]);
            }
            constexpr int PV_MFMA = TWO ? 2 : 1;
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * D, 1);
#pragma unroll
            for (int v = 0; v < 32 - D; v++) {
                __builtin_amdgcn_sched_group_barrier(0x008, PV_MFMA, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, D * PV_MFMA, 1);
        }

        // slot (c+2) % 3 held chunk c-1, which every wave finished before this iteration's
        // barrier; when c+2 >= nchunks the values are never read
#pragma unroll
        for (int k = 0; k < IDX_PER_THREAD; k++) {
            const int i = min(tid + k * NT, CHUNK);
            source_of(pre_pos[k], pre[k], &cidx[(c + 2) % 3][i], &rowsrc[(c + 2) % 3][i]);
        }
    }

    // ---- epilogue: the full sum of head h16 over its 4 lanes --------------------------------
    float ltot = l_run + __shfl_xor(l_run, 16);
    ltot += __shfl_xor(ltot, 32);
    const int64_t th = (int64_t)t * a.H + head;

    if (a.splits > 1) {
        float *po = a.ws_o + (th * a.splits + split) * 512 + 4 * g;
#pragma unroll
        for (int v = 0; v < 32; v++)
            *reinterpret_cast<v4f *>(po + 16 * v) = acc[v];
        if (g == 0) {
            a.ws_ml[(th * a.splits + split) * 2 + 0] = m_run;
            a.ws_ml[(th * a.splits + split) * 2 + 1] = ltot;
        }
        return;
    }

    // one range: merge with the sink (if any) and write BF16 out and the LSE
    const bool any = m_run != -INFINITY;
    float big_m = m_run;
    float big_l = ltot;
    float w = 1.0f;
    if (a.sinks != nullptr) {
        const float sk = a.sinks[head] * LOG2E;
        big_m = fmaxf(m_run, sk);
        w = any ? exp2f(m_run - big_m) : 0.0f;
        big_l = w * ltot + ANCHOR * exp2f(sk - big_m);
    }
    const float inv = any ? a.bmm2 * w / big_l : 0.0f;
    uint16_t *op = a.out + th * 512 + 4 * g;
#pragma unroll
    for (int v = 0; v < 32; v++) {
        const v4f x = acc[v] * inv;
        uint2 pk;
        pk.x = bf16_bits(x[0]) | (bf16_bits(x[1]) << 16);
        pk.y = bf16_bits(x[2]) | (bf16_bits(x[3]) << 16);
        *reinterpret_cast<uint2 *>(op + 16 * v) = pk;
    }
    if (a.lse != nullptr && g == 0) {
        float lse2 = any ? big_m - LOG2_ANCHOR + log2f(big_l) : -INFINITY;
        a.lse[th] = a.lse_log2 ? lse2 : lse2 * LN2;
    }
}

// Merge of the split partials of one (token, head): 128 threads, 4 columns each; two units
// per 256-thread workgroup.  Weights 2^(m_s - M) (0 for an empty range), the sink as
// 448 * 2^(sink2 - M), out = BF16(bmm2 * sum w_s O_s / L), LSE2 = M - log2 448 + log2 L.
__global__ void __launch_bounds__(256) split_merge_kernel(DecodeParams a)
{
    const int unit = blockIdx.x * 2 + (threadIdx.x >> 7);
    const int i = threadIdx.x & 127;
    if (unit >= a.T * a.H)
        return;
    const int head = unit % a.H;
    const float *ml = a.ws_ml + (int64_t)unit * a.splits * 2;
    float big_m = -INFINITY;
    for (int s = 0; s < a.splits; s++)
        big_m = fmaxf(big_m, ml[2 * s]);
    const bool any = big_m != -INFINITY;
    float sk = 0.0f;
    if (a.sinks != nullptr) {
        sk = a.sinks[head] * LOG2E;
        big_m = fmaxf(big_m, sk);
    }
    float big_l = 0.0f;
    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    const float *po = a.ws_o + (int64_t)unit * a.splits * 512 + 4 * i;
    for (int s = 0; s < a.splits; s++) {
        const float ms = ml[2 * s];
        if (ms == -INFINITY)
            continue;
        const float w = exp2f(ms - big_m);
        big_l += w * ml[2 * s + 1];
        acc += w * *reinterpret_cast<const v4f *>(po + (int64_t)s * 512);
    }
    if (a.sinks != nullptr)
        big_l += ANCHOR * exp2f(sk - big_m);
    const float inv = any ? a.bmm2 / big_l : 0.0f;
    const v4f x = acc * inv;
    uint2 pk;
    pk.x = bf16_bits(x[0]) | (bf16_bits(x[1]) << 16);
    pk.y = bf16_bits(x[2]) | (bf16_bits(x[3]) << 16);
    *reinterpret_cast<uint2 *>(a.out + (int64_t)unit * 512 + 4 * i) = pk;
    if (a.lse != nullptr && i == 0) {
        const float lse2 = any ? big_m - LOG2_ANCHOR + log2f(big_l) : -INFINITY;
        a.lse[unit] = a.lse_log2 ? lse2 : lse2 * LN2;
    }
}

template <int TILES, int RB, int QK, bool TWO>
hipError_t launch_one(const DecodeParams &p, hipStream_t stream)
{
    const unsigned blocks = (unsigned)p.T * (unsigned)p.groups * (unsigned)p.splits;
    hipLaunchKernelGGL((decode_kernel<TILES, RB, QK, TWO>), dim3(blocks), dim3(64 * TILES), 0,
                       stream, p);
    return hipGetLastError();
}

template <int RB, int QK, bool TWO>
hipError_t launch_tiles(const DecodeParams &p, int tiles, hipStream_t stream)
{
    switch (tiles) {
    case 1: return launch_one<1, RB, QK, TWO>(p, stream);
    case 2: return launch_one<2, RB, QK, TWO>(p, stream);
    case 4: return launch_one<4, RB, QK, TWO>(p, stream);
    case 8: return launch_one<8, RB, QK, TWO>(p, stream);
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
    hipError_t e = two_term ? launch_shape<true>(p, tiles, row_bytes, qk_dim, stream)
                            : launch_shape<false>(p, tiles, row_bytes, qk_dim, stream);
    if (e != hipSuccess || p.splits == 1)
        return e;
    const unsigned units = (unsigned)p.T * (unsigned)p.H;
    hipLaunchKernelGGL(split_merge_kernel, dim3((units + 1) / 2), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace smla
