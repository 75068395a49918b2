// mla_value: the MLA value tail after the split merge, for gfx950 (MI355X).
//
// Method (the dcp page, DcpValue class docstring and its merge method): per token row t and
// head h, the S sources' BF16 partials are weighted by exp2(lse_s - top) / sum over the sources
// with a finite LSE (empty ones weigh 0 and are never read), summed in FP32 and rounded once to
// BF16 (the merged latent row); W_UV, BF16 inputs with FP32 accumulation, maps the 512 latent
// values to the head's 128 outputs; the product is rounded to BF16, multiplied by the sigmoid
// of the gate, and rounded to BF16 again.  Rows whose request total is 0 (padded rows, whose
// gate may be NaN) are written as zeros.
//
// Decomposition: one workgroup of 8 waves takes one head and 16 rows.
//   1. Every wave issues its W_UV fragments first (they depend on nothing): the B operands of
//      v_mfma_f32_16x16x32_bf16 for its 16-value tile over the 16 k-steps of 32, each a 16-byte
//      run of latent-contiguous weights, so the loads are in flight during the merge.
//   2. The rows' source weights go to LDS, then the merge: each thread takes two 16-byte runs
//      (8 latent values) of the tile, issues the loads of up to 8 sources of both before
//      summing any (empty sources are not loaded), sums in FP32 in source order and writes the
//      BF16 runs to the LDS latent tile.
//   3. Products: latent (LDS, A operand) x W_UV (registers, B operand), FP32 accumulators.
//   4. BF16 rounding, gate, BF16 rounding, stores.
// Bound: HBM (the partials and W_UV are read once per workgroup; W_UV per head is 128 KB and
// is shared through L2 by the row tiles of a head).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int RT = 16;           // rows per workgroup
constexpr int NT = 512;          // threads per workgroup (8 waves)
constexpr int SB = 8;            // sources loaded together in the merge
constexpr int D = 512;           // latent width
constexpr int DV = 128;          // values per head
constexpr int MAXS = 64;         // most sources
constexpr int ROWB = D * 2 + 16; // LDS row pitch of the latent tile (padded: the 16 rows of an
                                 // A-fragment read fall in 16 different bank groups)

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two floats rounded to BF16 (nearest even), `lo` in the low half
__device__ inline uint32_t bf16x2(float lo, float hi)
{
    const v2bf r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ inline float bf16_round(float x) { return bf16_lo(bf16x2(x, 0.0f)); }

__global__ void __launch_bounds__(NT) mla_value_kernel(ValueParams a)
{
    __shared__ __attribute__((aligned(16))) uint8_t lat[RT * ROWB];
    __shared__ float wts[RT][MAXS];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.x, r0 = blockIdx.y * RT;
    const int64_t TH = (int64_t)a.T * a.H;

    // ---- 1. W_UV fragments of this wave's value tile (v = 16 wave + lane % 16), k = 32 step +
    // 8 (lane / 16) .. + 7: B operand of the 16x16x32 instruction
    v4i wf[16];
    {
        const int v = 16 * wave + (lane & 15), kq = lane >> 4;
        const uint16_t *wp = a.w_uv + h * a.w_sh + (int64_t)v * a.w_sv + 8 * kq;
#pragma unroll
        for (int s = 0; s < 16; s++)
            wf[s] = *reinterpret_cast<const v4i *>(wp + 32 * s);
    }

    // the gate values and live flags of this lane's four outputs (rows r0 + 4 (lane / 16) + j,
    // value 16 wave + lane % 16) go out now too: they depend on nothing
    float gate[4];
    bool out_live[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int t = r0 + 4 * (lane >> 4) + j;
        gate[j] = 0.0f;
        out_live[j] = false;
        if (t < a.T) {
            out_live[j] = a.totals == nullptr || a.totals[t / a.rows_per_request] > 0;
            gate[j] = bf16_lo(a.gate[(int64_t)t * a.H * DV + h * DV + 16 * wave + (lane & 15)]);
        }
    }

    // ---- 2. source weights of each row (the LSEs of all rows and sources loaded at once, then
    // one thread per row), then the merged BF16 latent tile
    for (int i = tid; i < RT * a.S; i += NT) {
        const int row = i / a.S, src = i - row * a.S, t = r0 + row;
        wts[row][src] = t < a.T ? a.lse2[src * TH + (int64_t)t * a.H + h] : -INFINITY;
    }
    __syncthreads();
    if (tid < RT) {
        float top = -INFINITY;
        for (int s = 0; s < a.S; s++) {
            const float v = wts[tid][s];
            if (isfinite(v))
                top = fmaxf(top, v);
        }
        float total = 0.0f;
        for (int s = 0; s < a.S; s++) {
            const float v = wts[tid][s];
            const float wgt = top != -INFINITY && isfinite(v) ? exp2f(v - top) : 0.0f;
            wts[tid][s] = wgt;
            total += wgt;
        }
        const float inv = total > 0.0f ? 1.0f / total : 0.0f;
        for (int s = 0; s < a.S; s++)
            wts[tid][s] *= inv;
    }
    __syncthreads();
    {
        // runs x0 = tid and x1 = tid + NT of the tile's RT * 64 16-byte runs
        int row[2], c8[2];
        bool live[2];
        const uint16_t *src[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int x = tid + j * NT;
            row[j] = x >> 6;
            c8[j] = x & 63;
            live[j] = r0 + row[j] < a.T;
            src[j] = a.partials + ((int64_t)(r0 + row[j]) * a.H + h) * D + 8 * c8[j];
        }
        float acc[2][8];
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 8; e++)
                acc[j][e] = 0.0f;
        for (int s0 = 0; s0 < a.S; s0 += SB) {
            uint4 u[2][SB];
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int k = 0; k < SB; k++) {
                    const int s = s0 + k;
                    u[j][k] = make_uint4(0u, 0u, 0u, 0u);
                    // an empty source (weight 0) is never read
                    if (s < a.S && live[j] && wts[row[j]][s] != 0.0f)
                        u[j][k] = *reinterpret_cast<const uint4 *>(src[j] + s * TH * D);
                }
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int k = 0; k < SB; k++) {
                    const int s = s0 + k;
                    const float wgt = s < a.S ? wts[row[j]][s] : 0.0f;
                    acc[j][0] += wgt * bf16_lo(u[j][k].x);
                    acc[j][1] += wgt * bf16_hi(u[j][k].x);
                    acc[j][2] += wgt * bf16_lo(u[j][k].y);
                    acc[j][3] += wgt * bf16_hi(u[j][k].y);
                    acc[j][4] += wgt * bf16_lo(u[j][k].z);
                    acc[j][5] += wgt * bf16_hi(u[j][k].z);
                    acc[j][6] += wgt * bf16_lo(u[j][k].w);
                    acc[j][7] += wgt * bf16_hi(u[j][k].w);
                }
        }
#pragma unroll
        for (int j = 0; j < 2; j++) {
            uint4 r;
            r.x = bf16x2(acc[j][0], acc[j][1]);
            r.y = bf16x2(acc[j][2], acc[j][3]);
            r.z = bf16x2(acc[j][4], acc[j][5]);
            r.w = bf16x2(acc[j][6], acc[j][7]);
            *reinterpret_cast<uint4 *>(lat + row[j] * ROWB + 16 * c8[j]) = r;
        }
    }
    __syncthreads();

    // ---- 3. C[16 rows x 16 values] += latent[16 x 32] W_UV[32 x 16] over the 16 k-steps
    v4f c = v4f{0.f, 0.f, 0.f, 0.f};
    {
        const int m = lane & 15, kq = lane >> 4;
#pragma unroll
        for (int s = 0; s < 16; s++) {
            const v4i af = *reinterpret_cast<const v4i *>(lat + m * ROWB + 2 * (32 * s + 8 * kq));
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, af),
                                                        __builtin_bit_cast(v8bf, wf[s]), c, 0, 0, 0);
        }
    }

    // ---- 4. lane holds value v = 16 wave + lane % 16 of rows 4 (lane / 16) + j
    // (padding between the last products and the first read of their results)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
    {
        const int v = 16 * wave + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int t = r0 + 4 * (lane >> 4) + j;
            if (t >= a.T)
                continue;
            float y = 0.0f;
            if (out_live[j]) {
                const float sig = 1.0f / (1.0f + expf(-gate[j]));
                y = bf16_round(c[j]) * sig;
            }
            a.out[(int64_t)t * a.H * DV + h * DV + v] = (uint16_t)(bf16x2(y, 0.0f) & 0xFFFFu);
        }
    }
}

}  // namespace

hipError_t launch_mla_value(const ValueParams &p, hipStream_t stream)
{
    const dim3 grid((unsigned)p.H, (unsigned)((p.T + RT - 1) / RT));
    hipLaunchKernelGGL(mla_value_kernel, grid, dim3(NT), 0, stream, p);
    return hipGetLastError();
}

}  // namespace smla
