// LSE merge of S split-KV partials on gfx950 (dcp page, DcpValue.merge): per (token, head) the
// valid sources (finite base-2 LSE) are weighted by 2^(lse_s - top) / sum_r 2^(lse_r - top),
// their BF16 rows summed in FP32 and rounded to BF16 once; no valid source gives +0 and -inf.
//
// Pure HBM streaming.  One wave per (token, head) unit, eight units per workgroup.  Lane s holds
// source s's LSE (one vector load for all sources: the only access that precedes the partials'
// loads); the top and the sum of 2^(lse_s - top) are wave reductions (butterfly order), and
// lane s's weight reaches the other lanes by a shuffle.  Each lane then takes 16-byte runs of 8
// columns, issuing the loads of a block of up to 8 valid sources back to back before summing
// them in source order; one 16-byte store per run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_internal.h"

namespace smla {
namespace {

constexpr float LN2 = 0.6931471805599453f;
constexpr int MAX_SOURCES = 64;

__device__ inline uint32_t bf16_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// NaN and +-inf both mark an empty source.
__device__ inline bool valid_lse(float x) { return __builtin_isfinite(x); }

constexpr int WAVES = 8;   // units per workgroup
constexpr int SB = 8;      // sources loaded together

__device__ inline float wave_max(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ inline float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

__global__ void __launch_bounds__(64 * WAVES) lse_merge_kernel(LseMergeParams p)
{
    const int lane = threadIdx.x & 63;
    const int64_t unit = (int64_t)blockIdx.x * WAVES +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t TH = (int64_t)p.T * p.H;
    if (unit >= TH)
        return;
    const int per_unit = p.D / 8;
    // the unit's weights: lane s < S holds source s's LSE; top over the valid sources, then
    // 2^(lse_s - top) / sum (the same values on every lane after the reductions)
    const float l = lane < p.S ? p.lse2[lane * TH + unit] : -INFINITY;
    const bool valid = valid_lse(l);
    const float top = wave_max(valid ? l : -INFINITY);
    if (top == -INFINITY) {  // no valid source: +0 and -inf
        for (int k = lane; k < per_unit; k += 64)
            reinterpret_cast<uint4 *>(p.out)[unit * per_unit + k] = make_uint4(0, 0, 0, 0);
        if (lane == 0 && p.lse_out != nullptr)
            p.lse_out[unit] = -INFINITY;
        return;
    }
    const float e = valid ? exp2f(l - top) : 0.0f;
    const float sum = wave_sum(e);
    const float w_lane = e * (1.0f / sum);
    const uint4 *src = reinterpret_cast<const uint4 *>(p.partials) + unit * per_unit;
    // the loop is wave-uniform (every lane runs each step, `on` guards the memory accesses), so
    // that every lane is active at the shuffles that broadcast the weights
    for (int k0 = 0; k0 < per_unit; k0 += 64) {
        const int k = k0 + lane;
        const bool on = k < per_unit;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int s0 = 0; s0 < p.S; s0 += SB) {
            uint4 x[SB];
            float wgt[SB];
#pragma unroll
            for (int j = 0; j < SB; j++) {
                const int s = s0 + j;
                wgt[j] = __shfl(w_lane, s < p.S ? s : 0);
                wgt[j] = s < p.S ? wgt[j] : 0.0f;
                x[j] = make_uint4(0, 0, 0, 0);
                if (on && wgt[j] != 0.0f)  // an empty source is never read
                    x[j] = src[s * TH * per_unit + k];
            }
#pragma unroll
            for (int j = 0; j < SB; j++) {
                acc[0] += wgt[j] * bf16_lo(x[j].x);
                acc[1] += wgt[j] * bf16_hi(x[j].x);
                acc[2] += wgt[j] * bf16_lo(x[j].y);
                acc[3] += wgt[j] * bf16_hi(x[j].y);
                acc[4] += wgt[j] * bf16_lo(x[j].z);
                acc[5] += wgt[j] * bf16_hi(x[j].z);
                acc[6] += wgt[j] * bf16_lo(x[j].w);
                acc[7] += wgt[j] * bf16_hi(x[j].w);
            }
        }
        uint4 res;
        res.x = bf16_bits(acc[0]) | (bf16_bits(acc[1]) << 16);
        res.y = bf16_bits(acc[2]) | (bf16_bits(acc[3]) << 16);
        res.z = bf16_bits(acc[4]) | (bf16_bits(acc[5]) << 16);
        res.w = bf16_bits(acc[6]) | (bf16_bits(acc[7]) << 16);
        if (on)
            reinterpret_cast<uint4 *>(p.out)[unit * per_unit + k] = res;
    }
    if (lane == 0 && p.lse_out != nullptr) {
        const float lse2 = top + log2f(sum);
        p.lse_out[unit] = p.lse_log2 ? lse2 : lse2 * LN2;
    }
}

}  // namespace

hipError_t launch_lse_merge(const LseMergeParams &p, hipStream_t stream)
{
    if (p.S > MAX_SOURCES)
        return hipErrorInvalidValue;
    const int64_t units = (int64_t)p.T * p.H;
    const int64_t blocks = (units + WAVES - 1) / WAVES;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(lse_merge_kernel, dim3((unsigned)blocks), dim3(64 * WAVES), 0, stream, p);
    return hipGetLastError();
}

}  // namespace smla
