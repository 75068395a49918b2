// LSE merge of S split-KV partials on gfx950 (dcp page, DcpValue.merge): per (token, head) the
// valid sources (finite base-2 LSE) are weighted by 2^(lse_s - top) / sum_r 2^(lse_r - top),
// their BF16 rows summed in FP32 and rounded to BF16 once; no valid source gives +0 and -inf.
//
// Pure HBM streaming: one thread per 8 columns (one 16-byte load per source, one 16-byte
// store).  The per-unit weights are computed once per thread from the S LSE values (a few
// L1-resident floats shared by the D/8 threads of the unit); the source loads of a thread are
// independent and issued back to back.
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

template <int SMAX>
__global__ void __launch_bounds__(256) lse_merge_kernel(LseMergeParams p)
{
    const int per_unit = p.D / 8;
    const int64_t total = (int64_t)p.T * p.H * per_unit;
    const int64_t TH = (int64_t)p.T * p.H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t unit = i / per_unit;
        const int k = (int)(i - unit * per_unit);
        float top = -INFINITY;
        for (int s = 0; s < p.S; s++) {
            const float l = p.lse2[s * TH + unit];
            if (valid_lse(l))
                top = fmaxf(top, l);
        }
        uint4 res = make_uint4(0, 0, 0, 0);
        if (top != -INFINITY) {
            float w[SMAX];
            float sum = 0.0f;
#pragma unroll
            for (int s = 0; s < SMAX; s++) {
                w[s] = 0.0f;
                if (s < p.S) {
                    const float l = p.lse2[s * TH + unit];
                    w[s] = valid_lse(l) ? exp2f(l - top) : 0.0f;
                    sum += w[s];
                }
            }
            float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            const uint4 *src = reinterpret_cast<const uint4 *>(p.partials) + unit * per_unit + k;
#pragma unroll
            for (int s = 0; s < SMAX; s++) {
                if (s < p.S && w[s] != 0.0f) {
                    const float scale = w[s] / sum;
                    const uint4 x = src[s * TH * per_unit];
                    acc[0] += scale * bf16_lo(x.x);
                    acc[1] += scale * bf16_hi(x.x);
                    acc[2] += scale * bf16_lo(x.y);
                    acc[3] += scale * bf16_hi(x.y);
                    acc[4] += scale * bf16_lo(x.z);
                    acc[5] += scale * bf16_hi(x.z);
                    acc[6] += scale * bf16_lo(x.w);
                    acc[7] += scale * bf16_hi(x.w);
                }
            }
            res.x = bf16_bits(acc[0]) | (bf16_bits(acc[1]) << 16);
            res.y = bf16_bits(acc[2]) | (bf16_bits(acc[3]) << 16);
            res.z = bf16_bits(acc[4]) | (bf16_bits(acc[5]) << 16);
            res.w = bf16_bits(acc[6]) | (bf16_bits(acc[7]) << 16);
            if (k == 0 && p.lse_out != nullptr) {
                const float lse2 = top + log2f(sum);
                p.lse_out[unit] = p.lse_log2 ? lse2 : lse2 * LN2;
            }
        } else if (k == 0 && p.lse_out != nullptr) {
            p.lse_out[unit] = -INFINITY;
        }
        reinterpret_cast<uint4 *>(p.out)[unit * per_unit + k] = res;
    }
}

template <int SMAX>
hipError_t launch_smax(const LseMergeParams &p, hipStream_t stream)
{
    const int64_t total = (int64_t)p.T * p.H * (p.D / 8);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(lse_merge_kernel<SMAX>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lse_merge(const LseMergeParams &p, hipStream_t stream)
{
    if (p.S <= 4)
        return launch_smax<4>(p, stream);
    if (p.S <= 8)
        return launch_smax<8>(p, stream);
    if (p.S <= 16)
        return launch_smax<16>(p, stream);
    if (p.S <= MAX_SOURCES)
        return launch_smax<MAX_SOURCES>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace smla
