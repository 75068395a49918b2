// sparse_mla_decode_noalloc: sparse_mla_decode for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
// split-KV workspace comes from a file-scope static device array, `scratch`, instead of a
// caller's buffer; everything else is sparse_mla_decode's own path.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "smla.h"
#include "smla_internal.h"

// The workspace of every sparse_mla_decode_noalloc call on a device (each device holds its own
// copy, for the life of the process).  Host code never uses this name as an address: the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[SMLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = SMLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mu;
void *g_scratch[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call made with that device
// current.
hipError_t scratch_address(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

smla_status sparse_mla_decode_noalloc(const void *q, int64_t q_stride_t, int64_t q_stride_h,
                                      const void *kv_a, int64_t rows_a,
                                      const void *kv_b, int64_t rows_b, int32_t split_col,
                                      int32_t row_bytes, int32_t qk_dim,
                                      const int32_t *indices, const int32_t *lens,
                                      int32_t T, int32_t H, int32_t W,
                                      float bmm1_scale, float bmm2_scale, const float *sinks,
                                      void *out, float *lse, uint32_t flags,
                                      const smla_plan *plan, hipStream_t stream)
{
    // sizes are checked (and the plan resolved) before the scratch is looked at, so that a
    // problem too large for it is rejected with its own status and nothing is launched
    if (T < 0 || H <= 0 || H % 16 != 0 || W < 1)
        return SMLA_EINVAL;
    if (T == 0)
        return sparse_mla_decode(q, q_stride_t, q_stride_h, kv_a, rows_a, kv_b, rows_b,
                                 split_col, row_bytes, qk_dim, indices, lens, T, H, W,
                                 bmm1_scale, bmm2_scale, sinks, out, lse, flags, plan, nullptr, 0,
                                 stream);
    smla_plan chosen;
    if (plan != nullptr) {
        chosen = *plan;
    } else {
        const smla_status st = smla_decode_plan(T, H, W, row_bytes, flags, &chosen);
        if (st != SMLA_OK)
            return st;
    }
    const size_t need = smla_decode_workspace_size(&chosen, T, H);  // 0 for a bad plan too
    if (need > kScratchBytes)
        return SMLA_ESCRATCH;
    void *ws = nullptr;
    if (need > 0 && scratch_address(&ws) != hipSuccess)
        return SMLA_EHIP;
    // the header (status word, arrival counters) is zeroed by a kernel on the stream before
    // the decode: every call starts clean, whatever an earlier call left there
    return smla::decode_impl(q, q_stride_t, q_stride_h, kv_a, rows_a, kv_b, rows_b, split_col,
                             row_bytes, qk_dim, indices, lens, T, H, W, bmm1_scale, bmm2_scale,
                             sinks, out, lse, flags, &chosen, ws, need > 0 ? kScratchBytes : 0,
                             true, stream);
}

}  // extern "C"
