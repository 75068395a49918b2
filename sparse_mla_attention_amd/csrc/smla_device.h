// Device helpers shared by the decode kernels (not part of the C ABI): vector types, FP8
// matrix instructions, asynchronous row loads with explicit waits, LDS-only barriers,
// device-scope accesses of the split exchange, the workgroup-to-work map, and the LDS swizzles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {
namespace dev {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define SMLA_LDS(T) __attribute__((address_space(3))) T
#define SMLA_GLOBAL(T) __attribute__((address_space(1))) T

constexpr float ANCHOR = 448.0f;                   // P anchor: E4M3's largest finite value
constexpr float LOG2_ANCHOR = 8.807354922057604f;  // log2(448)
constexpr float LN2 = 0.6931471805599453f;
constexpr float LOG2E = 1.4426950408889634f;

// XOR on the 16-byte piece index of latent row `key` in a V slot: eight consecutive keys put
// a 32-byte column pair on eight distinct bank groups (the transposed reads of P.V) and
// sixteen consecutive keys put one piece on sixteen (the QK waves' row writes).
__device__ inline int vsw(int key) { return ((key & 7) << 1) | ((key >> 3) & 1); }

// XOR on the 16-byte piece index of head h's 64-byte P row.
__device__ inline int psw(int h) { return (h >> 2) & 3; }

// Byte offset of byte `b` of row `row` in a BF16 output tile of 1024-byte rows: the 16-byte
// granule index is XORed with the row's low four bits, so that the same column of 16
// consecutive rows (one head per lane, as the accumulators hold them) falls in 16 different
// bank groups; a row read as 64 consecutive granules stays conflict free.
__device__ inline int tile_off(int row, int b)
{
    return row * 1024 + ((((b >> 4) ^ (row & 15)) << 4) | (b & 15));
}

__device__ inline v8i join(v4i x, v4i y)
{
    return v8i{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// 16-byte global load through a global (not flat) address: flat loads also count on the LDS
// wait counter, so every LDS wait would wait for the row loads in flight as well.
__device__ inline v4i gload(const uint8_t *p)
{
    return *(const SMLA_GLOBAL(v4i) *)(p);
}

template <typename T>
__device__ inline T lds_load(const uint8_t *base, int off)
{
    return *reinterpret_cast<const T *>(base + off);
}

// Row loads of the QK waves, issued from inline assembly so that the compiler's wait counting
// does not see them: with the three register stages rotating through an unrolled loop it made
// every trip wait for nearly every load in flight.  The kernel waits for them itself with
// counts that follow from the fixed issue order (NLD loads per chunk, nothing else).  The stage
// registers are operands of those waits, so no use of a stage is scheduled before its wait;
// the registers of a stage are never copied or reused while its loads are in flight (values
// that the compiler could copy, such as the row indices, are not loaded this way).

__device__ inline void gload_row_async(v4i (&st)[9], const uint8_t *row)
{
    asm volatile("global_load_dwordx4 %0, %9, off\n\t"
                 "global_load_dwordx4 %1, %9, off offset:64\n\t"
                 "global_load_dwordx4 %2, %9, off offset:128\n\t"
                 "global_load_dwordx4 %3, %9, off offset:192\n\t"
                 "global_load_dwordx4 %4, %9, off offset:256\n\t"
                 "global_load_dwordx4 %5, %9, off offset:320\n\t"
                 "global_load_dwordx4 %6, %9, off offset:384\n\t"
                 "global_load_dwordx4 %7, %9, off offset:448\n\t"
                 "global_load_dwordx4 %8, %9, off offset:512"
                 : "=&v"(st[0]), "=&v"(st[1]), "=&v"(st[2]), "=&v"(st[3]), "=&v"(st[4]),
                   "=&v"(st[5]), "=&v"(st[6]), "=&v"(st[7]), "=&v"(st[8])
                 : "v"(row));
}

__device__ inline void gload_row_async(v4i (&st)[8], const uint8_t *row)
{
    asm volatile("global_load_dwordx4 %0, %8, off\n\t"
                 "global_load_dwordx4 %1, %8, off offset:64\n\t"
                 "global_load_dwordx4 %2, %8, off offset:128\n\t"
                 "global_load_dwordx4 %3, %8, off offset:192\n\t"
                 "global_load_dwordx4 %4, %8, off offset:256\n\t"
                 "global_load_dwordx4 %5, %8, off offset:320\n\t"
                 "global_load_dwordx4 %6, %8, off offset:384\n\t"
                 "global_load_dwordx4 %7, %8, off offset:448"
                 : "=&v"(st[0]), "=&v"(st[1]), "=&v"(st[2]), "=&v"(st[3]), "=&v"(st[4]),
                   "=&v"(st[5]), "=&v"(st[6]), "=&v"(st[7])
                 : "v"(row));
}

// The same loads into accumulation registers (AGPRs): the matrix instructions read their
// operands from either register file, and this keeps the load stages out of the VGPRs.
__device__ inline void gload_row_async_acc(v4i (&st)[9], const uint8_t *row)
{
    asm volatile("global_load_dwordx4 %0, %9, off\n\t"
                 "global_load_dwordx4 %1, %9, off offset:64\n\t"
                 "global_load_dwordx4 %2, %9, off offset:128\n\t"
                 "global_load_dwordx4 %3, %9, off offset:192\n\t"
                 "global_load_dwordx4 %4, %9, off offset:256\n\t"
                 "global_load_dwordx4 %5, %9, off offset:320\n\t"
                 "global_load_dwordx4 %6, %9, off offset:384\n\t"
                 "global_load_dwordx4 %7, %9, off offset:448\n\t"
                 "global_load_dwordx4 %8, %9, off offset:512"
                 : "=&a"(st[0]), "=&a"(st[1]), "=&a"(st[2]), "=&a"(st[3]), "=&a"(st[4]),
                   "=&a"(st[5]), "=&a"(st[6]), "=&a"(st[7]), "=&a"(st[8])
                 : "v"(row));
}

template <int N>
__device__ inline void wait_vm_acc(v4i (&st)[9])
{
    asm volatile("s_waitcnt vmcnt(%9)"
                 : "+a"(st[0]), "+a"(st[1]), "+a"(st[2]), "+a"(st[3]), "+a"(st[4]),
                   "+a"(st[5]), "+a"(st[6]), "+a"(st[7]), "+a"(st[8])
                 : "i"(N));
}

// Wait until at most N vector memory loads are in flight; `x` is live across the wait.
template <int N>
__device__ inline void wait_vm(v4i (&st)[9])
{
    asm volatile("s_waitcnt vmcnt(%9)"
                 : "+v"(st[0]), "+v"(st[1]), "+v"(st[2]), "+v"(st[3]), "+v"(st[4]),
                   "+v"(st[5]), "+v"(st[6]), "+v"(st[7]), "+v"(st[8])
                 : "i"(N));
}

template <int N>
__device__ inline void wait_vm(v4i (&st)[8])
{
    asm volatile("s_waitcnt vmcnt(%8)"
                 : "+v"(st[0]), "+v"(st[1]), "+v"(st[2]), "+v"(st[3]), "+v"(st[4]),
                   "+v"(st[5]), "+v"(st[6]), "+v"(st[7])
                 : "i"(N));
}

// 16x16x128 FP8, unit scales (QK).
__device__ inline v4f mfma16(v8i a, v8i b, v4f c)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 16x16x32 FP8 (the 64-byte rope step of QK as two of these): 8 bytes per lane and operand.
__device__ inline v4f mfma16k32(v2i a, v2i b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(__builtin_bit_cast(long, a),
                                                      __builtin_bit_cast(long, b), c, 0, 0, 0);
}

// 32x32x64 FP8, unit A scale and the per-lane B scale byte sb (E8M0: lane l scales column
// l % 32 of its own 32-key block): 127 (2^0) for P's first term, 123 (2^-4) for its second.
__device__ inline v16f mfma32(v8i a, v8i b, v16f c, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// BF16 of a finite float, round to nearest even.
__device__ inline uint32_t bf16_bits(float x)
{
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two floats rounded to BF16 (nearest even) and packed, `lo` in the low half: one
// v_cvt_pk_bf16_f32.
typedef __bf16 v2bf16 __attribute__((ext_vector_type(2)));
__device__ inline uint32_t bf16x2(float lo, float hi)
{
    const v2bf16 r = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, r);
}

// Pad between the last matrix instruction of a chain and the first vector read of its result.
// A result of the block-scaled 32x32x64 FP8 instruction read 19 wait states after issue was
// measured to hold the chain's previous partial sum, so fresh results are read behind 24
// explicit wait states (the compiler's own padding comes on top).
__device__ inline void mfma_result_pad()
{
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
    __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that orders LDS only.  __syncthreads() is a workgroup fence over all
// memory, which makes every wave wait for its outstanding global loads before the barrier: the
// row loads in flight across iterations would be drained at every chunk.
__device__ inline void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Device-scope (all XCDs) relaxed accesses of the split exchange: coherent without a fence.
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

}  // namespace dev
}  // namespace smla
