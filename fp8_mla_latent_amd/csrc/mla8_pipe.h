// Device helpers of the split-T partial kernels (mla8_kernels.hip,
// mla8_partial32.hip): exact e4m3 -> fp16 widening, the query scaling
// exponent, and the LDS tile pipeline (barrier without a memory fence,
// counted waits, direct global -> LDS loads).
#pragma once

#include "mla8_device.h"

namespace mla8 {

// ---------------------------------------------------------------------------
// 8 e4m3 bytes (two dwords, byte 0 first) -> 8 fp16 values, exactly.
// HI selects bytes 2,3 of the dword instead of bytes 0,1.
template <bool HI>
__device__ __forceinline__ f16x2 cvt2(uint32_t v)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, HI);
}

__device__ __forceinline__ f16x8 cvt8(uint32_t lo, uint32_t hi)
{
    const f16x2 a = cvt2<false>(lo), b = cvt2<true>(lo), c = cvt2<false>(hi),
                e = cvt2<true>(hi);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], e[0], e[1]};
}

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Scaling exponent k of a head whose largest |e| is emax: emax 2^k in
// [2^14, 2^15).  k <= 100 keeps 2^-k a normal f32 (a head below 2^-86 then
// keeps fewer bits, irrelevant next to any score it could produce).
__device__ __forceinline__ int query_exp(float emax)
{
    int ex = 0;
    if (emax > 0.0f)
        (void)frexpf(emax, &ex);
    return (emax > 0.0f) ? min(15 - ex, 100) : 0;
}

constexpr float kTau = 8.0f;  // lazy-max slack, log2 units: weights stay <= 2^8

// ---------------------------------------------------------------------------
// LDS barrier without a memory fence: wait for this wave's LDS operations,
// then s_barrier.  A fenced __syncthreads would also wait for every
// outstanding global->LDS row load (vmcnt 0) and empty the load pipeline.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt not waited
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
    asm volatile("" ::: "memory");
}

#define MLA8_LDS __attribute__((address_space(3)))

// Direct global -> LDS loads, lane i writing LDS bytes [lds + 16i, +16)
// (dwordx4) or [lds + 4i, +4) (dword); lds is a wave-uniform LDS byte
// address.  Issued through asm so that the compiler's wait insertion does not
// track them: every wait on them is the explicit wait_vmcnt<> of the tile
// pipeline (a tracked load would be waited with vmcnt(0) wherever its LDS
// object is read, draining the pipeline).  These are the kernel's only users
// of m0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_b128(const void* src, uint32_t lds)
{
    lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform: keep it in an SGPR
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(src)
                 : "memory", "m0");
}

__device__ __forceinline__ void dma_b32(const void* src, uint32_t lds)
{
    lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform: keep it in an SGPR
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 :
                 : "s"(lds), "v"(src)
                 : "memory", "m0");
}
// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
// The base is passed through readfirstlane so that it is in SGPRs whatever
// the compiler's uniformity analysis concludes about it.
__device__ __forceinline__ const void* uniform_ptr(const void* p)
{
    const uint64_t b = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma_b128_s(const void* base, uint32_t voff, uint32_t lds)
{
    lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform: keep it in an SGPR
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(uniform_ptr(base))
                 : "memory", "m0");
}

__device__ __forceinline__ void dma_b32_s(const void* base, uint32_t voff, uint32_t lds)
{
    lds = __builtin_amdgcn_readfirstlane(lds);  // wave-uniform: keep it in an SGPR
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(uniform_ptr(base))
                 : "memory", "m0");
}
#pragma clang diagnostic pop


}  // namespace mla8
