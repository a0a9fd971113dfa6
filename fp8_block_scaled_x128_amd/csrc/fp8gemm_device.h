// fp8gemm_device.h -- device helpers shared by the gfx950 GEMM kernels (direct-to-LDS loads,
// explicit memory-counter waits, the FP8 matrix-core step, bf16 packing, uniform values).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gemm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------------------------------
// device helpers
// ------------------------------------------------------------------------------------------

// Direct-to-LDS loads.  Lane i of the wave moves 16 (x4) or 4 (x1) bytes from global address
// sbase + voff (uniform 64-bit base, per-lane 32-bit offset) to LDS address lds_base + 16*i (4*i).  Written as inline asm so that the compiler does
// not insert a full vmcnt wait before every later LDS read (it cannot tell the ring's stages
// apart); the kernel waits for these loads itself with s_waitcnt vmcnt.  They have no register
// outputs.  M0 is written here and used by nothing else in these kernels (checked on the built
// code object by the build script).
__device__ __forceinline__ void dma_x4(uint32_t lds_base, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds_base), "v"(voff), "s"(sbase) : "memory");
}
__device__ __forceinline__ void dma_x1(uint32_t lds_base, const void* sbase, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :: "s"(lds_base), "v"(voff), "s"(sbase) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Wait until at most `extra + per * k` of this wave's DMA loads are in flight, 0 <= k <= KMAX
// (loads complete in issue order, so everything older than those is done).
template <int PER, int KMAX, int EXTRA>
__device__ __forceinline__ void wait_slices(int k) {
    if constexpr (KMAX == 0) {
        wait_vmcnt<EXTRA>();
    } else {
        if (k >= KMAX) wait_vmcnt<EXTRA + PER * KMAX>();
        else wait_slices<PER, KMAX - 1, EXTRA>(k);
    }
}

// Buffer resource flags of a raw (untyped) buffer on gfx9, and the sc1 cache-policy bit: an
// access coherent at agent scope (what the compiler emits for agent-scope atomic loads/stores).
constexpr int kBufferFlags = 0x00020000;
constexpr int kSc1 = 16;

// Values that are the same in every lane but not provably so to the compiler (results of
// cross-lane reductions, pointers derived from them) are moved to scalar registers explicitly.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<P*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ v4f mfma16x16x128(const v8i& x, const v8i& y) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // format code 0 = E4M3 for both operands; scale operands 0 select the unscaled form
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 0, 0, 0, 0, 0, 0);
}

// E2M1 x E4M3 partial: X = 16 rows of E2M1 codes (16 bytes per lane, the upper half of the
// operand unused), Y = 16 rows of E4M3 codes, with the E8M0 scale `scale_x` (one byte, 127 = 1)
// applied to this lane's 32 X elements; the Y operand is unscaled (127).
__device__ __forceinline__ v4f mfma16x16x128_fp4_fp8(const v8i& x, const v8i& y, int scale_x) {
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    // format codes: 4 = E2M1 for X, 0 = E4M3 for Y
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, zero, 4, 0, 0, scale_x, 0, 127);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even (v_cvt_pk_bf16_f32)
    uint16_t ua, ub;
    __builtin_memcpy(&ua, &a, 2);
    __builtin_memcpy(&ub, &b, 2);
    return (uint32_t)ua | ((uint32_t)ub << 16);
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace fp8gemm
