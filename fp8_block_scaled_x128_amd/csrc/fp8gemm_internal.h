// fp8gemm_internal.h -- types shared by the gfx950 kernels and the host dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "fp8gemm_args.h"

namespace fp8gemm {

inline FastDiv make_fastdiv(uint32_t d) {
    if (d == 0) d = 1;  // empty dimensions launch nothing; keep the fields well defined
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const uint64_t mul = (((1ull << 32) * ((1ull << s) - d)) / d) + 1;
    return FastDiv{d, (uint32_t)mul, s};
}

struct KernelEntry {
    const char* name;
    int kind;                   // KernelKind
    int layout;
    bool fp4;                   // B in E2M1 with E8M0 scales per 32 K (masked decode kernel only)
    int bm, bn, waves_m, waves_n, stages;
    int jn, kp;                 // stream kernel: B fragments per wave, K blocks per A phase
    int threads;
    bool splitk;                // compiled with the split-K partial reduction
    int lds_bytes;
    const void* func;
    void (*launch)(dim3 grid, const KernelArgs& a, hipStream_t s);
};

const KernelEntry* kernel_table(int* count);
const KernelEntry* stream_table(int* count);

// Static device scratch of the allocation-free dense entry point (scratch.hip): fp32 split-K
// partial tiles and int32 arrival counters.  16 MiB of partials hold every automatically chosen
// dense split launch on up to 256 CUs (at most one unit per CU, tiles of at most 128 x 128 fp32);
// larger needs are refused.
constexpr size_t kScratchPartialBytes = size_t(16) << 20;
constexpr size_t kScratchCounters = 4096;

struct ScratchPointers {
    float* partials = nullptr;
    int32_t* counters = nullptr;
    int32_t* err = nullptr;     // the device error word (static as well)
};

// Device addresses of the static arrays on the current device (hipGetSymbolAddress); 0 on success.
int scratch_pointers(ScratchPointers* out);

// Tiled kernel of a table entry with N and K fixed at compile time, built at run time
// (fp8gemm_jit.cpp).
struct JitKernel {
    hipFunction_t fn = nullptr;
    int occupancy = 1;          // workgroups per CU
    double compile_ms = 0.0;    // compile and load time of the first request
};

// Code object (gfx950) of entry e specialised to (N, K) and the kernel's symbol name; needs no GPU.
int jit_compile(const KernelEntry& e, int N, int K, std::vector<char>* code, std::string* lowered,
                std::string* log);
// Specialised kernel on `device` (the current device), compiled and loaded on first request and
// cached for the life of the process.
int jit_kernel(int device, const KernelEntry& e, int entry, int N, int K, const JitKernel** out);
int jit_cache_size();

// 1x128 activation quantiser: a workgroup covers kQuantBlocksPerWG consecutive 128-wide blocks
// of the flattened [G][rows][K] input; the grid is ceil(blocks / kQuantBlocksPerWG) rounded up to
// a multiple of 8 (the number of XCDs the workgroup order is arranged for).
constexpr int kQuantBlocksPerWG = 16;

struct QuantArgs {
    const uint16_t* X;          // [G][rows][K] bf16 bits ([G][rows][2K] for the SwiGLU variant)
    uint8_t* A;                 // [G][rows][K] E4M3 codes
    float* sa;                  // [G][nkb][rows]
    const int32_t* masked_m;    // [G] valid rows per group, or null (all rows)
    int32_t* err;               // device error word (FP8GEMM_DEVERR_BAD_COUNT)
    int32_t rows;               // rows per group
    int32_t K, nkb, G;
    uint32_t blocks;            // G * rows * nkb (< 2^31)
    FastDiv div_nkb;            // flat block -> row
    FastDiv div_rows;           // row -> group
};

void launch_quantize_1x128(const QuantArgs& a, dim3 grid, hipStream_t stream);

// SwiGLU + 1x128 quantiser: the same arguments, with X rows of 2K bf16 values (gate | up).
void launch_swiglu_quantize(const QuantArgs& a, dim3 grid, hipStream_t stream);

}  // namespace fp8gemm
