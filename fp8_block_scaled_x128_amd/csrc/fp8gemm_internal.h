// fp8gemm_internal.h -- types shared by the gfx950 kernels and the host dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gemm {

enum Layout { kDense = 0, kContiguous = 1, kMasked = 2 };

enum DevErr { kDevErrBadIndex = 1, kDevErrBadCount = 2 };

// Everything one launch needs; passed by value as the kernel argument.
struct KernelArgs {
    const uint8_t* A;           // [rows_total][K] E4M3 codes
    const float* sa;            // [rows_total][nkb]
    const uint8_t* B;           // [G][N][K]
    const float* sb;            // [G][nnb][nkb]
    uint16_t* D;                // [rows_total][N] bf16 bits
    const int32_t* m_indices;   // contiguous layout: [rows], -1 = padding
    const int32_t* masked_m;    // masked layout: [G]
    int32_t* err;               // device error word (FP8GEMM_DEVERR_* bits)
    float* ws;                  // split-K partial tiles [tiles][splits][BM*BN]
    int32_t* counters;          // split-K arrival counters [tiles], zero between launches
    int64_t rows;               // dense: M; contiguous: M_total; masked: M_max
    int64_t units;              // work units = groups * tiles_m * tiles_n * splits
    int32_t N, K, G;
    int32_t nkb, nnb;           // K/128, ceil(N/128)
    int32_t tiles_m, tiles_n;
    int32_t splits, kb_per_split;
    int32_t group_m;            // M tiles per band of the unit order (1 = plain order)
};

struct KernelEntry {
    const char* name;
    int layout;
    int bm, bn, waves_m, waves_n, stages;
    int prefetch;               // L2 prefetch distance in K slices (0 = none)
    int threads;
    bool splitk;                // compiled with the split-K partial reduction
    int lds_bytes;
    const void* func;
    void (*launch)(dim3 grid, const KernelArgs& a, hipStream_t s);
};

const KernelEntry* kernel_table(int* count);

}  // namespace fp8gemm
