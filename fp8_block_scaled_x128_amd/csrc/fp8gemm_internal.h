// fp8gemm_internal.h -- types shared by the gfx950 kernels and the host dispatcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8gemm {

enum Layout { kDense = 0, kContiguous = 1, kMasked = 2 };

enum DevErr { kDevErrBadIndex = 1, kDevErrBadCount = 2 };

// Kernel families: output tiles staged through an LDS ring (every layout and size), and the
// masked decode kernel that streams B into registers (masked groups of few valid rows).
enum KernelKind { kKindTiled = 0, kKindStream = 1 };

// Unsigned division by a launch constant d >= 1 as multiply-high, add and shift (the round-up
// reciprocal method of Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994), exact for dividends below 2^31.  Built on the host; on the device the
// fields are kernel arguments, so the division runs on the scalar unit.
struct FastDiv {
    uint32_t d;       // divisor
    uint32_t mul;     // floor(2^32 * (2^shift - d) / d) + 1
    uint32_t shift;   // ceil(log2(d))
};

inline FastDiv make_fastdiv(uint32_t d) {
    if (d == 0) d = 1;  // empty dimensions launch nothing; keep the fields well defined
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const uint64_t mul = (((1ull << 32) * ((1ull << s) - d)) / d) + 1;
    return FastDiv{d, (uint32_t)mul, s};
}

__host__ __device__ inline uint32_t fast_div(uint32_t n, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t hi = __umulhi(n, f.mul);
#else
    const uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
#endif
    return (hi + n) >> f.shift;
}

// Everything one launch needs; passed by value as the kernel argument.
struct KernelArgs {
    const uint8_t* A;           // [rows_total][K] E4M3 codes
    const float* sa;            // [rows_total][nkb]
    const uint8_t* B;           // [G][N][K]
    const float* sb;            // [G][nnb][nkb]
    const uint8_t* sbe;         // E2M1 B: E8M0 scales [G][N][K/32] (B is then [G][N][K/2])
    uint16_t* D;                // [rows_total][N] bf16 bits
    const int32_t* m_indices;   // contiguous layout: [rows], -1 = padding
    const int32_t* masked_m;    // masked layout: [G]
    int32_t* err;               // device error word (FP8GEMM_DEVERR_* bits)
    float* ws;                  // split-K partial tiles [tiles][splits][BM*BN]
    int32_t* counters;          // split-K arrival counters [tiles], zero between launches
    int64_t rows;               // dense: M; contiguous: M_total; masked: M_max
    int32_t units;              // work units = groups * tiles_m * tiles_n * splits (< 2^30)
    int32_t N, K, G;
    int32_t nkb, nnb;           // K/128, ceil(N/128)
    int32_t tiles_m, tiles_n;
    int32_t splits, kb_per_split;
    int32_t group_m;            // M tiles per band of the unit order (1 = plain order)
    // divisors of the unit decode
    FastDiv div_splits, div_tiles_m, div_tiles_n;
    FastDiv div_groups;         // masked decode kernel: groups in the unit order (G)
    FastDiv div_group_tiles;    // tiles_m * tiles_n
    FastDiv div_band_units;     // group_m * tiles_n
    FastDiv div_band_h;         // group_m (height of a full band)
    FastDiv div_band_h_last;    // height of the last band, tiles_m - group_m * (bands - 1)
};

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
