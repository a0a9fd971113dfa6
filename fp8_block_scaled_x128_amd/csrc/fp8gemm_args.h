// fp8gemm_args.h -- the kernel argument block and the enums and helpers the device code needs:
// included by the kernels, by the host dispatcher, and by the run-time compiled tiled kernel.
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

__host__ __device__ inline uint32_t fast_div(uint32_t n, const FastDiv& f) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t hi = __umulhi(n, f.mul);
#else
    const uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);
#endif
    return (hi + n) >> f.shift;
}

// Stream-K schedule of the tiles left over after the last full round of tiles (dense layout,
// 256-row tiles).  The leftover tiles' K blocks form one sequence in (tile, K block) order;
// workgroup w (logical id, 0 <= w < P) takes blocks [sk_start(w), sk_start(w + 1)), with
// sk_start(w) = w * per + min(w, extra): the first `extra` workgroups take per + 1 blocks, the
// others per.  A range is no longer than a tile's K extent (per < blocks per tile), so it
// touches at most two tiles (its segments 0 and 1).
__host__ __device__ inline int sk_start(int w, int per, int extra) { return w * per + (w < extra ? w : extra); }

// The workgroup whose range holds block g of the sequence (per >= 1).
__host__ __device__ inline int sk_owner(int g, int per, int extra) {
    const int big = extra * (per + 1);
    return g < big ? g / (per + 1) : extra + (g - big) / per;
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
    // stream-K (0 sk_tiles: none): the tiles after the first `units` take the schedule above,
    // sk_per and sk_extra for the grid's P workgroups; partials in ws slots 2w + segment
    int32_t sk_tiles, sk_per, sk_extra;
};

}  // namespace fp8gemm
