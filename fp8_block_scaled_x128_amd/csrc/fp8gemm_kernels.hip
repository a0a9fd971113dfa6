// fp8gemm_kernels.hip -- gfx950 (MI355X) tiled kernels of the FP8 block-scaled GEMM: the
// ahead-of-time instantiation table of the kernel body in fp8gemm_tiled.h (dense NT GEMM and the
// contiguous and masked M-grouped layouts of page "DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，
// 核心代碼僅300行", section 如何使用？).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8gemm_internal.h"
#include "fp8gemm_tiled.h"

namespace fp8gemm {

// ------------------------------------------------------------------------------------------
// instantiation table
// ------------------------------------------------------------------------------------------

template <int BM, int BN, int WMW, int WNW, int STAGES, int LAYOUT>
static void launch_impl(dim3 grid, const KernelArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((fp8gemm_kernel<BM, BN, WMW, WNW, STAGES, LAYOUT>), grid,
                       dim3(WMW * WNW * 64), 0, s, a);
}

template <int BM, int BN, int WMW, int WNW, int STAGES, int LAYOUT>
static KernelEntry entry(const char* name) {
    using T = Tile<BM, BN, WMW, WNW, STAGES, LAYOUT>;
    KernelEntry e;
    e.name = name;
    e.kind = kKindTiled;
    e.layout = LAYOUT;
    e.fp4 = false;
    e.bm = BM;
    e.bn = BN;
    e.waves_m = WMW;
    e.waves_n = WNW;
    e.stages = STAGES;
    e.jn = 0;
    e.kp = 0;
    e.threads = T::NT;
    e.splitk = T::SPLITK;
    e.lds_bytes = T::SMEM_BYTES;
    e.func = reinterpret_cast<const void*>(&fp8gemm_kernel<BM, BN, WMW, WNW, STAGES, LAYOUT>);
    e.launch = &launch_impl<BM, BN, WMW, WNW, STAGES, LAYOUT>;
    return e;
}

#define FP8GEMM_ENTRY(BM, BN, WMW, WNW, ST, L) \
    entry<BM, BN, WMW, WNW, ST, L>(#L " " #BM "x" #BN " waves " #WMW "x" #WNW " stages " #ST)

const KernelEntry* kernel_table(int* count) {
    static const KernelEntry table[] = {
        // Hardware counters of every entry the benchmark runs (matrix-core busy share, HBM bytes
        // against the algorithmic bytes, wait share) are in profiles/counters_dense_prefill.txt,
        // counters_dense_decode.txt and counters_grouped.txt, one block per workload.
        //
        // dense, prefill: 256x256 tiles, 8 waves (4 along M x 2 along N), 2-slice ring (matrix
        // cores busy 0.26-0.47 of the time on the five M = 4096 shapes it runs)
        FP8GEMM_ENTRY(256, 256, 4, 2, 2, kDense),
        // dense, prefill, narrower N tiles for widths whose 256-wide tiles leave CUs idle or
        // split into many stream-K segments (chosen by the estimated time of the busiest
        // workgroup: N = 1536 and 2112 take 256 x 192 with stream-K, N = 2112 at short K 256 x 160)
        FP8GEMM_ENTRY(256, 160, 4, 2, 2, kDense),
        FP8GEMM_ENTRY(256, 192, 4, 2, 2, kDense),
        // dense, medium
        FP8GEMM_ENTRY(128, 128, 2, 2, 4, kDense),
        FP8GEMM_ENTRY(128, 256, 2, 4, 2, kDense),
        // dense, decode: all rows of A in one tile, narrow N tiles (HBM bytes 1.0-1.7x the
        // algorithmic, waves waiting 40-63% of their cycles)
        FP8GEMM_ENTRY(64, 64, 1, 4, 4, kDense),
        FP8GEMM_ENTRY(64, 128, 1, 4, 3, kDense),
        FP8GEMM_ENTRY(128, 128, 2, 4, 3, kDense),
        // dense, decode, long K: a 6-slice ring consumed two slices per barrier (64x7168x16384:
        // 34.0 against 36.0 us for the 4-slice ring, same split; 8 slices 35.6 us)
        FP8GEMM_ENTRY(64, 64, 1, 4, 6, kDense),
        // contiguous grouped: 256-row tiles run one pass per group among their two 128-row blocks
        // (configuration 2: 891 us against 1179 us for 128x256 tiles; configuration 3: 546 / 651 us)
        FP8GEMM_ENTRY(256, 256, 4, 2, 2, kContiguous),
        FP8GEMM_ENTRY(128, 128, 2, 2, 4, kContiguous),
        FP8GEMM_ENTRY(128, 128, 2, 4, 3, kContiguous),
        FP8GEMM_ENTRY(64, 64, 1, 4, 4, kContiguous),
        FP8GEMM_ENTRY(64, 128, 1, 4, 3, kContiguous),
        // masked grouped
        FP8GEMM_ENTRY(64, 64, 1, 4, 4, kMasked),
        FP8GEMM_ENTRY(64, 128, 1, 4, 3, kMasked),
        FP8GEMM_ENTRY(128, 128, 2, 4, 3, kMasked),
        FP8GEMM_ENTRY(128, 128, 2, 2, 4, kMasked),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fp8gemm
