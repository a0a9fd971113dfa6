// quantize_kernels.hip -- gfx950 kernel of the 1x128 activation quantiser: bf16 activations to
// E4M3 codes plus one fp32 scale per block of 128 consecutive K values of a row, in the layout
// the GEMM kernels read (codes [G][rows][K], scales K-block-major [G][K/128][rows]).
//
// The pages take the fine-grained scaling from DeepSeek V3 (page "DeepSeek開源第三彈：V3/R1訓練
// 推理關鍵秘籍，核心代碼僅300行", section 深入了解DeepGEMM) and leave the quantiser itself open;
// per block: amax = max |x| floored at fp32(1e-4), s = fp32(amax / 448), code = E4M3
// round-to-nearest-even of fp32(x / s), saturated to +-448.
//
// The work is a stream: 2 bytes read and 1 + 4/128 bytes written per element, so the design is
// about HBM, not arithmetic.  Sixteen lanes own one 128-wide block (16 bytes, 8 values each),
// which makes every load instruction read whole 256-byte row segments; the block maximum is a
// four-step cross-lane reduction inside a 16-lane DPP row; a workgroup covers 16 rows x 4 blocks
// so the scale stores of one block are 64-byte runs.

#include "fp8gemm_internal.h"

namespace fp8gemm {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 4;                    // 4 x 16 lanes
constexpr int kBlocksPerLane = kQuantBlocksPerWG;  // 128-wide K blocks per lane (loads in flight)
static_assert(kWaves * kRowsPerWave == kQuantRowsPerWG, "workgroup tile");

// 8 bf16 values of one lane, element 2i in the low half of word i.
typedef uint32_t Chunk __attribute__((ext_vector_type(4)));

// Maximum over the 16 lanes of a DPP row (lanes 16j .. 16j+15); every lane gets the result.
__device__ inline uint32_t row16_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));  // row_mirror
    return v;
}

// Quantise the 8 values of one lane's chunk of a block; returns their 8 codes (element e in byte
// e) and the block's scale.
__device__ inline uint2 quantize_chunk(const Chunk& c, float* scale) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = c[i] & 0x7FFF7FFFu;  // |x| of both halves
        m = max(m, max(w & 0xFFFFu, w >> 16));
    }
    m = row16_max(m);  // |x| bit patterns order like the values
    const float amax = fmaxf(__uint_as_float(m << 16), 1e-4f);
    const float s = amax / 448.0f;  // correctly rounded fp32 division
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __builtin_amdgcn_fmed3f(__uint_as_float(c[i] << 16) / s, -448.0f, 448.0f);
        v[2 * i + 1] = __builtin_amdgcn_fmed3f(__uint_as_float(c[i] & 0xFFFF0000u) / s, -448.0f, 448.0f);
    }
    // each conversion packs two codes into the low (false) or high (true) half of a word
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
    *scale = s;
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

template <int NB>
__device__ inline void quantize_blocks(const QuantArgs& a, const uint16_t* xrow, uint8_t* arow,
                                       float* sa_col, int kb0, bool writes_scale) {
    Chunk c[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
        c[j] = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(xrow + (int64_t)(kb0 + j) * 128));
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        float s;
        const uint2 q = quantize_chunk(c[j], &s);
        *reinterpret_cast<uint2*>(arow + (int64_t)(kb0 + j) * 128) = q;
        if (writes_scale) sa_col[(int64_t)(kb0 + j) * a.rows] = s;
    }
}

__global__ __launch_bounds__(kWaves * 64) void quantize_1x128_kernel(QuantArgs a) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t g = fast_div(blockIdx.x, a.div_row_groups);
    const uint32_t rg = blockIdx.x - g * (uint32_t)a.row_groups;
    int64_t count = a.rows;
    if (a.masked_m) {
        const int32_t c = a.masked_m[g];
        if (c < 0 || c > a.rows) {
            if (rg == 0 && blockIdx.y == 0 && threadIdx.x == 0) atomicOr(a.err, (int32_t)kDevErrBadCount);
        }
        count = c < 0 ? 0 : (c > a.rows ? a.rows : c);
    }
    // The 16 lanes of a DPP row share one row, so a row past the end retires all of them.
    const int64_t r = (int64_t)rg * kQuantRowsPerWG + wave * kRowsPerWave + (lane >> 4);
    if (r >= count) return;
    const int chunk = lane & 15;
    const int64_t row = (int64_t)g * a.rows + r;
    const uint16_t* xrow = a.X + row * a.K + chunk * 8;
    uint8_t* arow = a.A + row * a.K + chunk * 8;
    float* sa_col = a.sa + (int64_t)g * a.nkb * a.rows + r;
    const int kb0 = blockIdx.y * kBlocksPerLane;
    const bool writes_scale = chunk == 0;
    if (kb0 + kBlocksPerLane <= a.nkb) {
        quantize_blocks<kBlocksPerLane>(a, xrow, arow, sa_col, kb0, writes_scale);
    } else {
        for (int kb = kb0; kb < a.nkb; ++kb) quantize_blocks<1>(a, xrow, arow, sa_col, kb, writes_scale);
    }
}

}  // namespace

void launch_quantize_1x128(const QuantArgs& a, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL(quantize_1x128_kernel, grid, dim3(kWaves * 64), 0, stream, a);
}

}  // namespace fp8gemm
