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
// about HBM, not arithmetic.  K is a multiple of 128, so a 128-wide block never straddles two
// rows and X, the codes and the block index are one flat sequence.  A workgroup takes 16
// consecutive blocks (one contiguous 4 KB span of X, 2 KB of codes); sixteen lanes own one block
// (16 bytes, 8 values each), so every load instruction reads 1 KB of consecutive memory, and the
// block maximum is a four-step cross-lane reduction inside a 16-lane DPP row.  Workgroup ids are
// remapped so that each XCD takes a contiguous range of spans: the scale stores of neighbouring
// rows (adjacent words of the K-block-major scale array) then meet in the same L2.  Contiguous
// per-workgroup spans sustain about 6 TB/s for this read/write mix on MI355X, against about
// 5 TB/s for tiles of 16 rows x 4 blocks.
//
// The same file holds the SwiGLU variant used between the two linear layers of an MoE expert
// (page "Perpustakaan operator GPU sumber terbuka DeepSeek DeepGEMM memperbarui versi besar,
// menambahkan Mega MoE…": first linear layer, SwiGLU activation, second linear layer): it reads
// a row's gate and up halves, forms silu(gate) * up in fp32 and quantises those values with the
// same block quantiser, fused, so the activation never makes a round trip through HBM.

#include "fp8gemm_internal.h"

namespace fp8gemm {
namespace {

static_assert(kQuantBlocksPerWG * 16 == 256, "16 lanes per block, 256 threads per workgroup");

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

// x / s rounded to nearest even, in three operations instead of a full division: with r = RN(1/s),
// q = RN(x * r) is within one unit in the last place of x / s, the residual x - q * s is exact
// in a fused multiply-add, and RN(q + residual * r) is the correctly rounded quotient (Markstein,
// "Computation of elementary functions on the IBM RISC System/6000 processor", IBM J. Res. Dev.
// 34(1), 1990).  Where the quotient falls below 2^-11 (a subnormal x) the result may differ in its
// last bits but not in its E4M3 code (signed zero); the sign is taken from x so that -0 stays -0.
// Enumerating every bf16 x against every scale a block can have confirms both claims.
__device__ inline float div_rn(float x, float s, float r) {
    const float q = x * r;
    const float e = __builtin_fmaf(-q, s, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, q), x);
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
    const float r = 1.0f / s;       // correctly rounded reciprocal, shared by the block
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __builtin_amdgcn_fmed3f(div_rn(__uint_as_float(c[i] << 16), s, r), -448.0f, 448.0f);
        v[2 * i + 1] = __builtin_amdgcn_fmed3f(div_rn(__uint_as_float(c[i] & 0xFFFF0000u), s, r), -448.0f, 448.0f);
    }
    // each conversion packs two codes into the low (false) or high (true) half of a word
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
    *scale = s;
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// The same block quantiser on 8 fp32 values (a lane's share of a 128-value block): |x| bit
// patterns of finite fp32 values order like the values, so the block maximum is again an integer
// reduction; then s = amax / 448, the correctly rounded quotients, saturation and the RNE
// conversion, as above.
__device__ inline uint2 quantize_f32x8(const float (&x)[8], float* scale) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
    m = row16_max(m);
    const float amax = fmaxf(__uint_as_float(m), 1e-4f);
    const float s = amax / 448.0f;
    const float r = 1.0f / s;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = __builtin_amdgcn_fmed3f(div_rn(x[i], s, r), -448.0f, 448.0f);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], hi, true);
    *scale = s;
    return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// SwiGLU of one element in fp32: silu(g) * u = (g * sigmoid(g)) * u, sigmoid(g) = 1 / (1 + e^-g).
// e^-g is the hardware base-2 exponential of -g * log2(e) and the reciprocal the hardware one
// (each within about one unit in the last place; the result feeds a 3-bit-mantissa code).  For
// g below about -88, e^-g is infinite, sigmoid 0 and the product a signed zero.
__device__ inline float swiglu1(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    const float sig = __builtin_amdgcn_rcpf(1.0f + e);
    return (g * sig) * u;
}

__global__ __launch_bounds__(256) void quantize_1x128_kernel(QuantArgs a) {
    // XCD-aware order: dispatch sends consecutive workgroups to consecutive XCDs, so workgroup
    // i works on logical span (i % 8) * (P / 8) + i / 8 (the grid size P is a multiple of 8).
    const uint32_t P = gridDim.x;
    const uint32_t wg = (blockIdx.x & 7u) * (P >> 3) + (blockIdx.x >> 3);
    const uint32_t b = wg * kQuantBlocksPerWG + (threadIdx.x >> 4);  // 128-wide block, flat
    if (b >= a.blocks) return;  // the 16 lanes of a block leave together
    const uint32_t row = fast_div(b, a.div_nkb);  // row over all groups
    const uint32_t kb = b - row * (uint32_t)a.nkb;
    const uint32_t g = fast_div(row, a.div_rows);
    const uint32_t r = row - g * (uint32_t)a.rows;
    if (a.masked_m) {
        const int32_t c = a.masked_m[g];
        if ((c < 0 || c > a.rows) && r == 0 && kb == 0 && (threadIdx.x & 15) == 0)
            atomicOr(a.err, (int32_t)kDevErrBadCount);
        if ((int32_t)r >= c) return;  // c < 0 counts as 0; c > rows cannot stop a row < rows
    }
    const int chunk = threadIdx.x & 15;
    const int64_t off = (int64_t)b * 128 + chunk * 8;
    const Chunk c = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(a.X + off));
    float s;
    const uint2 q = quantize_chunk(c, &s);
    *reinterpret_cast<uint2*>(a.A + off) = q;
    if (chunk == 0) a.sa[((int64_t)g * a.nkb + kb) * a.rows + r] = s;
}

// SwiGLU activation and requantisation between the two GEMMs of an MoE expert: X rows hold 2K
// bf16 values, the gate in columns [0, K) and the up projection in [K, 2K); the K activations
// silu(gate) * up of a row are quantised per 1x128 block exactly as quantize_1x128_kernel does
// (codes [G][rows][K], scales [G][K/128][rows]).  Same mapping: 16 lanes per block, 16 blocks
// per workgroup, XCD-aware order; a lane reads 16 bytes of gate and 16 of up.
__global__ __launch_bounds__(256) void swiglu_quantize_kernel(QuantArgs a) {
    const uint32_t P = gridDim.x;
    const uint32_t wg = (blockIdx.x & 7u) * (P >> 3) + (blockIdx.x >> 3);
    const uint32_t b = wg * kQuantBlocksPerWG + (threadIdx.x >> 4);
    if (b >= a.blocks) return;
    const uint32_t row = fast_div(b, a.div_nkb);
    const uint32_t kb = b - row * (uint32_t)a.nkb;
    const uint32_t g = fast_div(row, a.div_rows);
    const uint32_t r = row - g * (uint32_t)a.rows;
    if (a.masked_m) {
        const int32_t c = a.masked_m[g];
        if ((c < 0 || c > a.rows) && r == 0 && kb == 0 && (threadIdx.x & 15) == 0)
            atomicOr(a.err, (int32_t)kDevErrBadCount);
        if ((int32_t)r >= c) return;
    }
    const int chunk = threadIdx.x & 15;
    const uint16_t* xr = a.X + (int64_t)row * (2 * (int64_t)a.K) + kb * 128 + chunk * 8;
    const Chunk gc = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(xr));
    const Chunk uc = __builtin_nontemporal_load(reinterpret_cast<const Chunk*>(xr + a.K));
    float h[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[2 * i] = swiglu1(__uint_as_float(gc[i] << 16), __uint_as_float(uc[i] << 16));
        h[2 * i + 1] = swiglu1(__uint_as_float(gc[i] & 0xFFFF0000u), __uint_as_float(uc[i] & 0xFFFF0000u));
    }
    float s;
    const uint2 q = quantize_f32x8(h, &s);
    *reinterpret_cast<uint2*>(a.A + (int64_t)row * a.K + kb * 128 + chunk * 8) = q;
    if (chunk == 0) a.sa[((int64_t)g * a.nkb + kb) * a.rows + r] = s;
}

}  // namespace

void launch_quantize_1x128(const QuantArgs& a, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL(quantize_1x128_kernel, grid, dim3(256), 0, stream, a);
}

void launch_swiglu_quantize(const QuantArgs& a, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL(swiglu_quantize_kernel, grid, dim3(256), 0, stream, a);
}

}  // namespace fp8gemm
