/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the FP8 block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library path may call, link or load this file;
 * only the test suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 * It shares no code, header, table or constant with the HIP implementation.
 *
 * Sources (cited by page title and section):
 *   [P1] "DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，核心代碼僅300行"
 *        - section 深入了解DeepGEMM: FP8 GEMM with fine-grained scaling (a design taken from
 *          DeepSeek V3); FP8 tensor-core accumulation is imprecise, so partial results are
 *          promoted and accumulated a second time at higher precision (two-level accumulation).
 *        - section 如何使用？: the three entry points gemm_fp8_fp8_bf16_nt (NT: left operand not
 *          transposed, right operand transposed), m_grouped_gemm_fp8_fp8_bf16_nt_contiguous and
 *          m_grouped_gemm_fp8_fp8_bf16_nt_masked; FP8 inputs, BF16 output.
 *   [P3] "DeepGEMM：AI計算の経済性を変えるオープンソースライブラリ"
 *        - section DeepGEMMが重要な理由, item 4: contiguous grouped GEMM (token sequences grouped
 *          per expert) and masked grouped GEMM (sparse expert activation).
 *
 * The pages say "fine-grained scaling" only.  The reading taken here (listed with every other
 * reading in the design notes): A carries one fp32 scale per 1x128 block of a row (sa[M][K/128]),
 * B one fp32 scale per 128x128 block (sb[ceil(N/128)][K/128]); FP8 is OCP E4M3 (e4m3fn).
 *
 * What is computed is the plain definition of the dequantised product, rounded once:
 *
 *   D[m][n] = bf16_rne( sum_kb  sa[m][kb] * sb[n/128][kb] * sum_{k in block kb} e4m3(A[m][k]) * e4m3(B[n][k]) )
 *
 * The inner block sum is exact in fp64 in any order: every e4m3 value is an integer multiple of
 * 2^-9 of magnitude below 2^18 * 2^-9, so each product is a multiple of 2^-18 below 2^36 * 2^-18
 * and 128 of them stay below 2^43 * 2^-18, inside fp64's 53-bit significand.  The scale product
 * sa*sb of two fp32 values is exact in fp64 (48-bit significand).  The sum over K-blocks is done
 * with fp64 fused multiply-add, then rounded once, fp64 -> bf16, round to nearest even.
 *
 * The activation quantiser (oracle_quantize_1x128) is the step just before the product: the pages
 * take fine-grained scaling from DeepSeek V3 ([P1], section 深入了解DeepGEMM) and name no
 * quantiser, so its definition is the plain reading of a 1x128 block scale: per block of 128
 * consecutive K values of a row, amax = max |x| (floored at fp32(1e-4) so that an all-zero block
 * keeps a finite scale), s = fp32(amax / 448), code = E4M3 round-to-nearest-even of fp32(x / s)
 * saturated to +-448.  448 is E4M3's largest finite value, so the largest element of every block
 * maps to +-448.
 *
 * Parity pins (tests/test_oracle_pins.py): e4m3 decode against the OCP table anchors and an
 * independent library decoder; bf16 rounding against exact rational rounding; whole products
 * against exact rational brute force on tiny shapes, integer closed forms, power-of-two scale
 * closed forms, a library fp64 matmul of the dequantised operands, and the grouping/permutation/
 * padding invariants; the E4M3 encoder against torch's float8 cast over every fp32 neighbour of
 * every E4M3 value and rounding midpoint; the quantiser against hand-worked golden blocks, the
 * block-maximum, sign-symmetry and power-of-two scaling invariants and the format's rounding
 * error bound.  No function below is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_API __attribute__((visibility("default")))

/* ---- element formats --------------------------------------------------------------------- */

/* OCP 8-bit floating point, E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * Exponent field 0 is subnormal (f * 2^-9); S.1111.111 is NaN; there is no infinity, so the
 * largest finite value is S.1111.110 = 1.75 * 2^8 = 448. */
ORACLE_API double oracle_e4m3_value(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int f = code & 0x7;
    double v;
    if (e == 0xF && f == 0x7) return NAN;
    if (e == 0)
        v = ldexp((double)f, -9);                 /* f/8 * 2^(1-7) */
    else
        v = ldexp(1.0 + (double)f / 8.0, e - 7);
    return sign ? -v : v;
}

/* Round an fp64 value to bfloat16 (1 sign, 8 exponent bits with bias 127, 7 stored mantissa
 * bits), round to nearest, ties to even, in a single step.  Result: the 16-bit pattern. */
ORACLE_API uint16_t oracle_bf16_bits(double x) {
    if (isnan(x)) return 0x7FC0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (ax == 0.0) return sign;
    int e2;
    frexp(ax, &e2);                       /* ax in [2^(e2-1), 2^e2) */
    int unit_exp = e2 - 1 - 7;            /* weight of the last kept bit for a normal bf16 */
    if (e2 - 1 < -126) unit_exp = -126 - 7; /* subnormal range: fixed quantum 2^-133 */
    double q = ldexp(nearbyint(ldexp(ax, -unit_exp)), unit_exp); /* default mode is RNE */
    if (q >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80);  /* overflow -> inf */
    float qf = (float)q;                  /* exact: q has <= 8 significant bits in range */
    uint32_t bits;
    memcpy(&bits, &qf, sizeof bits);
    return (uint16_t)(sign | (uint16_t)((bits >> 16) & 0x7FFF));
}

/* Encode a finite value as E4M3, round to nearest, ties to even, saturating at +-448 (the largest
 * finite value; E4M3 has no infinity).  Between 2^-6 and 448 a binade [2^E, 2^(E+1)) holds 8
 * values, spaced 2^(E-3); below 2^-6 the values are the multiples of 2^-9 (subnormals, code = the
 * multiple itself, and the multiple 8 is the code of 2^-6, the smallest normal).  The sign bit is
 * kept for values that round to zero. */
ORACLE_API uint8_t oracle_e4m3_code(double x) {
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double ax = fabs(x);
    if (ax >= 448.0) return (uint8_t)(sign | 0x7E);
    if (ax < ldexp(1.0, -6)) {
        double f = nearbyint(ldexp(ax, 9));       /* 0..8 multiples of 2^-9 */
        return (uint8_t)(sign | (uint8_t)f);
    }
    int e2;
    frexp(ax, &e2);                               /* ax in [2^(e2-1), 2^e2) */
    int E = e2 - 1;                               /* -6 .. 8 */
    double q = nearbyint(ldexp(ax, 3 - E));       /* 8 .. 16 eighths of 2^E */
    if (q == 16.0) { q = 8.0; ++E; }              /* rounded up into the next binade */
    if (E > 8 || (E == 8 && q > 14.0)) return (uint8_t)(sign | 0x7E);
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)(q - 8.0));
}

/* ---- one output element ------------------------------------------------------------------ */

/* Two-level sum for one output: per 128-wide K block an exact fp64 dot product of the decoded
 * codes, then scaled by sa*sb and accumulated across blocks (fp64 fused multiply-add).
 * a_row/b_row: K codes each; sa_row/sb_row: ceil(K/128) scales each. */
static double element(const double* a_row, const float* sa_row, const double* b_row,
                      const float* sb_row, int64_t K) {
    int64_t nkb = (K + 127) / 128;
    double acc = 0.0;
    for (int64_t kb = 0; kb < nkb; ++kb) {
        int64_t k0 = kb * 128, k1 = k0 + 128 < K ? k0 + 128 : K;
        double block = 0.0;
        for (int64_t k = k0; k < k1; ++k) block += a_row[k] * b_row[k];
        double s = (double)sa_row[kb] * (double)sb_row[kb];
        acc = fma(s, block, acc);
    }
    return acc;
}

static void decode_rows(const uint8_t* codes, int64_t rows, int64_t K, double* out) {
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = oracle_e4m3_value((uint8_t)c);
    for (int64_t i = 0; i < rows * K; ++i) out[i] = table[codes[i]];
}

static int pick_threads(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

ORACLE_API int oracle_num_threads(int nthreads) { return pick_threads(nthreads); }

/* ---- dense NT ---------------------------------------------------------------------------- */

/* D[M][N] (bf16 bits) = A[M][K] . B[N][K]^T with sa[M][ceil(K/128)], sb[ceil(N/128)][ceil(K/128)].
 * acc (optional, may be NULL): the fp64 value before the final rounding.  Returns 0, or -1 when
 * out of memory. */
ORACLE_API int oracle_gemm_nt(const uint8_t* A, const float* sa, const uint8_t* B, const float* sb,
                              int64_t M, int64_t N, int64_t K, uint16_t* D, double* acc,
                              int nthreads) {
    int64_t nkb = (K + 127) / 128;
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(N * K + 1));
    if (!Ad || !Bd) { free(Ad); free(Bd); return -1; }
    decode_rows(A, M, K, Ad);
    decode_rows(B, N, K, Bd);
    int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double v = element(Ad + m * K, sa + m * nkb, Bd + n * K, sb + (n / 128) * nkb, K);
            D[m * N + n] = oracle_bf16_bits(v);
            if (acc) acc[m * N + n] = v;
        }
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* ---- M-grouped, contiguous layout --------------------------------------------------------- */

/* Rows of all groups are concatenated along M.  Row r belongs to group g = m_indices[r] and is
 * multiplied by B[g] (B is [G][N][K], sb is [G][ceil(N/128)][ceil(K/128)]).  m_indices[r] == -1
 * marks a padding row: it has no defined output (valid[r] = 0, its D row is set to 0).  An index
 * outside [-1, G) is treated as padding too. */
ORACLE_API int oracle_grouped_contiguous(const uint8_t* A, const float* sa, const uint8_t* B,
                                         const float* sb, const int32_t* m_indices, int64_t M,
                                         int64_t N, int64_t K, int32_t G, uint16_t* D,
                                         uint8_t* valid, double* acc, int nthreads) {
    int64_t nkb = (K + 127) / 128, nnb = (N + 127) / 128;
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K + 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)((int64_t)G * N * K + 1));
    if (!Ad || !Bd) { free(Ad); free(Bd); return -1; }
    decode_rows(A, M, K, Ad);
    decode_rows(B, (int64_t)G * N, K, Bd);
    int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t r = 0; r < M; ++r) {
        int32_t g = m_indices[r];
        int ok = g >= 0 && g < G;
        if (valid) valid[r] = (uint8_t)ok;
        for (int64_t n = 0; n < N; ++n) {
            double v = 0.0;
            if (ok)
                v = element(Ad + r * K, sa + r * nkb, Bd + ((int64_t)g * N + n) * K,
                            sb + ((int64_t)g * nnb + n / 128) * nkb, K);
            D[r * N + n] = ok ? oracle_bf16_bits(v) : 0;
            if (acc) acc[r * N + n] = v;
        }
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* ---- M-grouped, masked layout ------------------------------------------------------------- */

/* Group g owns a fixed block of M_max rows: A[g][M_max][K], sa[g][M_max][ceil(K/128)],
 * D[g][M_max][N].  Only rows r < min(masked_m[g], M_max) are valid; the others have no defined
 * output (valid = 0, D set to 0).  A negative masked_m counts as 0. */
ORACLE_API int oracle_grouped_masked(const uint8_t* A, const float* sa, const uint8_t* B,
                                     const float* sb, const int32_t* masked_m, int32_t G,
                                     int64_t M_max, int64_t N, int64_t K, uint16_t* D,
                                     uint8_t* valid, double* acc, int nthreads) {
    int64_t nkb = (K + 127) / 128, nnb = (N + 127) / 128;
    int64_t rows = (int64_t)G * M_max;
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(rows * K + 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)((int64_t)G * N * K + 1));
    if (!Ad || !Bd) { free(Ad); free(Bd); return -1; }
    decode_rows(A, rows, K, Ad);
    decode_rows(B, (int64_t)G * N, K, Bd);
    int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t gr = 0; gr < rows; ++gr) {
        int64_t g = gr / (M_max > 0 ? M_max : 1), r = gr % (M_max > 0 ? M_max : 1);
        int64_t count = masked_m[g] < 0 ? 0 : (masked_m[g] > M_max ? M_max : masked_m[g]);
        int ok = r < count;
        if (valid) valid[gr] = (uint8_t)ok;
        for (int64_t n = 0; n < N; ++n) {
            double v = 0.0;
            if (ok)
                v = element(Ad + gr * K, sa + gr * nkb, Bd + (g * N + n) * K,
                            sb + (g * nnb + n / 128) * nkb, K);
            D[gr * N + n] = ok ? oracle_bf16_bits(v) : 0;
            if (acc) acc[gr * N + n] = v;
        }
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* ---- M-grouped, masked layout, B in E2M1 with E8M0 scales per 32 K ------------------------ */

/* OCP MX 4-bit float E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit.  Exponent field 0
 * is subnormal: m * 2^-1.  There is no infinity or NaN; the values are 0, 0.5, 1, 1.5, 2, 3, 4, 6
 * and their negatives. */
ORACLE_API double oracle_e2m1_value(uint8_t code) {
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

/* OCP MX scale E8M0: an unsigned 8-bit exponent, value 2^(s - 127); 0xFF is NaN. */
ORACLE_API double oracle_e8m0_value(uint8_t s) { return s == 0xFF ? NAN : ldexp(1.0, (int)s - 127); }

/* The masked grouped product with an FP4 right operand (page "Perpustakaan operator GPU sumber
 * terbuka DeepSeek DeepGEMM memperbarui versi besar, menambahkan Mega MoE…": FP8 x FP4 matrix
 * multiplication, the precision combination of Mega MoE; the pages give no FP4 format, the
 * reading taken is OCP MXFP4).  B[g][n] holds K E2M1 codes, two per byte (element k in byte k/2,
 * the even element in the low nibble): B is [G][N][K/2] bytes.  sb[g][n][k/32] is the E8M0 scale
 * of the 32 consecutive values k/32*32 .. +31 of that row.  A, sa (row-major [G*M_max][K/128]),
 * masked_m, D, valid and acc as oracle_grouped_masked.  Per valid output:
 *   D = bf16_rne( sum_kb sa[kb] * sum_{k in block kb} e4m3(A[k]) * e2m1(B[k]) * 2^(sb[k/32] - 127) )
 * Each 32-value sum is exact in fp64 (products are multiples of 2^-10 below 2^12); scaling by a
 * power of two is exact; the four scaled sums of a 128-value block are added in fp64, then the
 * blocks are accumulated as in the FP8 product.  K must be a multiple of 32. */
ORACLE_API int oracle_grouped_masked_fp4(const uint8_t* A, const float* sa, const uint8_t* B,
                                         const uint8_t* sb, const int32_t* masked_m, int32_t G,
                                         int64_t M_max, int64_t N, int64_t K, uint16_t* D,
                                         uint8_t* valid, double* acc, int nthreads) {
    int64_t nkb = (K + 127) / 128, nsb = K / 32;
    int64_t rows = (int64_t)G * M_max;
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(rows * K + 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)((int64_t)G * N * K + 1));
    if (!Ad || !Bd) { free(Ad); free(Bd); return -1; }
    decode_rows(A, rows, K, Ad);
    double e2m1[16];
    for (int c = 0; c < 16; ++c) e2m1[c] = oracle_e2m1_value((uint8_t)c);
    for (int64_t i = 0; i < (int64_t)G * N * K; ++i) {
        uint8_t byte = B[i / 2];
        Bd[i] = e2m1[(i & 1) ? (byte >> 4) : (byte & 0xF)];
    }
    int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t gr = 0; gr < rows; ++gr) {
        int64_t g = gr / (M_max > 0 ? M_max : 1), r = gr % (M_max > 0 ? M_max : 1);
        int64_t count = masked_m[g] < 0 ? 0 : (masked_m[g] > M_max ? M_max : masked_m[g]);
        int ok = r < count;
        if (valid) valid[gr] = (uint8_t)ok;
        for (int64_t n = 0; n < N; ++n) {
            double v = 0.0;
            if (ok) {
                const double* a = Ad + gr * K;
                const double* b = Bd + (g * N + n) * K;
                const uint8_t* srow = sb + (g * N + n) * nsb;
                for (int64_t kb = 0; kb < nkb; ++kb) {
                    double block = 0.0;
                    for (int64_t k0 = kb * 128; k0 < kb * 128 + 128 && k0 < K; k0 += 32) {
                        double sub = 0.0;
                        for (int64_t k = k0; k < k0 + 32; ++k) sub += a[k] * b[k];
                        block += oracle_e8m0_value(srow[k0 / 32]) * sub;
                    }
                    v = fma((double)sa[gr * nkb + kb], block, v);
                }
            }
            D[gr * N + n] = ok ? oracle_bf16_bits(v) : 0;
            if (acc) acc[gr * N + n] = v;
        }
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* ---- selected elements ------------------------------------------------------------------- */

/* The same element computation for `count` chosen outputs, for full-size problems where the
 * whole product is too slow on a CPU.  For sample i: the A row is a_rows[i] (row of A and of sa,
 * flattened over groups), the B row is b_rows[i] (row of B flattened over groups, i.e.
 * g*N + n) and the B scale row is sb_rows[i] (g*ceil(N/128) + n/128).  Out: bf16 bits and the
 * fp64 value (optional). */
ORACLE_API int oracle_elements(const uint8_t* A, const float* sa, const uint8_t* B,
                               const float* sb, int64_t K, const int64_t* a_rows,
                               const int64_t* b_rows, const int64_t* sb_rows, int64_t count,
                               uint16_t* out, double* acc, int nthreads) {
    int64_t nkb = (K + 127) / 128;
    int nt = pick_threads(nthreads);
    (void)nt;
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = oracle_e4m3_value((uint8_t)c);
    int failed = 0;
#pragma omp parallel num_threads(nt)
    {
        double* a = (double*)malloc(sizeof(double) * (size_t)(K + 1));
        double* b = (double*)malloc(sizeof(double) * (size_t)(K + 1));
        int mine_ok = a && b;
        if (!mine_ok) {
#pragma omp atomic write
            failed = 1;
        }
        /* every thread reaches the work-sharing loop; one without buffers does nothing */
#pragma omp for schedule(dynamic, 64)
        for (int64_t i = 0; i < count; ++i) {
            if (!mine_ok) continue;
            const uint8_t* ar = A + a_rows[i] * K;
            const uint8_t* br = B + b_rows[i] * K;
            for (int64_t k = 0; k < K; ++k) { a[k] = table[ar[k]]; b[k] = table[br[k]]; }
            double v = element(a, sa + a_rows[i] * nkb, b, sb + sb_rows[i] * nkb, K);
            out[i] = oracle_bf16_bits(v);
            if (acc) acc[i] = v;
        }
        free(a);
        free(b);
    }
    return failed ? -1 : 0;
}

/* ---- activation quantiser, 1x128 blocks ---------------------------------------------------- */

/* One block of n <= 128 fp32 values xs -> n codes and the block's scale:
 *   amax = max |x|
 *   amax = max(amax, fp32(1e-4))           (an all-zero or tiny block keeps a finite scale)
 *   s    = fp32(amax / 448)                (the scale stored in sa)
 *   v    = fp32(x / s)                     (the value to encode)
 *   code = E4M3_rne(v), saturating at +-448
 * Both quotients are formed in fp64 and rounded once to fp32; for a quotient of two fp32 values
 * fp64 carries more than 2*24+2 bits, so that double rounding equals the correctly rounded fp32
 * quotient. */
static float quantize_block(const float* xs, int64_t n, uint8_t* codes) {
    const float floor_amax = 1e-4f;
    float amax = 0.0f;
    for (int64_t k = 0; k < n; ++k) {
        float a = fabsf(xs[k]);
        if (a > amax) amax = a;
    }
    if (amax < floor_amax) amax = floor_amax;
    float s = (float)((double)amax / 448.0);
    for (int64_t k = 0; k < n; ++k) {
        float v = (float)((double)xs[k] / (double)s);
        codes[k] = oracle_e4m3_code((double)v);
    }
    return s;
}

/* X [M][K] bfloat16 bit patterns -> codes [M][K] (E4M3) and sa [M][ceil(K/128)] (fp32), one scale
 * per block of 128 consecutive K values of a row (a shorter last block when K is not a multiple
 * of 128), by quantize_block on the bf16 values (|x| of a bf16 value is a bf16 value, so amax is
 * exact).  Inputs must be finite (a NaN or infinity gives unspecified codes).  Returns 0. */
ORACLE_API int oracle_quantize_1x128(const uint16_t* X, int64_t M, int64_t K, uint8_t* codes,
                                     float* sa, int nthreads) {
    int64_t nkb = (K + 127) / 128;
    int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t kb = 0; kb < nkb; ++kb) {
            int64_t k0 = kb * 128, k1 = k0 + 128 < K ? k0 + 128 : K;
            float xs[128];
            for (int64_t k = k0; k < k1; ++k) {
                uint32_t bits = (uint32_t)X[m * K + k] << 16;   /* bf16 is the top half of fp32 */
                memcpy(&xs[k - k0], &bits, sizeof bits);
            }
            float s = quantize_block(xs, k1 - k0, codes + m * K + k0);
            sa[m * nkb + kb] = s;
        }
    }
    return 0;
}

/* ---- SwiGLU and requantisation (the step between an MoE expert's two linear layers) -------- */

/* Page "Perpustakaan operator GPU sumber terbuka DeepSeek DeepGEMM memperbarui versi besar,
 * menambahkan Mega MoE…" (the Mega MoE news item): an MoE layer at inference is EP dispatch, a
 * first linear layer, SwiGLU activation, a second linear layer and EP combine.  SwiGLU is not
 * spelled out there; the reading taken is the usual one, with the first layer's output row split
 * into halves, gate = columns [0, I), up = columns [I, 2I):
 *   h = silu(gate) * up,  silu(x) = x * sigmoid(x) = x / (1 + e^-x)
 * formed in fp64 from the bf16 inputs and rounded once to fp32 (the activation handed on), then
 * quantised per block of 128 consecutive columns with quantize_block (the left operand of the
 * second layer).  X [M][2I] bf16 bit patterns -> codes [M][I], sa [M][ceil(I/128)], and the fp64
 * activations h [M][I] when h is not NULL.  Inputs must be finite with h inside the fp32 range.
 * Returns 0. */
ORACLE_API int oracle_swiglu_quantize_1x128(const uint16_t* X, int64_t M, int64_t I, uint8_t* codes,
                                            float* sa, double* h, int nthreads) {
    int64_t nkb = (I + 127) / 128;
    int nt = pick_threads(nthreads);
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t m = 0; m < M; ++m) {
        const uint16_t* gate = X + m * 2 * I;
        const uint16_t* up = gate + I;
        for (int64_t kb = 0; kb < nkb; ++kb) {
            int64_t k0 = kb * 128, k1 = k0 + 128 < I ? k0 + 128 : I;
            float xs[128];
            for (int64_t k = k0; k < k1; ++k) {
                uint32_t gb = (uint32_t)gate[k] << 16, ub = (uint32_t)up[k] << 16;
                float g, u;
                memcpy(&g, &gb, sizeof g);
                memcpy(&u, &ub, sizeof u);
                double silu = (double)g / (1.0 + exp(-(double)g));
                double v = silu * (double)u;
                if (h) h[m * I + k] = v;
                xs[k - k0] = (float)v;
            }
            sa[m * nkb + kb] = quantize_block(xs, k1 - k0, codes + m * I + k0);
        }
    }
    return 0;
}
