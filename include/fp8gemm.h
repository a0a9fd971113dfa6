/*
 * fp8gemm.h -- C ABI of the MI355X (gfx950) FP8 block-scaled GEMM library (libfp8gemm.so).
 *
 * Operation (page "DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，核心代碼僅300行", sections
 * 深入了解DeepGEMM and 如何使用？): FP8 GEMM with fine-grained scaling in NT layout (left operand
 * not transposed, right operand transposed), BF16 output, plus the two M-grouped MoE layouts
 * (contiguous and masked; also page "DeepGEMM：AI計算の経済性を変えるオープンソースライブラリ",
 * section DeepGEMMが重要な理由, item 4):
 *
 *   D[m][n] = bf16( sum_kb sa[m][kb] * sb[n/128][kb] * sum_{k in [128kb, 128kb+128)} A[m][k] * B[n][k] )
 *
 * with A, B in OCP E4M3 ("e4m3fn"), sa one fp32 scale per 1x128 block of a row of A and sb one
 * fp32 scale per 128x128 block of B.  The GPU forms each 128-wide K block's partial product on
 * the matrix cores, then scales it by sa*sb and adds it into an fp32 accumulator (the pages'
 * two-level accumulation), and rounds once to bf16 (round to nearest even).
 *
 * Conventions for every GEMM entry point:
 *   - All matrix and scale pointers are DEVICE pointers; the caller owns every buffer.
 *   - All arrays are dense with the last index contiguous:
 *       A  [rows][K] uint8 codes      sa [(G)][K/128][rows] float  (K-block-major: the scales of
 *       B  [(G)][N][K] uint8 codes        one 128-wide K block for consecutive rows are adjacent)
 *       D  [rows][N] bfloat16         sb [(G)][ceil(N/128)][K/128] float
 *     sa[kb][m] is the scale of A[m][128kb .. 128kb+127].  The pages fix no scale layout; this
 *     one lets one K block's scales for a whole tile arrive as one contiguous run (the reference
 *     library likewise asks for a specially aligned layout of its left-hand scales).  Measured
 *     on MI355X, the same kernel reading a row-major [rows][K/128] sa (a strided gather per K
 *     block) ran 2-16% slower: 4096x4096x7168 +8%, 128x7168x16384 +16%, 64x2112x7168 +2%.
 *   - K must be a positive multiple of 128; M, N may be any non-negative size (N tails are
 *     masked).  A, B and D must be 16-byte aligned; sa, sb and the index vectors 4-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls are asynchronous:
 *     they validate on the host (no device access, no synchronisation), enqueue the kernel and
 *     return.  An argument error is reported before anything is enqueued.
 *   - Results are deterministic: the same inputs give the same bits, whatever the launch
 *     configuration's timing (split-K and stream-K partials are summed in a fixed K order).
 *     The launch configuration itself depends on the shape, the device's CU count and the CU
 *     cap, so a different cap (or stream-K turned off) may sum the same products in another
 *     order, within the same tolerance.
 *   - Split-K workspace: each stream has its own library-owned workspace (fp32 partial tiles
 *     and arrival counters, CUs x 512 KiB + 16 KiB on the stream's device).  It serves the
 *     K splits of decode-sized launches and the stream-K schedule of large dense launches (the
 *     256-row tiles left over after the last full round of tiles, shared out over every CU
 *     by K block).  It is allocated once, at full size, by fp8gemm_prepare_stream or by the
 *     first call on the stream whose launch needs it (one hipMalloc pair and one blocking
 *     hipMemset), and it is never freed,
 *     moved or regrown, so a HIP graph captured on the stream stays valid for the life of the
 *     process.  Nothing is allocated while the stream is capturing: a split-K call on a stream
 *     that has no workspace yet, made during capture, returns FP8GEMM_ERR_UNSUPPORTED (a
 *     stream-K launch keeps whole tiles instead); call
 *     fp8gemm_prepare_stream before capturing (and before any capture starts in the process,
 *     since the blocking hipMemset must not run while another thread captures).  A graph uses
 *     the workspace of the stream it was captured on: its replays must not overlap each other
 *     or calls on that stream.
 *   - Thread safety: calls may come from any host thread.  Calls on different streams may run
 *     concurrently.  fp8gemm_set_num_cus is a global knob, not synchronised with calls in
 *     flight.
 *   - Environment (read at each call; for experiments and tests, not needed in normal use):
 *     FP8GEMM_FORCE_CONFIG forces a table entry (BMxBN:WMxWN:STAGES:SPLIT for the tiled kernel,
 *     stream:MT:W:JN:KP:PF:SPLIT for the masked decode kernel), FP8GEMM_STREAMK=0 or 1 turns
 *     stream-K off, or on wherever dense 256-row tiles leave a partial round, and FP8GEMM_LOG
 *     prints each launch configuration to stderr.  FP8GEMM_HIPRTC names the hipRTC library for
 *     the run-time specialised kernels (default $ROCM_PATH/lib/libhiprtc.so.7).
 *
 * Return value of every int function: a fp8gemm_status code.
 */
#ifndef FP8GEMM_H
#define FP8GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp8gemm_status {
    FP8GEMM_OK = 0,
    FP8GEMM_ERR_NULL_PTR = 1,    /* a required pointer is NULL */
    FP8GEMM_ERR_BAD_SHAPE = 2,   /* negative size, K not a positive multiple of 128, G <= 0, expected_m < 0 */
    FP8GEMM_ERR_MISALIGNED = 3,  /* A, B or D not 16-byte aligned, or a scale/index vector not 4-byte aligned */
    FP8GEMM_ERR_UNSUPPORTED = 4, /* a size beyond the supported range (an operand of 2^40 bytes or more, K > 2^24,
                                    2^30 or more output tiles x K splits in one launch, 2^31 or more
                                    128-value blocks in one quantiser call, a forced launch shape whose
                                    split-K partials exceed the stream's workspace), or a split-K call
                                    on an unprepared stream during graph capture */
    FP8GEMM_ERR_LAUNCH = 5,      /* the HIP launch failed (hipGetLastError after the launch) */
    FP8GEMM_ERR_HIP = 6          /* a HIP runtime call failed (device query, workspace allocation, copy) */
} fp8gemm_status;

/* Dense NT GEMM, gemm_fp8_fp8_bf16_nt (page "DeepSeek開源第三彈…", section 如何使用？).
 *   A [M][K] e4m3, sa [K/128][M], B [N][K] e4m3, sb [ceil(N/128)][K/128], D [M][N] bf16.
 *   M == 0 or N == 0 is a valid no-op. */
int fp8gemm_nt(const void* A, const float* sa, const void* B, const float* sb, void* D,
               int64_t M, int64_t N, int64_t K, void* stream);

/* fp8gemm_nt for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The same operation, arguments,
 * validation, launch shape and results (bit for bit) as fp8gemm_nt, but the split-K partial tiles
 * and arrival counters live in a static device array of the library (16 MiB of fp32 partials and
 * 4096 counters per GPU, held until the process ends) instead of a per-stream workspace, and the
 * call allocates nothing, ever, and never synchronises.  A launch whose partials or tiles exceed
 * that array returns FP8GEMM_ERR_UNSUPPORTED before enqueueing anything; every automatically
 * chosen dense launch on up to 256 CUs fits.  All calls of this entry point on one GPU share the
 * array: calls whose kernels overlap in time on the same GPU (on different streams, or graphs
 * replayed concurrently) race on it and give unspecified results; serialise them.  The arrival
 * counters start at zero when the library's code object is loaded and every launch leaves them
 * at zero; the partials are written before they are read. */
int fp8gemm_nt_noalloc(const void* A, const float* sa, const void* B, const float* sb, void* D,
                       int64_t M, int64_t N, int64_t K, void* stream);

/* M-grouped GEMM, contiguous layout, m_grouped_gemm_fp8_fp8_bf16_nt_contiguous (same page and
 * section; page "DeepGEMM：AI計算の経済性を…", section DeepGEMMが重要な理由: token sequences are
 * grouped per expert).  The rows of all groups are concatenated along M:
 *   A [M_total][K], sa [K/128][M_total], B [G][N][K], sb [G][ceil(N/128)][K/128],
 *   m_indices [M_total] int32 (device): row r is multiplied by B[m_indices[r]];
 *   m_indices[r] == -1 marks a padding row, whose D row is left untouched.
 *   D [M_total][N].
 * Precondition: within each aligned block of 128 rows all rows that are not -1 carry the same
 * group id (groups are padded to multiples of 128 rows).  A row whose id is outside [-1, G), or
 * differs from the id of its 128-row block, is treated as padding and flags
 * FP8GEMM_DEVERR_BAD_INDEX in the device error word (see fp8gemm_read_device_error). */
int fp8gemm_grouped_contiguous(const void* A, const float* sa, const void* B, const float* sb,
                               const int32_t* m_indices, void* D, int64_t M_total, int64_t N,
                               int64_t K, int32_t G, void* stream);

/* M-grouped GEMM, masked layout, m_grouped_gemm_fp8_fp8_bf16_nt_masked (same page and section;
 * page "DeepGEMM：AI計算の経済性を…", section DeepGEMMが重要な理由: sparse expert activation).
 * Every group owns a fixed block of M_max rows:
 *   A [G][M_max][K], sa [G][K/128][M_max], B [G][N][K], sb [G][ceil(N/128)][K/128],
 *   masked_m [G] int32 (device): rows r < masked_m[g] of group g are valid; D rows at or past it
 *   are left untouched.  A count above M_max is clamped to M_max and flags
 *   FP8GEMM_DEVERR_BAD_COUNT; a negative count is taken as 0 and flags it too.
 *   expected_m >= 0: a hint of the typical masked_m, used only to pick the launch shape;
 *   it never changes results.  D [G][M_max][N]. */
int fp8gemm_grouped_masked(const void* A, const float* sa, const void* B, const float* sb,
                           const int32_t* masked_m, void* D, int32_t G, int64_t M_max, int64_t N,
                           int64_t K, int64_t expected_m, void* stream);

/* M-grouped GEMM, masked layout, with B in 4-bit floating point: the FP8 x FP4 mixed precision of
 * page "Perpustakaan operator GPU sumber terbuka DeepSeek DeepGEMM memperbarui versi besar,
 * menambahkan Mega MoE…" (Mega MoE supports only the FP8 x FP4 combination; FP8 x FP4 matrix
 * multiplication is listed among the additions).  The pages give no FP4 element or scale format;
 * the reading taken is OCP MXFP4 for B and the FP8 left operand of fp8gemm_grouped_masked:
 *   A [G][M_max][K] e4m3 codes, sa [G][K/128][M_max] fp32 (as fp8gemm_grouped_masked),
 *   B [G][N][K/2] bytes: E2M1 codes (1 sign, 2 exponent bits with bias 1, 1 mantissa bit:
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), two per byte, element k of a row in byte
 *     k/2, the even element in the low nibble,
 *   sb [G][N][K/32] uint8: E8M0 scales (value 2^(s - 127); 255 is NaN and gives unspecified
 *     results), one per 32 consecutive K values of a row of B,
 *   D[g][m][n] = bf16( sum_kb sa[g][kb][m] * sum_{k in block kb} e4m3(A) * e2m1(B) * 2^(sb - 127) ),
 *   masked_m, expected_m and D as fp8gemm_grouped_masked.  K: a positive multiple of 128; B, A
 *   and D 16-byte aligned, sa, sb and masked_m 4-byte aligned.  The 32-value scales are applied
 *   inside the matrix-core instruction; the fresh fp32 partial of each 128-wide K block is then
 *   scaled by sa and accumulated in fp32 (the two-level accumulation). */
int fp8gemm_fp8fp4_grouped_masked(const void* A, const float* sa, const void* B, const uint8_t* sb,
                                  const int32_t* masked_m, void* D, int32_t G, int64_t M_max, int64_t N,
                                  int64_t K, int64_t expected_m, void* stream);

/* Activation quantiser, 1x128 blocks: the step that produces the left operand and its scales.
 * The pages take fine-grained scaling from DeepSeek V3 (page "DeepSeek開源第三彈…", section
 * 深入了解DeepGEMM) and give no quantiser; this one is the plain reading of a 1x128 block scale.
 * For every block of 128 consecutive K values of a row of X:
 *   amax = max |x| over the block, floored at fp32(1e-4) (an all-zero block keeps a finite scale)
 *   s    = fp32(amax / 448)                   (448: the largest finite E4M3 value)
 *   code = E4M3 round-to-nearest-even of fp32(x / s), saturated to +-448
 * so the largest element of every block is coded +-448 and code * s approximates x.
 *   X  [M][K] bfloat16 (device), A [M][K] e4m3 codes (device, written), sa [K/128][M] fp32
 *   (device, written; the K-block-major scale layout fp8gemm_nt and fp8gemm_grouped_contiguous
 *   read).  K: positive multiple of 128 (else FP8GEMM_ERR_BAD_SHAPE); M == 0 is a no-op.
 *   X and A 16-byte aligned, sa 4-byte aligned (else FP8GEMM_ERR_MISALIGNED).  X must hold
 *   finite values: a NaN or infinity gives unspecified codes and scales for its block. */
int fp8gemm_quantize_1x128(const void* X, void* A, float* sa, int64_t M, int64_t K, void* stream);

/* The same quantiser for the masked layout (see fp8gemm_grouped_masked): X and A [G][M_max][K],
 * sa [G][K/128][M_max], masked_m [G] int32 (device).  Rows r < masked_m[g] of group g are
 * quantised; A and sa entries of the rows at or past it are left untouched.  A count outside
 * [0, M_max] is clamped and flags FP8GEMM_DEVERR_BAD_COUNT.  G <= 0 is FP8GEMM_ERR_BAD_SHAPE. */
int fp8gemm_quantize_1x128_masked(const void* X, void* A, float* sa, const int32_t* masked_m,
                                  int32_t G, int64_t M_max, int64_t K, void* stream);

/* SwiGLU activation and requantisation: the step between the two linear layers of an MoE
 * expert (page "Perpustakaan operator GPU sumber terbuka DeepSeek DeepGEMM memperbarui versi
 * besar, menambahkan Mega MoE…": an MoE layer at inference is EP dispatch, first linear layer,
 * SwiGLU activation, second linear layer, EP combine).  The pages do not spell SwiGLU out; the
 * reading taken is the usual one:
 *   X [M][2I] bfloat16 (device): the first layer's output, gate in columns [0, I), up projection
 *   in columns [I, 2I);  h = silu(gate) * up with silu(x) = x / (1 + e^-x), formed in fp32;
 * then the 1x128 quantiser above on h (fp32 values instead of bf16):
 *   A [M][I] e4m3 codes (device, written), sa [I/128][M] fp32 (device, written) -- the left
 *   operand of the second layer.  I: positive multiple of 128 (else FP8GEMM_ERR_BAD_SHAPE).
 *   X and A 16-byte aligned, sa 4-byte aligned.  Inputs must be finite, with silu(gate) * up
 *   inside the fp32 range; otherwise the codes and scale of that block are unspecified. */
int fp8gemm_swiglu_quantize_1x128(const void* X, void* A, float* sa, int64_t M, int64_t I, void* stream);

/* The same for the masked layout: X [G][M_max][2I], A [G][M_max][I], sa [G][I/128][M_max],
 * masked_m [G] int32 (device); rows at or past masked_m[g] are left untouched; a count outside
 * [0, M_max] is clamped and flags FP8GEMM_DEVERR_BAD_COUNT. */
int fp8gemm_swiglu_quantize_1x128_masked(const void* X, void* A, float* sa, const int32_t* masked_m,
                                         int32_t G, int64_t M_max, int64_t I, void* stream);

/* One MoE expert layer per group on the masked layout (same page: the first linear layer,
 * SwiGLU and the second linear layer; dispatch and combine are not part of it):
 *   Y1  = grouped_masked(A, sa, W1, s1)            Y1 [G][M_max][2I] bf16   (first layer)
 *   Hq, sh = swiglu_quantize_1x128_masked(Y1)      Hq [G][M_max][I] e4m3, sh [G][I/128][M_max]
 *   out = grouped_masked(Hq, sh, W2, s2)           out [G][M_max][H] bf16   (second layer)
 * with A [G][M_max][H], sa [G][H/128][M_max], W1 [G][2I][H], s1 [G][2I/128][H/128],
 * W2 [G][H][I], s2 [G][H/128][I/128].  Y1, Hq and sh are caller-owned workspaces (device),
 * nothing is allocated.  H and I: positive multiples of 128.  Every argument of the three steps
 * is checked before anything is enqueued; the three launches follow each other on `stream`.
 * Rows at or past masked_m[g] of Y1, Hq, sh and out are left untouched. */
int fp8gemm_moe_expert_masked(const void* A, const float* sa, const void* W1, const float* s1,
                              const void* W2, const float* s2, const int32_t* masked_m, void* Y1,
                              void* Hq, float* sh, void* out, int32_t G, int64_t M_max, int64_t H,
                              int64_t I, int64_t expected_m, void* stream);

/* Device-side precondition flags (bits of the device error word). */
#define FP8GEMM_DEVERR_BAD_INDEX 1 /* contiguous: an m_indices entry outside [-1, G) or off its block's group */
#define FP8GEMM_DEVERR_BAD_COUNT 2 /* masked GEMM or quantiser: a masked_m entry outside [0, M_max] */

/* Human-readable name of a status code (static storage; never NULL). */
const char* fp8gemm_status_string(int status);

/* Optional eager set-up on the current device: device query and the device error word.  The
 * GEMM calls do it lazily otherwise.  Returns FP8GEMM_ERR_HIP when no device is usable. */
int fp8gemm_init(void);

/* Create `stream`'s split-K workspace now, on the current device (see "Split-K workspace" above),
 * so that later calls on the stream, captured in HIP graphs or not, allocate nothing.  Calling it
 * again for a prepared stream does nothing.  Not while any stream of the process is capturing.
 * Returns FP8GEMM_ERR_HIP if the allocation fails, FP8GEMM_ERR_UNSUPPORTED if `stream` is
 * capturing. */
int fp8gemm_prepare_stream(void* stream);

/* Run-time shape specialisation (the pages' JIT idea: every kernel compiled at run time with
 * the block sizes and stages chosen for the shape, page "DeepSeek開源第三彈…", sections
 * 深入了解DeepGEMM and 如何使用？).  The launch shape stays the table's choice; the tiled kernel
 * is compiled with hipRTC for gfx950 with N and K as compile-time constants, loaded as a module
 * on the current device and cached there for the life of the process (keyed by table entry, N
 * and K).  Nothing is written to disk.
 *
 * fp8gemm_nt_specialized: the same operation, arguments, validation and results as fp8gemm_nt
 *   (the same bits: the kernel body and its arithmetic order are identical).  The first call for
 *   a new (launch shape, N, K) on a device compiles the kernel on the calling thread (a few
 *   hundred milliseconds, serialised across threads) before enqueueing; later calls only launch.
 *   A failed compile or module load returns FP8GEMM_ERR_HIP (the compiler log goes to stderr).
 *   Not for HIP graph capture until the kernel is cached (call fp8gemm_specialize_nt first). */
int fp8gemm_nt_specialized(const void* A, const float* sa, const void* B, const float* sb, void* D,
                           int64_t M, int64_t N, int64_t K, void* stream);

/* Compile and load, ahead of use, the kernel fp8gemm_nt_specialized would run for (M, N, K)
 * on the current device.  *compile_ms (if not NULL) receives the compile + load time in
 * milliseconds, or 0 when the kernel was already cached.  M, N > 0; K as for fp8gemm_nt. */
int fp8gemm_specialize_nt(int64_t M, int64_t N, int64_t K, double* compile_ms);

/* The gfx950 code object of the tiled table entry (layout 0 dense, 1 contiguous, 2 masked;
 * tile bm x bn, waves_m x waves_n waves, `stages` ring stages) specialised to (N, K), for
 * inspection; no GPU is needed.  *size: in, the capacity of buf (bytes); out, the code object's
 * size.  buf == NULL queries the size only.  log (log_len bytes, may be NULL) receives the
 * kernel's symbol name, or the compiler log on failure.  An entry not in the table, N <= 0 or a
 * bad K is FP8GEMM_ERR_BAD_SHAPE, as is a buffer too small; a compile failure FP8GEMM_ERR_HIP. */
int fp8gemm_specialized_code_object(int layout, int bm, int bn, int waves_m, int waves_n, int stages,
                                    int64_t N, int64_t K, void* buf, size_t* size, char* log, int log_len);

/* Number of specialised kernels cached in this process (all devices). */
int fp8gemm_specialized_count(void);

/* Cap the number of compute units the launch shapes are sized for and the persistent grids
 * occupy (the "set max SM count" utility of page "DeepSeek開源第三彈…", section 如何使用？).
 * n == 0 restores all CUs; n < 0 is FP8GEMM_ERR_BAD_SHAPE. */
int fp8gemm_set_num_cus(int n);

/* The launch configuration chosen by the last GEMM call on the calling host thread, as text
 * (e.g. "nt tile=256x256 waves=4x2 stages=2 split=1 grid=256"), NUL-terminated into buf[len].
 * Returns FP8GEMM_ERR_NULL_PTR when buf is NULL or len <= 0. */
int fp8gemm_last_config(char* buf, int len);

/* Synchronise `stream`, then read and clear the current device's error word into *err
 * (FP8GEMM_DEVERR_* bits; 0 when every index and count met the preconditions). */
int fp8gemm_read_device_error(void* stream, int32_t* err);

#ifdef __cplusplus
}
#endif

#endif /* FP8GEMM_H */
