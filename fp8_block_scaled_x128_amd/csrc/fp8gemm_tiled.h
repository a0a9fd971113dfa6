// fp8gemm_tiled.h -- the tiled gfx950 kernel body of the FP8 block-scaled GEMM.  Included by the
// ahead-of-time build (fp8gemm_kernels.hip, N and K as arguments) and compiled at run time with
// N and K fixed (fp8gemm_jit.cpp).
//
// One kernel body serves the dense NT GEMM and the two M-grouped MoE layouts (page
// "DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，核心代碼僅300行", sections 深入了解DeepGEMM and
// 如何使用？: a single core kernel, fine-grained scaling, two-level accumulation; NT layout;
// contiguous and masked grouped variants).
//
// Per work unit (an output tile, for one K range) a workgroup
//   1. streams 128-wide K slices of the B tile, the A tile and their scales from HBM into an
//      LDS ring with direct-to-LDS DMA loads (global_load_lds_dword[x4]), STAGES slices ahead;
//   2. per slice and per 16x16 sub-tile issues ONE v_mfma_f32_16x16x128_f8f6f4 with a zero
//      accumulator input, so the matrix core returns the fresh fp32 partial of exactly that
//      128-wide block (the FP8 matrix-core sum is not exact fp32, so the partial is kept short);
//   3. promotes the partial: acc += partial * (sa[m][kb] * sb[n/128][kb]) with VALU FMAs in
//      fp32 -- the pages' two-level accumulation, re-derived for MFMA;
//   4. rounds acc once to bf16 (round to nearest even) and stores D, or, when the K range is
//      split across workgroups, writes its fp32 partial tile to a workspace; the last workgroup
//      of the tile to arrive sums all partials in split order and stores D.
//
// MFMA orientation: the matrix core computes C[i][j] = sum_k X[i][k] Y[j][k] with lane l
// holding X row (l % 16), Y row (l % 16) and output column (l % 16), rows 4*(l/16)..+3.  The
// kernel feeds B rows as X and A rows as Y, so every lane owns 4 consecutive n of one m: the
// promotion scale sa[m]*sb[n/128] is one value per lane per sub-tile and the bf16 results of a
// lane are contiguous in D.  Both operands give lane l the K bytes [32*(l/16), +32) of the
// slice, in the same order (the hardware pairs equal positions of X and Y).
//
// LDS layout of one slice: rows of 128 bytes, 16-byte chunk c of row r stored at chunk
// position c ^ s(r) with s(r) = (r>>1 & 3) | ((r>>2 ^ r>>3) & 1) << 2.  A fragment read
// (ds_read_b128, lane l: row l%16, chunk 2*(l/16)+h) is served 16 lanes per LDS cycle; measured
// on gfx950, the lanes served together are those of one half-wave with equal parity of lane
// bits 2..4.  The permutation gives those 16 lanes 16 distinct 16-byte bank groups of the
// 256-byte-wide LDS (it is also conflict-free for runs of 8 or 16 consecutive lanes), so a
// fragment read runs at the full ds_read_b128 rate; the DMA writes are contiguous 1 KB runs.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8gemm_args.h"
#include "fp8gemm_device.h"

namespace fp8gemm {

// Chunk permutation of a 128-byte LDS row (see the layout note at the top of the file).
__device__ __forceinline__ int swz(int row) {
    return ((row >> 1) & 3) | ((((row >> 2) ^ (row >> 3)) & 1) << 2);
}

// ------------------------------------------------------------------------------------------
// the kernel
// ------------------------------------------------------------------------------------------

template <int BM, int BN, int WMW, int WNW, int STAGES, int LAYOUT>
struct Tile {
    static constexpr int NW = WMW * WNW;            // waves per workgroup
    static constexpr int NT = 64 * NW;
    static constexpr int WM = BM / WMW;             // rows of M per wave
    static constexpr int WN = BN / WNW;             // rows of N per wave
    static constexpr int JM = WM / 16;              // 16-wide M sub-tiles per wave
    static constexpr int IN = WN / 16;              // 16-wide N sub-tiles per wave
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(BN % 8 == 0 && BM % (8 * NW) == 0, "whole 8-row groups; every wave moves the same A rows count");
    static_assert(BM % 64 == 0, "scale rows of A are moved 64 at a time");
    static constexpr int B_OFF = 0;
    static constexpr int A_OFF = BN * 128;
    static constexpr int SA_OFF = (BN + BM) * 128;
    static constexpr int SB_OFF = SA_OFF + BM * 4;
    static constexpr int STAGE_BYTES = SB_OFF + 256;
    static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    // x4 loads per wave per slice for B; when the BN/8 row groups do not split evenly over the
    // waves, the spare slots repeat the last group (the same bytes to the same LDS rows), so every
    // wave issues the same number of loads and waits with the same counts
    static constexpr int B_GROUPS = BN / 8;
    static constexpr int B_DMA = (B_GROUPS + NW - 1) / NW;
    static constexpr int A_DMA = BM / (8 * NW);
    static constexpr int AUX = (BM / 64 + 1 + NW - 1) / NW;  // x1 loads per wave: sa chunks + sb
    static constexpr int NDMA = B_DMA + A_DMA + AUX;          // loads per wave per slice
    static_assert(NDMA * (STAGES - 1) < 64, "vmcnt range");
    // every wave's N range lies inside one 128-row block of B scales
    static constexpr bool NB_UNIFORM = (BN % 128 == 0) && (128 % WN == 0);
    // K slices consumed per workgroup barrier.  Deep rings (5 or more stages, the decode tiles)
    // take two: one barrier per pair, both slices' fragment reads issued together, then all their
    // MFMAs, then the promotions in slice order (the same arithmetic order as one at a time).
    static constexpr int SPB = STAGES >= 5 ? 2 : 1;
    static_assert(SPB == 1 || IN <= 2, "paired slices: decode tiles (at most two N sub-tiles per wave)");
    // split-K partial reduction is compiled for tiles small enough to need it (decode shapes)
    static constexpr bool SPLITK = BM * BN <= 128 * 256;
    // the dense 256-row tiles take leftover tiles stream-K (after the last full round of tiles)
    static constexpr bool STREAMK = LAYOUT == kDense && BM == 256;
    // Epilogue staging: each wave writes its WM x WN bf16 results row-major into a private LDS
    // region (after the K loop, over the ring), then stores whole 16-byte chunks of rows.  The
    // row pitch holds an odd number of 16-byte units, so the 8-byte writes of 32 lanes in the
    // MFMA layout (16 rows x 2 column groups) fall into 64 distinct banks.
    static_assert(WM <= 64, "row mask: one bit per row of a wave's slab");
    static_assert(WN % 8 == 0, "16-byte chunks of a wave's rows");
    static constexpr int ROW_BYTES = 2 * WN;
    static constexpr int CPR = ROW_BYTES / 16;                  // 16-byte chunks per row
    static constexpr int PITCH = ROW_BYTES + ((CPR % 2 == 0) ? 16 : 0);
    static constexpr int STG_WAVE_BYTES = WM * PITCH;
    static constexpr int STORES = (WM * CPR + 63) / 64;         // store instructions per wave
    static constexpr int SMEM_BYTES = LDS_BYTES > NW * STG_WAVE_BYTES ? LDS_BYTES : NW * STG_WAVE_BYTES;
    static_assert(SMEM_BYTES <= 160 * 1024, "LDS budget (staging)");
};

// NC, KC > 0 fix N and K at compile time (the run-time specialised variant); 0 reads them from
// the arguments.
template <int BM, int BN, int WMW, int WNW, int STAGES, int LAYOUT, int NC = 0, int KC = 0>
__global__ __launch_bounds__(WMW * WNW * 64) void fp8gemm_kernel(const KernelArgs args) {
    using T = Tile<BM, BN, WMW, WNW, STAGES, LAYOUT>;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::SMEM_BYTES];
    __shared__ int s_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WMW;              // wave position along M
    const int wn = wave / WMW;              // wave position along N
    const int row16 = lane & 15;
    const int grp = lane >> 4;
    // every fragment row a lane reads is row16 plus a multiple of 16, so its two 16-byte chunks
    // sit at the same swizzled positions in every row
    const int frag_lo = ((2 * grp) ^ swz(row16)) << 4;
    const int frag_hi = ((2 * grp + 1) ^ swz(row16)) << 4;

    static_assert(KC % 128 == 0 && NC >= 0, "compile-time K is a multiple of 128");
    const int K = KC > 0 ? KC : args.K;
    const int N = NC > 0 ? NC : args.N;
    const int nkb = KC > 0 ? KC / 128 : args.nkb;
    const int nnb = NC > 0 ? (NC + 127) / 128 : args.nnb;
    const uint32_t smem_base = lds_addr(smem);

    // XCD-aware order: workgroups are dealt to the 8 XCDs round robin, so give the workgroups
    // of one XCD a contiguous range of logical ids (consecutive units share operand panels).
    const int P = gridDim.x;
    int logical = blockIdx.x;
    if ((P & 7) == 0) logical = (blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3);

    // Units [0, units) are whole tiles (or K splits of them); with stream-K each workgroup then
    // takes two more iterations over its segments of the leftover tiles, segment 1 first (either
    // may be empty).  Segment 1 starts at a tile's first K block and segment 0, when the range
    // crosses a tile boundary, ends at a tile's last one, so in this order every workgroup of
    // such a schedule reads K block j or j + (K blocks per tile - blocks per workgroup) at step j:
    // two K phases, which the workgroups of an XCD share through L2 (in range order they would
    // run at up to four).  The run-time specialised variants (N or K fixed) keep whole tiles:
    // with N fixed the compiler keeps more values live and the exchange code would spill.
    constexpr bool SK = T::STREAMK && NC == 0 && KC == 0;
    const int sk_iters = (SK && args.sk_tiles > 0) ? 2 * P : 0;
    for (int unit = logical; unit < args.units + sk_iters; unit += P) {
        // ---- a stream-K segment: K blocks [sk_kb0, sk_kb0 + sk_nks) of leftover tile sk_tile --
        const bool sk = SK && unit >= args.units;
        const int sk_seg = sk ? 1 - (unit - args.units) / P : 0;
        int sk_tile = 0, sk_kb0 = 0, sk_nks = 0;
        if (sk) {
            const int r0 = sk_start(logical, args.sk_per, args.sk_extra);
            const int r1 = sk_start(logical + 1, args.sk_per, args.sk_extra);
            const int g = sk_seg == 0 ? r0 : (r0 / nkb + 1) * nkb;      // segment 1: the next tile's start
            if (g >= r1) continue;                                       // uniform: no such segment
            sk_tile = g / nkb;
            sk_kb0 = g - sk_tile * nkb;
            sk_nks = min(nkb - sk_kb0, r1 - g);
        }
        // ---- decode the unit: split s fastest, then M tile, N tile, group -------------------
        // (uniform integer work on the scalar unit: multiply-shift divisions by launch constants)
        uint32_t u = (uint32_t)unit;
        const uint32_t tile_id = sk ? (uint32_t)(args.units + sk_tile) : fast_div(u, args.div_splits);
        const int split = sk ? 0 : (int)(u - tile_id * (uint32_t)args.splits);
        u = tile_id;
        int tm, tn;
        if (args.group_m > 1) {
            // bands of group_m M tiles; inside a band the M tile varies fastest
            const uint32_t grp_i = fast_div(u, args.div_group_tiles);
            const uint32_t v = u - grp_i * args.div_group_tiles.d;
            const uint32_t band = fast_div(v, args.div_band_units);
            const uint32_t inb = v - band * args.div_band_units.d;
            const int band_m0 = (int)band * args.group_m;
            const bool full = band_m0 + args.group_m <= args.tiles_m;
            const FastDiv& bh = full ? args.div_band_h : args.div_band_h_last;
            const uint32_t q = fast_div(inb, bh);
            tm = band_m0 + (int)(inb - q * bh.d);
            tn = (int)q;
            u = grp_i;
        } else {
            const uint32_t q = fast_div(u, args.div_tiles_m);
            tm = (int)(u - q * (uint32_t)args.tiles_m);
            u = q;
            const uint32_t q2 = fast_div(u, args.div_tiles_n);
            tn = (int)(u - q2 * (uint32_t)args.tiles_n);
            u = q2;
        }
        const int gidx = (int)u;                       // group (masked layout), else 0
        const int m0 = tm * BM;                        // first row of the tile (within group)
        const int n0 = tn * BN;
        const int kb0 = sk ? sk_kb0 : split * args.kb_per_split;
        const int kb1 = sk ? sk_kb0 + sk_nks : min(nkb, kb0 + args.kb_per_split);
        const int nks = kb1 - kb0;

        // ---- rows of A, group of B ---------------------------------------------------------
        int64_t arow0;        // first row of A / sa / D for this tile
        int row_limit;        // rows [0, row_limit) of the tile are in range of the A array
        int valid_rows;       // rows [0, valid_rows) may be valid (contiguous: further masked)
        int g = 0;
        int g_second = -1;    // contiguous 256-row tiles: the second 128-row block's group when it differs
        if constexpr (LAYOUT == kMasked) {
            g = gidx;
            int cnt = args.masked_m[g];
            if (cnt < 0 || cnt > args.rows) {
                if (tm == 0 && tn == 0 && split == 0 && tid == 0)
                    atomicOr(args.err, kDevErrBadCount);
                cnt = cnt < 0 ? 0 : (int)args.rows;
            }
            if (m0 >= cnt) continue;                   // uniform: whole workgroup skips
            arow0 = (int64_t)g * args.rows + m0;
            row_limit = (int)min((int64_t)BM, args.rows - m0);
            valid_rows = min(BM, cnt - m0);
        } else if constexpr (LAYOUT == kContiguous) {
            arow0 = m0;
            row_limit = (int)min((int64_t)BM, args.rows - m0);
            // the group of each 128-row block of the tile: the largest id among its rows; any row
            // whose id is neither -1 nor its block's group breaks the precondition
            constexpr int NBLK = BM > 128 ? BM / 128 : 1;
            int gblk[NBLK];
            int bad = 0;
#pragma unroll
            for (int h = 0; h < NBLK; ++h) {
                const int r0 = h * 128, r1 = min(row_limit, r0 + min(BM, 128));
                int gmax = -1;
                for (int r = r0 + lane; r < r1; r += 64) {
                    const int id = args.m_indices[arow0 + r];
                    if (id < -1 || id >= args.G) bad = 1;
                    else gmax = max(gmax, id);
                }
                gmax = __builtin_amdgcn_readfirstlane(wave_max(gmax));
                for (int r = r0 + lane; r < r1; r += 64) {
                    const int id = args.m_indices[arow0 + r];
                    if (id >= 0 && id < args.G && id != gmax) bad = 1;
                }
                gblk[h] = gmax;
            }
            bad = __builtin_amdgcn_readfirstlane(wave_max(bad));
            if (bad && wave == 0 && lane == 0 && split == 0 && tn == 0) atomicOr(args.err, kDevErrBadIndex);
            // one pass when the blocks share a group (or one is padding only), else one per group;
            // each pass stores only the rows of its own group
            g = gblk[0];
            if constexpr (NBLK == 2) {
                if (g < 0) g = gblk[1];
                else if (gblk[1] >= 0 && gblk[1] != g) g_second = gblk[1];
            }
            if (g < 0) continue;                       // padding only: nothing to compute
            valid_rows = row_limit;
        } else {
            arow0 = m0;
            row_limit = (int)min((int64_t)BM, args.rows - m0);
            valid_rows = row_limit;
        }
        (void)valid_rows;
        (void)g_second;
        const uint8_t* Ag = args.A + arow0 * K;
        // sa is stored K-block-major: [group][K/128][rows], so the scales of one K block for
        // consecutive rows are contiguous (one DMA instruction covers 64 rows)
        int64_t sa_first = arow0;                     // element (kb, r) of the group: kb*rows + r
        if constexpr (LAYOUT == kMasked) sa_first = (int64_t)g * nkb * args.rows + m0;
        const float* sag = args.sa + sa_first;
        const int nb_first = n0 >> 7;
        for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1) {
            if (g_second < 0) break;
            g = g_second;
        }
        const uint8_t* Bg = args.B + (int64_t)g * N * K;
        const float* sbg = args.sb + (int64_t)g * nnb * nkb;
        const int nb_count = min(nnb, (n0 + BN + 127) >> 7) - nb_first;

        // ---- per-lane DMA source offsets (32-bit, relative to uniform per-slice bases) -------
        // B and A: x4 load q of wave w covers tile rows 8 (w count + q) .. + 7; lane -> (row, chunk)
        auto b_row = [&](int q) -> int { return 8 * min(wave * T::B_DMA + q, T::B_GROUPS - 1); };
        uint32_t b_off[T::B_DMA];
#pragma unroll
        for (int q = 0; q < T::B_DMA; ++q) {
            const int r = b_row(q) + (lane >> 3);
            const int c = (lane & 7) ^ swz(r);
            const int n = min(r, N - 1 - n0);          // clamp the N tail to a real row
            b_off[q] = (uint32_t)n * (uint32_t)K + (uint32_t)(c * 16);
        }
        uint32_t a_off[T::A_DMA];
#pragma unroll
        for (int q = 0; q < T::A_DMA; ++q) {
            const int r = 8 * (wave * T::A_DMA + q) + (lane >> 3);
            const int c = (lane & 7) ^ swz(r);
            const int rr = min(r, row_limit - 1);
            a_off[q] = (uint32_t)rr * (uint32_t)K + (uint32_t)(c * 16);
        }
        // aux x1 loads: chunk x < BM/64 moves sa rows 64x..64x+63, chunk BM/64 moves sb
        uint32_t aux_off[T::AUX];
#pragma unroll
        for (int t = 0; t < T::AUX; ++t) {
            const int x = wave + T::NW * t;
            if (x < BM / 64) {
                const int r = min(64 * x + lane, row_limit - 1);
                aux_off[t] = (uint32_t)r * 4u;
            } else {
                const int nb = nb_first + min(lane, nb_count - 1);
                aux_off[t] = (uint32_t)nb * (uint32_t)nkb * 4u;
            }
        }
        const uint8_t* Bt = uniform_ptr(Bg + (int64_t)n0 * K + (int64_t)kb0 * 128);  // slice-0 bases
        const uint8_t* At = uniform_ptr(Ag + (int64_t)kb0 * 128);
        const float* sat = uniform_ptr(sag + (int64_t)kb0 * args.rows);
        const float* sbt = uniform_ptr(sbg + kb0);

        auto stage_addr = [&](int i) { return smem_base + (uint32_t)((i % STAGES) * T::STAGE_BYTES); };
        // B loads q in [q0, q1) of slice i
        auto issue_b = [&](int i, int q0, int q1) {
            const uint32_t st = stage_addr(i);
            const uint8_t* bs = uniform_ptr(Bt + (int64_t)i * 128);
#pragma unroll
            for (int q = 0; q < T::B_DMA; ++q)
                if (q >= q0 && q < q1) dma_x4(st + T::B_OFF + b_row(q) * 128, bs, b_off[q]);
        };
        // A tile and scale loads of slice i
        auto issue_a = [&](int i) {
            const uint32_t st = stage_addr(i);
            const uint8_t* as = uniform_ptr(At + (int64_t)i * 128);
#pragma unroll
            for (int q = 0; q < T::A_DMA; ++q)
                dma_x4(st + T::A_OFF + 8 * (wave * T::A_DMA + q) * 128, as, a_off[q]);
#pragma unroll
            for (int t = 0; t < T::AUX; ++t) {
                const int x = wave + T::NW * t;
                if (x < BM / 64) dma_x1(st + T::SA_OFF + 256 * x, uniform_ptr(sat + (int64_t)i * args.rows), aux_off[t]);
                else dma_x1(st + T::SB_OFF, uniform_ptr(sbt + i), aux_off[t]);
            }
        };

        // ---- accumulators -------------------------------------------------------------------
        v4f acc[T::IN][T::JM];
#pragma unroll
        for (int i = 0; i < T::IN; ++i)
#pragma unroll
            for (int j = 0; j < T::JM; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

        // ---- one 128-wide K slice on the matrix cores ---------------------------------------
        auto compute_slice = [&](int i) {
            const uint8_t* st = smem + (i % STAGES) * T::STAGE_BYTES;
            const float* sa_l = reinterpret_cast<const float*>(st + T::SA_OFF);
            const float* sb_l = reinterpret_cast<const float*>(st + T::SB_OFF);
            auto load_bf = [&](int i2) {
                const int r = wn * T::WN + 16 * i2 + row16;
                const uint8_t* rp = st + T::B_OFF + r * 128;
                const v4i lo = *reinterpret_cast<const v4i*>(rp + frag_lo);
                const v4i hi = *reinterpret_cast<const v4i*>(rp + frag_hi);
                return (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            };
            // A fragments (Y operand) and their scales for this wave's JM sub-tiles
            v8i af[T::JM];
            float sav[T::JM];
#pragma unroll
            for (int j = 0; j < T::JM; ++j) {
                const int r = wm * T::WM + 16 * j + row16;
                const uint8_t* rp = st + T::A_OFF + r * 128;
                const v4i lo = *reinterpret_cast<const v4i*>(rp + frag_lo);
                const v4i hi = *reinterpret_cast<const v4i*>(rp + frag_hi);
                af[j] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                sav[j] = sa_l[r];
            }
            float sw[T::JM];
            if constexpr (T::NB_UNIFORM) {
                const float sbw = sb_l[((n0 + wn * T::WN) >> 7) - nb_first];
#pragma unroll
                for (int j = 0; j < T::JM; ++j) sw[j] = sav[j] * sbw;
            }
            v8i bf = load_bf(0);
            auto promote = [&](int i2, const v4f (&p)[T::JM]) {
                float sbi = 0.f;
                if constexpr (!T::NB_UNIFORM) sbi = sb_l[((n0 + wn * T::WN + 16 * i2) >> 7) - nb_first];
#pragma unroll
                for (int j = 0; j < T::JM; ++j) {
                    float s;
                    if constexpr (T::NB_UNIFORM) s = sw[j];
                    else s = sav[j] * sbi;
                    acc[i2][j] += p[j] * s;
                }
            };
            // Software pipeline over the N sub-tiles: the MFMAs of sub-tile i2 are issued before
            // the promotion FMAs of sub-tile i2-1, so the matrix core and the VALU overlap and
            // only one sub-tile row of partials is live.
            v4f pprev[T::JM];
#pragma unroll
            for (int i2 = 0; i2 < T::IN; ++i2) {
                v4f pcur[T::JM];
#pragma unroll
                for (int j = 0; j < T::JM; ++j) pcur[j] = mfma16x16x128(bf, af[j]);
                if (i2 + 1 < T::IN) bf = load_bf(i2 + 1);
                if (i2 > 0) promote(i2 - 1, pprev);
#pragma unroll
                for (int j = 0; j < T::JM; ++j) pprev[j] = pcur[j];
                // issue order inside the step: one MFMA, the next fragment's LDS reads, then
                // alternate MFMAs with the promotion FMAs of the previous step, so that one wave
                // keeps the matrix core and the VALU busy at the same time
                if (i2 > 0) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);          // DS read
#pragma unroll
                    for (int j = 1; j < T::JM; ++j) {
                        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);      // VALU
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
                    }
                    __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);         // VALU
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            promote(T::IN - 1, pprev);
        };

        // ---- two slices at a time (decode tiles): the fragments of slices i and i+1, then all
        // their MFMAs, then the promotions, slice i first
        auto compute_pair = [&](int i) {
            v8i af[2][T::JM];
            v8i bfr[2][T::IN];
            float sw[2][T::IN][T::JM];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl) {
                const uint8_t* st = smem + ((i + sl) % STAGES) * T::STAGE_BYTES;
                const float* sa_l = reinterpret_cast<const float*>(st + T::SA_OFF);
                const float* sb_l = reinterpret_cast<const float*>(st + T::SB_OFF);
                float sav[T::JM];
#pragma unroll
                for (int j = 0; j < T::JM; ++j) {
                    const int r = wm * T::WM + 16 * j + row16;
                    const uint8_t* rp = st + T::A_OFF + r * 128;
                    const v4i lo = *reinterpret_cast<const v4i*>(rp + frag_lo);
                    const v4i hi = *reinterpret_cast<const v4i*>(rp + frag_hi);
                    af[sl][j] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    sav[j] = sa_l[r];
                }
#pragma unroll
                for (int i2 = 0; i2 < T::IN; ++i2) {
                    const int r = wn * T::WN + 16 * i2 + row16;
                    const uint8_t* rp = st + T::B_OFF + r * 128;
                    const v4i lo = *reinterpret_cast<const v4i*>(rp + frag_lo);
                    const v4i hi = *reinterpret_cast<const v4i*>(rp + frag_hi);
                    bfr[sl][i2] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    const float sbi = sb_l[((n0 + wn * T::WN + 16 * i2) >> 7) - nb_first];
#pragma unroll
                    for (int j = 0; j < T::JM; ++j) sw[sl][i2][j] = sav[j] * sbi;
                }
            }
            v4f p[2][T::IN][T::JM];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int i2 = 0; i2 < T::IN; ++i2)
#pragma unroll
                    for (int j = 0; j < T::JM; ++j) p[sl][i2][j] = mfma16x16x128(bfr[sl][i2], af[sl][j]);
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int i2 = 0; i2 < T::IN; ++i2)
#pragma unroll
                    for (int j = 0; j < T::JM; ++j) acc[i2][j] += p[sl][i2][j] * sw[sl][i2][j];
        };

        if constexpr (T::SPB == 1) {
            // ---- ring of whole slices: slice i + STAGES - 1 goes into the stage slice i - 1 used
#pragma unroll
            for (int i = 0; i < STAGES - 1; ++i)
                if (i < nks) { issue_b(i, 0, T::B_DMA); issue_a(i); }
            for (int i = 0; i < nks; ++i) {
                // slice i landed (this wave's loads), then every wave's loads
                wait_slices<T::NDMA, STAGES - 2, 0>(min(STAGES - 2, nks - 1 - i));
                __syncthreads();
                if (i + STAGES - 1 < nks) { issue_b(i + STAGES - 1, 0, T::B_DMA); issue_a(i + STAGES - 1); }
                compute_slice(i);
            }
        } else {
            // ---- ring consumed two slices per barrier: slices i + STAGES - 2 and i + STAGES - 1 go
            // into the stages slices i - 2 and i - 1 used (read before this barrier)
#pragma unroll
            for (int i = 0; i < STAGES - 2; ++i)
                if (i < nks) { issue_b(i, 0, T::B_DMA); issue_a(i); }
            for (int i = 0; i < nks; i += 2) {
                // slices i and i + 1 landed: at most slices i + 2 .. i + STAGES - 3 still in flight
                wait_slices<T::NDMA, STAGES - 4, 0>(min(STAGES - 4, nks - 2 - i));
                __syncthreads();
                if (i + STAGES - 2 < nks) { issue_b(i + STAGES - 2, 0, T::B_DMA); issue_a(i + STAGES - 2); }
                if (i + STAGES - 1 < nks) { issue_b(i + STAGES - 1, 0, T::B_DMA); issue_a(i + STAGES - 1); }
                if (i + 1 < nks) compute_pair(i);
                else compute_slice(i);
            }
        }

        // ---- epilogue -----------------------------------------------------------------------
        bool store_direct = true;
        if (T::SPLITK && args.splits > 1) {
            // Split-K exchange between the workgroups of one tile, which may sit on different
            // XCDs (each with its own L2).  Partials are written and read with agent-coherent
            // (sc1) 16-byte buffer accesses, so no L2-wide write-back or invalidate is needed:
            //   write partial (sc1) -> wait until written -> barrier -> counter += 1 (agent)
            //   last arrival: barrier -> read all partials (sc1) in split order -> store D
            const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                uniform_ptr(args.ws + tile_id * args.splits * (int64_t)(BM * BN)), 0,
                (int)(args.splits * BM * BN * 4), kBufferFlags);
            const int lane_off = (wave * (T::WM * T::WN) + lane * 4) * 4;
#pragma unroll
            for (int i2 = 0; i2 < T::IN; ++i2)
#pragma unroll
                for (int j = 0; j < T::JM; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        acc[i2][j], ws_rsrc,
                        lane_off + ((split * BM * BN) + (i2 * T::JM + j) * 256) * 4, 0, kSc1);
            wait_vmcnt<0>();
            __syncthreads();
            if (tid == 0) {
                const int old = __hip_atomic_fetch_add(args.counters + tile_id, 1, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                const int last = (old == args.splits - 1);
                if (last)   // ready for the next launch
                    __hip_atomic_store(args.counters + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_flag = last;
            }
            __syncthreads();
            store_direct = s_flag != 0;
            if (store_direct) {
                // sum every split's partial (this one's included) in split order, so the result
                // does not depend on which workgroup arrived last; the reads of CH splits are in
                // flight together (loads first, unconditionally, then the ordered sums)
                constexpr int CH = (T::IN * T::JM >= 16) ? 1 : 16 / (T::IN * T::JM);
                for (int s0 = 0; s0 < args.splits; s0 += CH) {
                    v4f x[CH][T::IN][T::JM];
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        const int s2 = min(s0 + c, args.splits - 1);
#pragma unroll
                        for (int i2 = 0; i2 < T::IN; ++i2)
#pragma unroll
                            for (int j = 0; j < T::JM; ++j)
                                x[c][i2][j] = __builtin_amdgcn_raw_buffer_load_b128(
                                    ws_rsrc, lane_off + ((s2 * BM * BN) + (i2 * T::JM + j) * 256) * 4, 0, kSc1);
                    }
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        if (s0 + c < args.splits) {
#pragma unroll
                            for (int i2 = 0; i2 < T::IN; ++i2)
#pragma unroll
                                for (int j = 0; j < T::JM; ++j)
                                    acc[i2][j] = (s0 + c == 0) ? x[c][i2][j] : acc[i2][j] + x[c][i2][j];
                        }
                    }
                }
            }
        }
        if constexpr (SK) {
            if (sk) {
                // Stream-K exchange between the workgroups that share a leftover tile (segments
                // from consecutive workgroups w_a..w_b, in K order).  As the split-K exchange
                // above: partials are written and read with agent-coherent (sc1) accesses, each
                // into its writer's slot 2w + segment, and an agent-scope counter finds the last
                // to arrive, which sums the partials in K order.  A tile's last segment is usually
                // the last to arrive (its workgroup reaches it at the end of its range, the other
                // segments at the start of theirs); when the tile has just one other segment, the
                // last segment checks the counter before writing and, if the other is in, adds it
                // to its own accumulators and writes nothing (two terms: IEEE addition commutes,
                // so that is the K-order sum).  Any other last arrival re-reads every partial, its
                // own included, in K order.
                const int g0 = sk_tile * nkb;
                const int w_a = sk_owner(g0, args.sk_per, args.sk_extra);
                const int w_b = sk_owner(g0 + nkb - 1, args.sk_per, args.sk_extra);
                const bool fold = logical == w_b && w_b == w_a + 1;
                const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                    uniform_ptr(args.ws), 0, 2 * P * BM * BN * 4, kBufferFlags);
                const int lane_off = (wave * (T::WM * T::WN) + lane * 4) * 4;
                auto slot_of = [&](int w2) {
                    const int seg2 = (sk_start(w2, args.sk_per, args.sk_extra) / nkb == sk_tile) ? 0 : 1;
                    return (2 * w2 + seg2) * (BM * BN * 4) + lane_off;
                };
                bool last = false;
                if (fold) {
                    if (tid == 0)
                        s_flag = __hip_atomic_load(args.counters + sk_tile, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) == 1;
                    __syncthreads();
                    last = s_flag != 0;
                    __syncthreads();          // every wave has read s_flag before it is written again
                }
                if (!last) {
                    const int own = slot_of(logical);
#pragma unroll
                    for (int i2 = 0; i2 < T::IN; ++i2)
#pragma unroll
                        for (int j = 0; j < T::JM; ++j)
                            __builtin_amdgcn_raw_buffer_store_b128(acc[i2][j], ws_rsrc, own + (i2 * T::JM + j) * 1024, 0,
                                                                   kSc1);
                    wait_vmcnt<0>();
                    __syncthreads();
                    if (tid == 0) {
                        const int old = __hip_atomic_fetch_add(args.counters + sk_tile, 1, __ATOMIC_RELAXED,
                                                               __HIP_MEMORY_SCOPE_AGENT);
                        s_flag = (old == w_b - w_a);
                    }
                    __syncthreads();
                    last = s_flag != 0;
                }
                if (last && tid == 0)   // ready for the next launch
                    __hip_atomic_store(args.counters + sk_tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                store_direct = last;
                if (last) {
                    constexpr int NSUB = T::IN * T::JM;
                    constexpr int CH = NSUB < 8 ? NSUB : 8;      // sub-tiles of one read batch
                    // folding: acc += the other segment's partial; otherwise every partial in K order
                    if (!fold) {
                        const int off_a = slot_of(w_a);
#pragma unroll
                        for (int i2 = 0; i2 < T::IN; ++i2)
#pragma unroll
                            for (int j = 0; j < T::JM; ++j)
                                acc[i2][j] = __builtin_amdgcn_raw_buffer_load_b128(ws_rsrc, off_a + (i2 * T::JM + j) * 1024,
                                                                                   0, kSc1);
                    }
                    const int w_first = fold ? w_a : w_a + 1, w_last = fold ? w_a : w_b;
                    for (int w2 = w_first; w2 <= w_last; ++w2) {
                        const int off2 = slot_of(w2);
#pragma unroll
                        for (int c0 = 0; c0 < NSUB; c0 += CH) {
                            v4f x[CH];
#pragma unroll
                            for (int c = 0; c < CH; ++c)
                                if (c0 + c < NSUB)
                                    x[c] = __builtin_amdgcn_raw_buffer_load_b128(ws_rsrc, off2 + (c0 + c) * 1024, 0, kSc1);
#pragma unroll
                            for (int c = 0; c < CH; ++c)
                                if (c0 + c < NSUB) acc[(c0 + c) / T::JM][(c0 + c) % T::JM] += x[c];
                        }
                    }
                }
            }
        }
        if (store_direct) {
            // The lane index is made opaque here, so the epilogue's per-lane addresses are formed
            // after the K loop rather than kept live across it (registers are at the limit there).
            int el = lane;
            asm volatile("" : "+v"(el));
            const int erow16 = el & 15;
            const int egrp = el >> 4;
            // Rows of this wave's slab that are stored (bit r: tile row wm * WM + r): valid rows
            // only, and in the contiguous layout only the rows of this pass's group.
            bool row_ok = false;
            if (el < T::WM) {
                const int rm = wm * T::WM + el;
                row_ok = rm < valid_rows;
                if constexpr (LAYOUT == kContiguous) {
                    if (row_ok) row_ok = args.m_indices[arow0 + rm] == g;
                }
            }
            const uint64_t rowmask = __builtin_amdgcn_ballot_w64(row_ok);
            // every wave is past its last slice before any wave overwrites the ring with its stage
            if (!T::SPLITK || args.splits == 1) __syncthreads();
            // bf16 results into this wave's LDS region, row-major: lane owns row 16 j + row16,
            // columns 16 i2 + 4 grp .. + 3 of the wave's slab
            uint8_t* stg = smem + wave * T::STG_WAVE_BYTES;
#pragma unroll
            for (int j = 0; j < T::JM; ++j)
#pragma unroll
                for (int i2 = 0; i2 < T::IN; ++i2) {
                    const v4f v = acc[i2][j];
                    uint2 pk;
                    pk.x = pack_bf16x2(v.x, v.y);
                    pk.y = pack_bf16x2(v.z, v.w);
                    *reinterpret_cast<uint2*>(stg + (16 * j + erow16) * T::PITCH + (16 * i2 + 4 * egrp) * 2) = pk;
                }
            // then whole 16-byte chunks (8 columns) of rows, consecutive lanes along a row (the
            // wave's own LDS writes precede its reads in order; no barrier is needed)
            const int ncol0 = n0 + wn * T::WN;
#pragma unroll
            for (int st = 0; st < T::STORES; ++st) {
                const int idx = 64 * st + el;
                const int r = idx / T::CPR;
                const int c = idx - r * T::CPR;
                if (r >= T::WM || !((rowmask >> r) & 1)) continue;
                const uint4 v = *reinterpret_cast<const uint4*>(stg + r * T::PITCH + c * 16);
                const int n = ncol0 + 8 * c;
                uint16_t* drow = args.D + (arow0 + wm * T::WM + r) * (int64_t)N;
                if ((N & 7) == 0 && n + 8 <= N) {
                    *reinterpret_cast<uint4*>(drow + n) = v;
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (n + e < N) drow[n + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                }
            }
        }
        // the next pass's or unit's prologue rewrites stages other waves may still be reading
        __syncthreads();
        }   // pass
    }
}

}  // namespace fp8gemm
