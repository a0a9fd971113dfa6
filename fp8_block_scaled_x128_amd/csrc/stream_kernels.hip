// stream_kernels.hip -- gfx950 kernel of the M-grouped masked FP8 (and FP8 x FP4) GEMM at decode sizes: each
// group holds at most a few hundred rows of which about expected_m are valid, so the time is the
// stream of every group's B from HBM.
//
// The operation and the two-level accumulation are those of the tiled kernel (page
// "DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，核心代碼僅300行", sections 深入了解DeepGEMM and
// 如何使用？, masked layout): per 128-wide K block one MFMA with a zero accumulator gives the
// block's fresh fp32 partial, which is scaled by sa[m][kb] * sb[n/128][kb] and added to an fp32
// accumulator; the result is rounded once to bf16.
//
// What differs is the data movement:
//   - A tile covers 128 rows of a group and only its 16-row sub-tiles that hold valid rows are
//     loaded and multiplied, so a group with up to 128 valid rows streams its B once (the tiled
//     kernel's 64-row tiles stream it twice for a group past 64 rows).
//   - B never touches LDS.  Each wave owns JN 16-row fragments of B and loads them straight
//     into registers, PF K blocks deep (PF - 1 blocks in flight while one is consumed), with no
//     workgroup barrier on the B path.
//   - A (shared by every wave of the workgroup) and its scales are staged in LDS in phases of KP
//     K blocks, double buffered: loaded into registers one phase ahead and written to LDS at the
//     phase start, one barrier per phase instead of one per K block.  These are ordinary loads,
//     so the compiler's memory-counter waits for the B registers count them exactly (loads it
//     cannot see, such as direct-to-LDS DMA written in assembly, would make those waits drain
//     the B prefetch at every phase).
//
// Fragment layout.  The MFMA pairs equal byte positions of its X and Y operands, so any fixed
// permutation of the 128 K positions, applied to both, leaves the block sum unchanged.  Lane l
// (row l%16 of a fragment, q = l/16) holds bytes [16q, 16q+16) and [64+16q, 64+16q+16) of its
// row's K block: each B load instruction then reads 64 contiguous bytes from each of 16 rows.
// In LDS a row of A is 128 bytes with 16-byte chunk c stored at position c ^ ((r >> 1) & 7);
// for the two fragment reads (chunks q and 4+q) the 16 lanes the LDS serves together (one
// half-wave with equal parity of lane bits 2..4, measured on gfx950) hit 16 distinct 16-byte
// bank groups.
//
// The K loop is compiled once per count of active 16-row sub-tiles, so each K block's work is
// straight-line code over exactly the active sub-tiles, and A's loads cover only their rows.
//
// With FP4 = true, B holds E2M1 codes (two per byte) with one E8M0 scale per 32 values of K
// (OCP MXFP4; page "Perpustakaan operator GPU sumber terbuka DeepSeek DeepGEMM memperbarui versi
// besar, menambahkan Mega MoE…": FP8 x FP4 GEMM).  A K block of a B row is then 64 bytes, the
// scales ride in the MFMA's per-lane scale operand, and A's fp32 scale is applied per block as
// for E4M3.  B is then loaded two K blocks at a time, so each 128-byte line of a row is read from
// L2 once.
//
// Work units are (M tile, group, N tile of BN = 16*JN*W rows, K split), the M tile outermost so
// the units of tiles past every group's count (skipped at once) spread evenly over a persistent
// grid; each XCD takes a contiguous range of units, so the N tiles of a group share one L2.
// When K is split, partial tiles are exchanged and summed in split order by the last workgroup
// of the tile to arrive, as in the tiled kernel.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fp8gemm_device.h"
#include "fp8gemm_internal.h"

namespace fp8gemm {

// f(std::integral_constant<int, n>) for the runtime count n in [1, MAX]
template <int C, int MAX, typename F>
__device__ __forceinline__ void with_count_from(int n, F& f) {
    if constexpr (C < MAX) {
        if (n == C) {
            f(std::integral_constant<int, C>{});
            return;
        }
        with_count_from<C + 1, MAX>(n, f);
    } else {
        f(std::integral_constant<int, MAX>{});
    }
}

template <int MAX, typename F>
__device__ __forceinline__ void with_count(int n, F& f) {
    with_count_from<1, MAX>(n, f);
}

template <int MT, int W, int JN, int KP, int PF>
struct Stream {
    static constexpr int NT = 64 * W;
    static constexpr int BN = 16 * JN * W;          // rows of B per tile
    static constexpr int MSUB = MT / 16;            // 16-row sub-tiles of A
    static constexpr int NBW = BN >= 128 ? BN / 128 : 1;    // 128-row scale blocks of B per tile
    static constexpr int SA_OFF = KP * MT * 128;
    static constexpr int SB_OFF = SA_OFF + KP * MT * 4;
    static constexpr int PHASE_BYTES = SB_OFF + 256;
    static constexpr int LDS_BYTES = 2 * PHASE_BYTES;
    static constexpr int NA4 = (KP * MT * 8 + NT - 1) / NT;  // 16-byte chunks of A per thread per phase
    static constexpr int NSA = (KP * MT + NT - 1) / NT;      // scales of A per thread per phase
    static constexpr int U = (KP % PF == 0) ? KP : (PF % KP == 0 ? PF : KP * PF);  // K blocks per loop trip
    static_assert(MT % 64 == 0, "scales of A are moved 64 rows at a time");
    static_assert(128 % (16 * JN) == 0, "a wave's B rows lie inside one 128-row scale block");
    static_assert(BN < 128 || BN % 128 == 0, "tiles of B are whole scale blocks or inside one");
    static_assert(NBW * KP <= 64, "one x1 DMA moves the tile's B scales of a phase");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(PF >= 2, "at least one K block in flight");
    static_assert(U % PF == 0, "every loop trip starts a ring cycle");
};

template <int MT, int W, int JN, int KP, int PF, bool FP4>
__global__ __launch_bounds__(W * 64) void fp8gemm_masked_decode_kernel(const KernelArgs args) {
    using T = Stream<MT, W, JN, KP, PF>;
    // bytes of one 128-wide K block of a B row: E4M3 codes, or E2M1 codes two to a byte
    constexpr int KBB = FP4 ? 64 : 128;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
    __shared__ int s_flag;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15;
    const int q = lane >> 4;
    const int rsw = (r16 >> 1) & 7;              // chunk permutation of every fragment row of this lane
    const int frag_lo = (q ^ rsw) << 4;
    const int frag_hi = ((4 + q) ^ rsw) << 4;

    const int K = args.K;
    const int N = args.N;
    const int nkb = args.nkb;
    const int nnb = args.nnb;

    // XCD-aware order: workgroups are dealt to the 8 XCDs round robin, so give the workgroups of
    // one XCD a contiguous range of units -- the N tiles of a group then share its A tile in one
    // L2 instead of every XCD fetching every group's A.
    const int P = gridDim.x;
    int logical = blockIdx.x;
    if ((P & 7) == 0) logical = (blockIdx.x & 7) * (P >> 3) + (blockIdx.x >> 3);
    for (int unit = logical; unit < args.units; unit += P) {
        // ---- unit -> (split fastest, N tile, group, M tile) --------------------------------
        uint32_t u = (uint32_t)unit;
        const uint32_t tile_id = fast_div(u, args.div_splits);
        const int split = (int)(u - tile_id * (uint32_t)args.splits);
        u = tile_id;
        uint32_t v = fast_div(u, args.div_tiles_n);
        const int tn = (int)(u - v * (uint32_t)args.tiles_n);
        const uint32_t tm_u = fast_div(v, args.div_groups);
        const int gidx = (int)(v - tm_u * args.div_groups.d);
        const int tm = (int)tm_u;
        const int m0 = tm * MT;
        const int n0 = tn * T::BN;
        const int kb0 = split * args.kb_per_split;
        const int nks = min(nkb, kb0 + args.kb_per_split) - kb0;

        // ---- rows of the group: the valid count, clamped (a bad count flags the error word) --
        const int g = gidx;
        int cnt = args.masked_m[g];
        if (cnt < 0 || cnt > args.rows) {
            if (tm == 0 && tn == 0 && split == 0 && tid == 0) atomicOr(args.err, kDevErrBadCount);
            cnt = cnt < 0 ? 0 : (int)args.rows;
        }
        if (m0 >= cnt) continue;                       // uniform: whole workgroup skips
        const int64_t arow0 = (int64_t)g * args.rows + m0;
        const int row_limit = (int)min((int64_t)MT, args.rows - m0);   // rows of the tile in the group
        const int valid_rows = min(MT, cnt - m0);
        const int nsub = (valid_rows + 15) >> 4;       // active 16-row sub-tiles

        const uint8_t* Ag = args.A + arow0 * K;
        const float* sag = args.sa + (int64_t)g * nkb * args.rows + m0;   // sa is [group][K/128][rows]
        const float* sbg = FP4 ? nullptr : args.sb + (int64_t)g * nnb * nkb;
        const int nb_first = n0 >> 7;
        const int nb_count = min(nnb, (n0 + T::BN + 127) >> 7) - nb_first;
        // this wave's scale block of B, relative to the tile's first
        const int nbi_w = min(((n0 + wave * JN * 16) >> 7) - nb_first, nb_count - 1);

        // ---- B: per-lane offsets of the JN fragments (rows past N read row N-1) -------------
        // E4M3: lane q takes bytes [16q, +16) and [64+16q, +16) of its row's K block.
        // E2M1: lane q takes bytes [16q, +16) -- elements 32q .. 32q+31, one 32-element scale
        // block, whose E8M0 scale (byte q of the row's 4 scale bytes of the block) the MFMA applies;
        // with the A lanes' chunks q and 4+q this pairs equal K (mapped on gfx950: the E2M1
        // operand's nibbles 0-15 of lane group q meet E4M3 lane group 2(q%2) bytes 16(q/2)..+15,
        // nibbles 16-31 lane group 2(q%2)+1).
        const int64_t brow = FP4 ? K / 2 : K;
        const uint8_t* Bt = uniform_ptr(args.B + ((int64_t)g * N + n0) * brow);
        const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t*>(Bt), 0, 0x7FFFFFFF, kBufferFlags);
        uint32_t b_off[JN];
        uint32_t s_row[JN];          // E2M1: byte offset of the fragment row's E8M0 scales
#pragma unroll
        for (int f = 0; f < JN; ++f) {
            const int r = min(wave * JN * 16 + 16 * f + r16, N - 1 - n0);
            b_off[f] = (uint32_t)r * (uint32_t)brow + (uint32_t)(16 * q) + (uint32_t)kb0 * KBB;
            s_row[f] = (uint32_t)r * (uint32_t)(nkb * 4);
        }
        // E2M1 scales: the resource ends with the scale array, so a 16-byte load that runs past the
        // array's end (K below 512, last row) reads zeros there instead of faulting
        __amdgpu_buffer_rsrc_t s_rsrc = b_rsrc;
        if constexpr (FP4) {
            const int64_t first = ((int64_t)g * N + n0) * nkb * 4;
            const int64_t extent = (int64_t)args.G * N * nkb * 4 - first;
            s_rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(uniform_ptr(args.sbe + first)), 0,
                                                       (int)min(extent, (int64_t)0x7FFFFFFF), kBufferFlags);
        }
        // E4M3: one K block per ring slot, its lane chunks q and 4+q.  E2M1: a pair of K blocks
        // (kb, kb + 1) per slot, lane chunk q of each: the two 64-byte halves of each row's 128-byte
        // line are requested back to back, so the line crosses from L2 once (requested one K block
        // apart, the line has left the CU's cache before its second half is read, and every line
        // crosses twice).  Past the unit's last block the second load repeats the first.
        v8i ring[FP4 ? PF / 2 : PF][JN];
        auto issue_b = [&](int kb, v8i (&dst)[JN]) {
#pragma unroll
            for (int f = 0; f < JN; ++f) {
                const uint32_t o = b_off[f] + (uint32_t)kb * KBB;
                const uint32_t o2 = FP4 ? (kb + 1 < nks ? o + 64u : o) : o + 64u;
                const v4i lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, (int)o, 0, 0));
                const v4i hi = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(b_rsrc, (int)o2, 0, 0));
                dst[f] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            }
        };
        // E2M1 scales of 4 consecutive K blocks per fragment row in one 16-byte load (a row's E8M0
        // bytes are contiguous: 4 per K block), loaded one loop trip ahead: a load whose lanes walk
        // 16 rows costs the CU's address path as much for 4 bytes as for 16.  The load starts at
        // block min(a, nkb - 4) so it stays inside the row; sh = a - start moves the words up.
        constexpr int SV = FP4 ? T::U / 4 : 1;
        static_assert(!FP4 || T::U % 4 == 0, "E2M1 scale loads cover 4 K blocks of one loop trip");
        static_assert(!FP4 || (PF % 2 == 0 && PF >= 4), "E2M1: whole pairs of K blocks, one pair in flight");
        v4u scur[SV][JN], snxt[SV][JN];
        int shc[SV], shn[SV];
        auto issue_s = [&](int first, v4u (&dst)[SV][JN], int (&sh)[SV]) {
#pragma unroll
            for (int i = 0; i < SV; ++i) {
                const int a = kb0 + first + 4 * i;
                const int start = max(0, min(a, nkb - 4));
                sh[i] = a - start;
#pragma unroll
                for (int f = 0; f < JN; ++f)
                    dst[i][f] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                        s_rsrc, (int)(s_row[f] + (uint32_t)start * 4u), 0, 0));
            }
        };
        // the scale word of trip block u2 (uniform index: selects, no memory)
        auto scale_word = [&](const v4u& v, int w) -> uint32_t {
            return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
        };

        // ---- A and scales of phase ph (K blocks [ph*KP, ph*KP + tp)): global -> registers, one
        // phase ahead, then registers -> LDS buffer ph&1 at the phase start.  Every load of the K
        // loop is unconditional (a K block or row past the end re-reads the last valid one, a cache
        // hit), so the compiler's memory-counter waits before each use stay exact and leave the
        // later loads in flight.
        // rows of A loaded: the NS active sub-tiles (a compile-time count, so a workgroup issues
        // only the loads its valid rows need), clamped to the array (rows past the count are
        // never read; a clamped row re-reads the last one, a cache hit)
        const int rows_needed = min(nsub * 16, row_limit);
        v4i a_reg[T::NA4];
        float sa_reg[T::NSA];
        float sb_reg = 0.f;
        auto load_a = [&](auto ns_c, int ph) {
            constexpr int RN = decltype(ns_c)::value * 16;           // rows staged per K block
            constexpr int NA = (KP * RN * 8 + T::NT - 1) / T::NT;    // 16-byte chunks per thread
            const int kbp = ph * KP;
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const int cid = tid + T::NT * i;          // chunk: 8 per row, RN rows per K block
                const int kb = min(kbp + cid / (RN * 8), nks - 1);
                const int r = min((cid >> 3) % RN, rows_needed - 1);
                a_reg[i] = *reinterpret_cast<const v4i*>(Ag + (int64_t)r * K + (int64_t)(kb0 + kb) * 128 + (cid & 7) * 16);
            }
#pragma unroll
            for (int i = 0; i < T::NSA; ++i) {
                const int sid = tid + T::NT * i;
                const int kb = min(kbp + sid / MT, nks - 1);
                const int r = min(sid % MT, rows_needed - 1);
                sa_reg[i] = sag[(int64_t)(kb0 + kb) * args.rows + r];
            }
            if constexpr (!FP4) {
                const int x = min(tid, T::NBW * KP - 1);
                const int nbi = min(x / KP, nb_count - 1);
                const int kb = min(kbp + x % KP, nks - 1);
                sb_reg = sbg[(int64_t)(nb_first + nbi) * nkb + kb0 + kb];
            }
        };
        auto store_a = [&](auto ns_c, int ph) {
            constexpr int RN = decltype(ns_c)::value * 16;
            constexpr int NA = (KP * RN * 8 + T::NT - 1) / T::NT;
            const int kbp = ph * KP;
            const int tp = min(KP, nks - kbp);
            uint8_t* dst = smem + (ph & 1) * T::PHASE_BYTES;
#pragma unroll
            for (int i = 0; i < NA; ++i) {
                const int cid = tid + T::NT * i;
                const int t = cid / (RN * 8);
                const int r = (cid >> 3) % RN;
                if (t < tp && r < rows_needed)
                    *reinterpret_cast<v4i*>(dst + (t * MT + r) * 128 + (((cid & 7) ^ ((r >> 1) & 7)) << 4)) = a_reg[i];
            }
#pragma unroll
            for (int i = 0; i < T::NSA; ++i) {
                const int sid = tid + T::NT * i;
                const int t = sid / MT;
                const int r = sid % MT;
                if (t < tp && r < rows_needed)
                    reinterpret_cast<float*>(dst + T::SA_OFF)[t * MT + r] = sa_reg[i];
            }
            if (!FP4 && tid < T::NBW * KP) reinterpret_cast<float*>(dst + T::SB_OFF)[tid] = sb_reg;
        };

        // ---- accumulators -------------------------------------------------------------------
        v4f acc[JN][T::MSUB];
#pragma unroll
        for (int f = 0; f < JN; ++f)
#pragma unroll
            for (int j = 0; j < T::MSUB; ++j) acc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};

        // one K block over the NS active sub-tiles (a compile-time count, so the block is
        // straight-line code: the A reads, then NS * JN independent MFMAs, then their promotions,
        // which the scheduler can overlap; a branch per sub-tile would serialise every MFMA with
        // the FMAs that read its result)
        auto compute = [&](auto ns_c, int kb, const v8i (&bf)[JN], const uint32_t (&sw)[JN]) {
            constexpr int NS = decltype(ns_c)::value;
            const int t = kb % KP;
            const uint8_t* ph = smem + ((kb / KP) & 1) * T::PHASE_BYTES;
            const uint8_t* ab = ph + t * MT * 128;
            const float* sal = reinterpret_cast<const float*>(ph + T::SA_OFF) + t * MT;
            // E4M3 B: the 128x128 block scale, applied with sa; E2M1 B: scales inside the MFMA
            const float sbv = FP4 ? 1.0f : reinterpret_cast<const float*>(ph + T::SB_OFF)[nbi_w * KP + t];
            if constexpr (JN == 1 || JN >= 4) {
                // one sub-tile at a time, so few registers stay live (JN MFMAs per step are
                // independent when JN >= 4; with one fragment per wave there is one K loop for
                // every count -- NS = all sub-tiles, the active ones chosen at run time -- and two
                // workgroups fit on a CU, whose waves cover each other's latencies)
#pragma unroll
                for (int j = 0; j < NS; ++j) {
                    if (JN == 1 && j >= nsub) break;
                    const uint8_t* rp = ab + (16 * j + r16) * 128;
                    const v4i lo = *reinterpret_cast<const v4i*>(rp + frag_lo);
                    const v4i hi = *reinterpret_cast<const v4i*>(rp + frag_hi);
                    const v8i a1 = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                    const float s1 = sal[16 * j + r16] * sbv;
                    v4f p1[JN];
#pragma unroll
                    for (int f = 0; f < JN; ++f) {
                        if constexpr (FP4) p1[f] = mfma16x16x128_fp4_fp8(bf[f], a1, (int)((sw[f] >> (8 * q)) & 0xFFu));
                        else p1[f] = mfma16x16x128(bf[f], a1);
                    }
#pragma unroll
                    for (int f = 0; f < JN; ++f) acc[f][j] += p1[f] * s1;
                    __builtin_amdgcn_sched_barrier(0);
                }
                return;
            }
            v8i af[NS];
            float s[NS];
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const uint8_t* rp = ab + (16 * j + r16) * 128;
                const v4i lo = *reinterpret_cast<const v4i*>(rp + frag_lo);
                const v4i hi = *reinterpret_cast<const v4i*>(rp + frag_hi);
                af[j] = (v8i){lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
                s[j] = sal[16 * j + r16] * sbv;
            }
            v4f p[NS][JN];
#pragma unroll
            for (int j = 0; j < NS; ++j)
#pragma unroll
                for (int f = 0; f < JN; ++f) {
                    if constexpr (FP4) p[j][f] = mfma16x16x128_fp4_fp8(bf[f], af[j], (int)((sw[f] >> (8 * q)) & 0xFFu));
                    else p[j][f] = mfma16x16x128(bf[f], af[j]);
                }
#pragma unroll
            for (int j = 0; j < NS; ++j)
#pragma unroll
                for (int f = 0; f < JN; ++f) acc[f][j] += p[j][f] * s[j];
        };

        // ---- K loop: B PF-1 blocks ahead in registers, A one phase ahead in LDS ----------------
        // the same issue order as in the loop (A of a phase, then B), so the memory-counter state
        // the compiler merges at the loop head does not force a full drain
        auto kloop = [&](auto ns_c) {
            load_a(ns_c, 0);
            asm volatile("" ::: "memory");
            if constexpr (FP4) issue_s(0, scur, shc);
            // E2M1: PP slots of block pairs, the pair starting at block kb + 2 (PP - 1) issued at
            // every even block kb into the slot the previous pair used
            constexpr int PP = PF / 2;
            const int last_pair = (nks - 1) & ~1;
            if constexpr (FP4) {
#pragma unroll
                for (int p = 0; p < PP - 1; ++p) issue_b(min(2 * p, last_pair), ring[p]);
            } else {
#pragma unroll
                for (int u2 = 0; u2 < PF - 1; ++u2) issue_b(min(u2, nks - 1), ring[u2]);
            }
            for (int base = 0; base < nks; base += T::U) {
                // U = lcm(KP, PF) K blocks: every trip starts a phase and a ring cycle
                if constexpr (FP4) issue_s(base + T::U, snxt, shn);
#pragma unroll
                for (int u2 = 0; u2 < T::U; ++u2) {
                    const int kb = base + u2;
                    if (u2 % KP == 0) {
                        // phase start: this phase's A into LDS, visible to every wave, then the
                        // next phase's loads (the buffer they go to was last read two phases ago)
                        store_a(ns_c, kb / KP);
                        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                        load_a(ns_c, kb / KP + 1);
                    }
                    if constexpr (FP4) {
                        if (u2 % 2 == 0) issue_b(min(kb + 2 * (PP - 1), last_pair), ring[(u2 / 2 + PP - 1) % PP]);
                    } else {
                        issue_b(min(kb + PF - 1, nks - 1), ring[(u2 + PF - 1) % PF]);
                    }
                    if (kb < nks) {
                        uint32_t sw[JN];
#pragma unroll
                        for (int f = 0; f < JN; ++f)
                            sw[f] = FP4 ? scale_word(scur[(u2 / 4) % SV][f], u2 % 4 + shc[(u2 / 4) % SV]) : 0u;
                        if constexpr (FP4) {
                            // this block's half of the pair in the operand's low four registers
                            // (the E2M1 operand reads only those)
                            v8i bsel[JN];
#pragma unroll
                            for (int f = 0; f < JN; ++f) {
                                const v8i x = ring[(u2 / 2) % PP][f];
                                bsel[f] = (u2 % 2 == 0) ? x : __builtin_shufflevector(x, x, 4, 5, 6, 7, 4, 5, 6, 7);
                            }
                            compute(ns_c, kb, bsel, sw);
                        } else {
                            compute(ns_c, kb, ring[u2 % PF], sw);
                        }
                    }
                    // keep each K block's LDS reads and MFMAs in its own step: hoisting later blocks'
                    // reads raises register use past what the ring and accumulators need
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (FP4) {
#pragma unroll
                    for (int i = 0; i < SV; ++i) {
                        shc[i] = shn[i];
#pragma unroll
                        for (int f = 0; f < JN; ++f) scur[i][f] = snxt[i][f];
                    }
                }
            }
        };
        // one instance of the K loop per active sub-tile count (one for all counts with one
        // fragment per wave)
        if constexpr (JN == 1) kloop(std::integral_constant<int, T::MSUB>{});
        else with_count<T::MSUB>(nsub, kloop);

        // ---- epilogue: split-K exchange (agent-coherent partials), then bf16 stores ---------
        bool store_direct = true;
        if (args.splits > 1) {
            const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                uniform_ptr(args.ws + (int64_t)tile_id * args.splits * (MT * T::BN)), 0,
                (int)(args.splits * MT * T::BN * 4), kBufferFlags);
            const int lane_off = (wave * JN * T::MSUB * 256 + lane * 4) * 4;
            // every sub-tile is written and read (those past the valid rows carry unused values),
            // so no access sits behind a branch and the reads below stay in flight together
#pragma unroll
            for (int f = 0; f < JN; ++f)
#pragma unroll
                for (int j = 0; j < T::MSUB; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        acc[f][j], ws_rsrc, lane_off + ((split * MT * T::BN) + (f * T::MSUB + j) * 256) * 4, 0,
                        kSc1);
            wait_vmcnt<0>();
            __syncthreads();
            if (tid == 0) {
                const int old = __hip_atomic_fetch_add(args.counters + tile_id, 1, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                const int last = (old == args.splits - 1);
                if (last)
                    __hip_atomic_store(args.counters + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                s_flag = last;
            }
            __syncthreads();
            store_direct = s_flag != 0;
            if (store_direct) {
                // sum every split's partial (this one's included) in split order, CH splits' reads
                // in flight at a time
                constexpr int CH = (JN * T::MSUB >= 16) ? 1 : 16 / (JN * T::MSUB);
                for (int s0 = 0; s0 < args.splits; s0 += CH) {
                    v4f x[CH][JN][T::MSUB];
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        const int s2 = min(s0 + c, args.splits - 1);
#pragma unroll
                        for (int f = 0; f < JN; ++f)
#pragma unroll
                            for (int j = 0; j < T::MSUB; ++j)
                                x[c][f][j] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(
                                    ws_rsrc, lane_off + ((s2 * MT * T::BN) + (f * T::MSUB + j) * 256) * 4, 0, kSc1));
                    }
#pragma unroll
                    for (int c = 0; c < CH; ++c) {
                        if (s0 + c < args.splits) {
#pragma unroll
                            for (int f = 0; f < JN; ++f)
#pragma unroll
                                for (int j = 0; j < T::MSUB; ++j)
                                    acc[f][j] = (s0 + c == 0) ? x[c][f][j] : acc[f][j] + x[c][f][j];
                        }
                    }
                }
            }
        }
        if (store_direct) {
#pragma unroll
            for (int j = 0; j < T::MSUB; ++j) {
                const int rm = 16 * j + r16;
                if (j >= nsub || rm >= valid_rows) continue;
                uint16_t* drow = args.D + (arow0 + rm) * (int64_t)N;
#pragma unroll
                for (int f = 0; f < JN; ++f) {
                    const int n = n0 + wave * JN * 16 + 16 * f + 4 * q;
                    const v4f x = acc[f][j];
                    if (n + 3 < N && (N & 3) == 0) {
                        uint2 pk;
                        pk.x = pack_bf16x2(x.x, x.y);
                        pk.y = pack_bf16x2(x.z, x.w);
                        *reinterpret_cast<uint2*>(drow + n) = pk;
                    } else {
                        const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            if (n + r < N) {
                                __bf16 h = (__bf16)e[r];
                                uint16_t hb;
                                __builtin_memcpy(&hb, &h, 2);
                                drow[n + r] = hb;
                            }
                        }
                    }
                }
            }
        }
        // the next unit's first phase rewrites LDS other waves may still be reading
        __syncthreads();
    }
}

// ------------------------------------------------------------------------------------------
// instantiation table
// ------------------------------------------------------------------------------------------

template <int MT, int W, int JN, int KP, int PF, bool FP4>
static void launch_stream(dim3 grid, const KernelArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((fp8gemm_masked_decode_kernel<MT, W, JN, KP, PF, FP4>), grid, dim3(W * 64), 0, s, a);
}

template <int MT, int W, int JN, int KP, int PF, bool FP4>
static KernelEntry stream_entry(const char* name) {
    using T = Stream<MT, W, JN, KP, PF>;
    KernelEntry e;
    e.name = name;
    e.kind = kKindStream;
    e.layout = kMasked;
    e.fp4 = FP4;
    e.bm = MT;
    e.bn = T::BN;
    e.waves_m = 1;
    e.waves_n = W;
    e.stages = PF;
    e.jn = JN;
    e.kp = KP;
    e.threads = T::NT;
    e.splitk = true;
    e.lds_bytes = T::LDS_BYTES;
    e.func = reinterpret_cast<const void*>(&fp8gemm_masked_decode_kernel<MT, W, JN, KP, PF, FP4>);
    e.launch = &launch_stream<MT, W, JN, KP, PF, FP4>;
    return e;
}

#define STREAM_ENTRY(MT, W, JN, KP, PF) \
    stream_entry<MT, W, JN, KP, PF, false>("masked decode " #MT " rows, " #W " waves x " #JN " fragments, phase " #KP ", depth " #PF)
#define STREAM_ENTRY_FP4(MT, W, JN, KP, PF) \
    stream_entry<MT, W, JN, KP, PF, true>("masked decode FP8xFP4 " #MT " rows, " #W " waves x " #JN " fragments, phase " #KP ", depth " #PF)

// Masked groups of at most 128 valid rows (one tile per group and N tile, B streamed once per
// group).  Measured on 16 groups x 256 rows (about 64 valid each), graphs of 3 launches:
//   N = 4096, K = 7168: 4 waves x 4 fragments 99 us (4.9 TB/s); x 2 fragments 104 us; 8 waves x 1
//     fragment 106 us; 4 waves x 1 fragment 126 us; the tiled kernel's 128x128 tile 168 us;
//     with E2M1 B (loaded in block pairs; operand copies beyond the memory-side cache): 4 waves x
//     2 fragments 8 blocks deep 85.0-85.8 us, x 4 fragments 4 deep 87.0-87.2 us; the same 2 x 8 with
//     E4M3 B: 111.5-111.8 us against 101.7-103.0 us for 4 x 4;
//   N = 7168, K = 2048: 4 waves x 4 fragments 60 us (4.2 TB/s); x 2: 64 us; x 1: 66 us.
// Wider tiles win: the A tile staged per workgroup then serves more B bytes.  Splitting K was
// slower everywhere (the groups times N tiles already fill the CUs).
//
// What bounds these kernels is the vector-memory issue rate of a CU, not HBM: a 16-byte-per-lane
// load whose lanes walk 16 rows (the MFMA's lane layout: lane l holds row l % 16) occupies the
// CU's address path about 58 cycles, against 18 for 8 rows x 128 bytes and 16 for a contiguous
// kilobyte (measured on gfx950 with L2-resident data); B, and for E2M1 its per-row scales, are
// loaded in the 16-row form.
const KernelEntry* stream_table(int* count) {
    static const KernelEntry table[] = {
        STREAM_ENTRY(128, 4, 2, 2, 4),
        STREAM_ENTRY(128, 4, 1, 2, 4),
        STREAM_ENTRY(128, 8, 1, 2, 4),
        STREAM_ENTRY(128, 4, 4, 2, 4),
        // E4M3 x E2M1 (B with one E8M0 scale per 32 K): half the B bytes per K block
        STREAM_ENTRY_FP4(128, 4, 2, 2, 4),
        STREAM_ENTRY_FP4(128, 4, 4, 2, 4),
        STREAM_ENTRY_FP4(128, 4, 1, 2, 4),
        STREAM_ENTRY_FP4(128, 4, 2, 2, 8),
        STREAM_ENTRY_FP4(128, 8, 1, 2, 4),
    };
    *count = (int)(sizeof(table) / sizeof(table[0]));
    return table;
}

}  // namespace fp8gemm
