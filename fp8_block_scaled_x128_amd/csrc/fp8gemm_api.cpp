// fp8gemm_api.cpp -- C ABI of libfp8gemm.so: argument validation, launch-shape selection,
// split-K workspace management and kernel launch (host code).
//
// Entry points and their meaning: include/fp8gemm.h (the dense NT GEMM and the two M-grouped
// MoE layouts of page "DeepSeek開源第三彈：V3/R1訓練推理關鍵秘籍，核心代碼僅300行", section
// 如何使用？).  The launch shape is chosen per call from the problem size (the pages' per-shape
// block-size choice, section 如何使用？, JIT design item; here an ahead-of-time table).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "fp8gemm.h"
#include "fp8gemm_internal.h"

using namespace fp8gemm;

namespace {

constexpr int kMaxDevices = 64;

struct Workspace {
    float* partials = nullptr;
    size_t partial_bytes = 0;
    int32_t* counters = nullptr;
    size_t counter_count = 0;
};

struct DeviceState {
    std::mutex mu;
    bool ready = false;
    int id = 0;
    int cus = 0;
    int32_t* err = nullptr;                              // device error word (static device memory)
    ScratchPointers scratch;                             // static split-K scratch of fp8gemm_nt_noalloc
    std::vector<int> occupancy;                          // per kernel-table entry
    std::unordered_map<hipStream_t, Workspace> ws;       // split-K workspace per stream
};

DeviceState g_dev[kMaxDevices];

// Every kernel of the library: the tiled table, then the stream table.
const std::vector<KernelEntry>& kernels() {
    static const std::vector<KernelEntry> all = [] {
        std::vector<KernelEntry> v;
        int n = 0;
        const KernelEntry* t = kernel_table(&n);
        v.insert(v.end(), t, t + n);
        t = stream_table(&n);
        v.insert(v.end(), t, t + n);
        return v;
    }();
    return all;
}
std::atomic<int> g_cu_cap{0};
thread_local char g_last_config[256] = "";

// Query the device once: CU count, occupancy of every kernel, the device addresses of the
// static error word and scratch.  Allocates nothing.
int device_state(DeviceState** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8GEMM_ERR_HIP;
    DeviceState& d = g_dev[dev];
    std::lock_guard<std::mutex> lock(d.mu);
    if (!d.ready) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8GEMM_ERR_HIP;
        d.cus = prop.multiProcessorCount;
        d.id = dev;
        const std::vector<KernelEntry>& tab = kernels();
        d.occupancy.assign(tab.size(), 1);
        for (size_t i = 0; i < tab.size(); ++i) {
            int blocks = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, tab[i].func, tab[i].threads, 0) ==
                    hipSuccess && blocks > 0)
                d.occupancy[i] = blocks;
        }
        // the error word and the no-allocation scratch are static device arrays: their device
        // addresses on this device (nothing is allocated; both are zero from the code object's load)
        if (scratch_pointers(&d.scratch) != 0) return FP8GEMM_ERR_HIP;
        d.err = d.scratch.err;
        d.ready = true;
    }
    *out = &d;
    return FP8GEMM_OK;
}

// Capacity of a stream's split-K workspace.  An automatically chosen split launch has at most one
// unit per CU (pick_split), and the largest tile compiled with the split-K exchange is 128 x 256
// fp32 (128 KiB); a stream-K launch of 256 x 256 tiles (one workgroup per CU) keeps two partial
// tiles per workgroup (512 KiB).  So cus * 512 KiB of partials and one counter per unit cover
// every such launch.  A forced configuration (FP8GEMM_FORCE_CONFIG) beyond it is refused.
constexpr size_t kMaxPartialBytesPerCu = 2 * 256 * 256 * sizeof(float);
// Fewest K blocks per workgroup that stream-K must save over whole tiles (see launch()).
int stream_k_min_blocks(int bn) { return bn >= 256 ? 12 : (bn >= 192 ? 9 : 6); }

// The stream-K plan of a dense launch of `tiles` 256-row tiles of width bn on P workgroups: the
// whole-tile rounds, then the leftover tiles' K blocks shared out, `per` to each workgroup and
// one more to the first `extra`.  Returns whether stream-K is taken (the thresholds of launch(),
// or FP8GEMM_STREAMK=0/1) and sets the K blocks of the busiest workgroup either way.
bool stream_k_plan(int64_t tiles, int64_t P, int nkb, int bn, int64_t* per, int64_t* extra, int64_t* blocks) {
    P = std::max<int64_t>(P, 1);
    const int64_t full = tiles / P, R = tiles % P;
    *per = R * nkb / P;
    *extra = R * nkb % P;
    const int64_t saved = nkb - *per - (*extra > 0 ? 1 : 0);
    const char* f = std::getenv("FP8GEMM_STREAMK");
    const bool want = (f && *f) ? f[0] == '1' : saved >= stream_k_min_blocks(bn) && 3 * *per >= nkb;
    const bool take = want && R > 0 && *per >= 1;
    *blocks = take ? full * nkb + *per + (*extra > 0 ? 1 : 0) : (tiles + P - 1) / P * nkb;
    return take;
}
size_t workspace_partial_bytes(int cus) { return (size_t)std::max(cus, 1) * kMaxPartialBytesPerCu; }
size_t workspace_counters(int cus) { return std::max<size_t>((size_t)cus, 4096); }

// The split-K workspace of `stream`: allocated once, at full capacity, the first time the stream
// needs one, and never freed or moved afterwards, so a HIP graph captured on the stream keeps
// valid pointers for the life of the process.  Counters are zeroed at allocation and every
// launch leaves them at zero.  No allocation is made while the stream is capturing (the stream
// must be prepared before: fp8gemm_prepare_stream or an earlier split-K call).
int workspace(DeviceState* d, hipStream_t stream, size_t partial_bytes, size_t counters,
              Workspace** out) {
    std::lock_guard<std::mutex> lock(d->mu);
    auto it = d->ws.find(stream);
    if (it == d->ws.end()) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return FP8GEMM_ERR_HIP;
        if (cs != hipStreamCaptureStatusNone) return FP8GEMM_ERR_UNSUPPORTED;
        Workspace w;
        const size_t bytes = workspace_partial_bytes(d->cus);
        const size_t n = workspace_counters(d->cus);
        if (hipMalloc(&w.partials, bytes) != hipSuccess) return FP8GEMM_ERR_HIP;
        // on a failure, release what was allocated (the first error is the one reported)
        if (hipMalloc(&w.counters, n * sizeof(int32_t)) != hipSuccess) {
            (void)hipFree(w.partials);
            return FP8GEMM_ERR_HIP;
        }
        if (hipMemset(w.counters, 0, n * sizeof(int32_t)) != hipSuccess) {
            (void)hipFree(w.partials);
            (void)hipFree(w.counters);
            return FP8GEMM_ERR_HIP;
        }
        w.partial_bytes = bytes;
        w.counter_count = n;
        it = d->ws.emplace(stream, w).first;
    }
    Workspace& w = it->second;
    if (w.partial_bytes < partial_bytes || w.counter_count < counters) return FP8GEMM_ERR_UNSUPPORTED;
    *out = &w;
    return FP8GEMM_OK;
}

int find_entry(int layout, int bm, int bn, int wm, int wn, int stages) {
    const std::vector<KernelEntry>& tab = kernels();
    for (size_t i = 0; i < tab.size(); ++i)
        if (tab[i].kind == kKindTiled && tab[i].layout == layout && tab[i].bm == bm && tab[i].bn == bn &&
            tab[i].waves_m == wm && tab[i].waves_n == wn && tab[i].stages == stages)
            return (int)i;
    return -1;
}

int find_stream(int layout, int mt, int w, int jn, int kp, int pf, bool fp4 = false) {
    const std::vector<KernelEntry>& tab = kernels();
    for (size_t i = 0; i < tab.size(); ++i)
        if (tab[i].kind == kKindStream && tab[i].layout == layout && tab[i].fp4 == fp4 && tab[i].bm == mt &&
            tab[i].waves_n == w && tab[i].jn == jn && tab[i].kp == kp && tab[i].stages == pf)
            return (int)i;
    return -1;
}

// Optional override for experiments:
//   FP8GEMM_FORCE_CONFIG=BMxBN:WMxWN:STAGES:SPLIT            (tiled kernel)
//   FP8GEMM_FORCE_CONFIG=stream:MT:W:JN:KP:PF:SPLIT           (masked decode kernel; with an
//                                                             E2M1 B, its E2M1 configuration)
bool forced_config(int layout, bool fp4, int* idx, int* split) {
    const char* s = std::getenv("FP8GEMM_FORCE_CONFIG");
    if (!s || !*s) return false;
    int i = -1, sp = 1;
    if (std::strncmp(s, "stream:", 7) == 0) {
        int mt, w, jn, kp, pf;
        if (std::sscanf(s + 7, "%d:%d:%d:%d:%d:%d", &mt, &w, &jn, &kp, &pf, &sp) < 6) return false;
        i = find_stream(layout, mt, w, jn, kp, pf, fp4);
    } else {
        if (fp4) return false;
        int bm, bn, wm, wn, st;
        if (std::sscanf(s, "%dx%d:%dx%d:%d:%d", &bm, &bn, &wm, &wn, &st, &sp) < 6) return false;
        i = find_entry(layout, bm, bn, wm, wn, st);
    }
    if (i < 0) return false;
    *idx = i;
    *split = std::max(1, sp);
    return true;
}

struct Choice {
    int entry;
    int split;
};

// K splits so that tiles * splits fills the CUs with at most one unit each (a second, partly
// empty round of units would double the time), each split keeping >= 4 K slices.
int pick_split(int64_t tiles, int nkb, int cus) {
    if (tiles >= cus) return 1;
    int64_t s = cus / tiles;
    s = std::min<int64_t>(s, std::max(1, nkb / 4));
    return (int)std::max<int64_t>(1, s);
}

// Masked groups at decode sizes (expected rows <= 128): the masked decode kernel, one 128-row
// tile per group and N tile, B read once straight into registers (HBM bytes 1.00x the
// algorithmic on the 16-group configuration with E4M3 weights, 1.03x with E2M1:
// profiles/counters_grouped.txt).  K splits only when the groups
// times N tiles leave CUs idle.  Returns -1 when the kernel's 32-bit per-lane offsets cannot
// address K (then the tiled kernel serves the call).
Choice choose_masked_decode(int64_t N, int nkb, int64_t groups, int cus, bool fp4) {
    const int64_t K = (int64_t)nkb * 128;
    // 256-row N tiles (4 fragments per wave), so the A tile staged per workgroup serves as many B
    // bytes as possible, while the groups times N tiles fill at least half the CUs; else 128-row
    // tiles, and 64-row tiles for short K (few blocks per unit: more units overlap their start-up)
    // (E2M1 B at that width: 128-row tiles, 8 blocks deep -- four slots of block pairs in flight)
    const int64_t tiles256 = groups * ((N + 255) / 256);
    const int wide = fp4 ? find_stream(kMasked, 128, 4, 2, 2, 8, true) : find_stream(kMasked, 128, 4, 4, 2, 4, false);
    Choice c{tiles256 * 2 >= cus ? wide
             : (K <= 2048 ? find_stream(kMasked, 128, 4, 1, 2, 4, fp4) : find_stream(kMasked, 128, 4, 2, 2, 4, fp4)),
             1};
    if (c.entry < 0) return c;
    const KernelEntry& e = kernels()[c.entry];
    if ((int64_t)std::max(e.bm, e.bn + 1) * K >= (int64_t(1) << 31)) return Choice{-1, 1};
    c.split = pick_split(groups * ((N + e.bn - 1) / e.bn), nkb, cus);
    return c;
}

// Launch-shape table.  Rows of A per tile decide the regime:
//  - <= 128 rows (decode): HBM-bound stream of B.  Masked groups: the masked decode kernel above.
//    Otherwise tiles span all rows of A (64, or 128 when A re-reads would cost as much as B:
//    K >= 8192 or very wide N), N tiles of 64 or 128 so that about one unit per CU is in flight,
//    and split-K to reach that count on narrow N.  64-row tiles over K >= 8192 take the 6-slice
//    ring consumed two slices per barrier.
//  - >= 1024 rows (prefill): MFMA-bound; 256x256 tiles, 8 waves.
//  - in between: 128x128 tiles.
Choice choose(int layout, int64_t rows, int64_t N, int nkb, int64_t expected_rows, int G, int cus, bool fp4) {
    Choice c{-1, 1};
    int forced = -1, fsplit = 1;
    if (forced_config(layout, fp4, &forced, &fsplit)) return Choice{forced, fsplit};
    const int64_t m = (layout == kMasked) ? std::max<int64_t>(1, std::min(expected_rows, rows)) : rows;
    const int64_t groups = (layout == kMasked) ? G : 1;
    // an E2M1 B runs only on the masked decode kernel (groups past 128 rows take several M tiles)
    if (fp4) return choose_masked_decode(N, nkb, groups, cus, true);
    if (layout == kMasked && m <= 128) {
        c = choose_masked_decode(N, nkb, groups, cus, false);
        if (c.entry >= 0) return c;
    }
    if (m <= 64) {
        const int64_t t64 = groups * ((N + 63) / 64);
        if (t64 * 2 >= 3 * cus) c.entry = find_entry(layout, 64, 128, 1, 4, 3);
        else if (layout == kDense && nkb >= 64) c.entry = find_entry(layout, 64, 64, 1, 4, 6);  // long K
        else c.entry = find_entry(layout, 64, 64, 1, 4, 4);
    } else if (m <= 128) {
        const int64_t K = (int64_t)nkb * 128;
        if (N >= 16384 || K >= 8192) c.entry = find_entry(layout, 128, 128, 2, 4, 3);
        else c.entry = find_entry(layout, 64, 64, 1, 4, 4);
    } else if (m >= 1024 && N >= 256 && layout == kDense) {
        // N tile width: the least estimated time of the busiest workgroup, i.e. its K blocks under
        // the schedule launch() will run (whole tiles, or stream-K for the leftover tiles), times
        // the time of one K block of that width, plus stream-K's exchange where it is taken: about
        // 0.07 K-block times per column of the tile for each segment a tile has beyond its first
        // (each adds a partial tile written and read).  Measured on MI355X: one round of 256 whole
        // tiles at K = 7168 takes 121.9, 110.6 and 101.0 us for widths 256, 192 and 160 (block
        // costs 1, 0.91, 0.83); 4096 x 1536 x 7168 with stream-K takes 82.2 us in 256 x 256 tiles
        // (21 K blocks per workgroup, three segments per tile), 68.0 in 256 x 192 (28, two) and
        // 77.1 in 256 x 160 (35, two).  Against the choice by whole rounds this picks 256 x 192 with
        // stream-K there and for 4096 x 2112 x 7168 (91.3 against 91.8 us); ties keep the wider tile.
        struct Width { int bn; int64_t block_cost; } widths[] = {{256, 100}, {192, 91}, {160, 83}};
        int64_t best = -1;
        const int64_t tiles_m = (m + 255) / 256;
        for (const Width& w : widths) {
            const int e = find_entry(layout, 256, w.bn, 4, 2, 2);
            if (e < 0) continue;
            const int64_t tiles = tiles_m * ((N + w.bn - 1) / w.bn);
            int64_t per = 0, extra = 0, blocks = 0;
            const bool sk = stream_k_plan(tiles, cus, nkb, w.bn, &per, &extra, &blocks);
            const int64_t segments = sk ? (nkb + per - 1) / per : 1;     // per tile, about
            const int64_t cost = blocks * w.block_cost + 7 * w.bn * (segments - 1);
            if (best < 0 || cost < best) {
                best = cost;
                c.entry = e;
            }
        }
    } else if (m >= 1024 && N >= 256 && layout == kContiguous) {
        c.entry = find_entry(layout, 256, 256, 4, 2, 2);
    } else {
        c.entry = find_entry(layout, 128, 128, 2, 2, 4);
    }
    if (c.entry < 0) return c;
    const KernelEntry& e = kernels()[c.entry];
    const int64_t tiles = groups * ((m + e.bm - 1) / e.bm) * ((N + e.bn - 1) / e.bn);
    c.split = pick_split(tiles, nkb, cus);
    return c;
}

// specialize: run the tiled kernel compiled at run time with this call's N and K (the launch
// shape is the table's choice either way).
// noalloc: split-K partials and counters in the device's static scratch (fp8gemm_nt_noalloc)
// instead of the stream's workspace; launches that need more than it holds are refused.
int launch(int layout, KernelArgs& a, int64_t expected_rows, hipStream_t stream, bool fp4 = false,
           bool specialize = false, bool noalloc = false) {
    DeviceState* d = nullptr;
    int st = device_state(&d);
    if (st != FP8GEMM_OK) return st;
    int cap = g_cu_cap.load();
    int cus = (cap > 0 && cap < d->cus) ? cap : d->cus;
    Choice c = choose(layout, a.rows, a.N, a.nkb, expected_rows, a.G, cus, fp4);
    if (c.entry < 0) return FP8GEMM_ERR_UNSUPPORTED;
    const KernelEntry& e = kernels()[c.entry];
    const JitKernel* jk = nullptr;
    if (specialize) {
        if (e.kind != kKindTiled) return FP8GEMM_ERR_UNSUPPORTED;
        st = jit_kernel(d->id, e, c.entry, a.N, a.K, &jk);
        if (st != FP8GEMM_OK) return st;
    }
    if (e.kind == kKindStream && (int64_t)std::max(e.bm, e.bn + 1) * a.K >= (int64_t(1) << 31))
        return FP8GEMM_ERR_UNSUPPORTED;     // a forced stream configuration beyond its offsets

    a.tiles_m = (int32_t)((a.rows + e.bm - 1) / e.bm);
    a.tiles_n = (int32_t)((a.N + e.bn - 1) / e.bn);
    int split = e.splitk ? std::min(c.split, a.nkb) : 1;
    a.kb_per_split = (a.nkb + split - 1) / split;
    a.splits = (a.nkb + a.kb_per_split - 1) / a.kb_per_split;
    const int64_t groups = (layout == kMasked) ? a.G : 1;
    const int64_t units = groups * a.tiles_m * a.tiles_n * a.splits;
    a.div_groups = make_fastdiv((uint32_t)groups);
    if (units >= (int64_t(1) << 30)) return FP8GEMM_ERR_UNSUPPORTED;   // unit ids stay far below 2^31
    a.units = (int32_t)units;
    // bands of M tiles in the unit order: 4 for 256-row tiles, 8 for 128-row contiguous tiles
    a.group_m = (layout != kMasked && a.tiles_m >= 8) ? (layout == kDense || e.bm >= 256 ? 4 : 8) : 1;
    a.div_splits = make_fastdiv((uint32_t)a.splits);
    a.div_tiles_m = make_fastdiv((uint32_t)a.tiles_m);
    a.div_tiles_n = make_fastdiv((uint32_t)a.tiles_n);
    a.div_group_tiles = make_fastdiv((uint32_t)(a.tiles_m * a.tiles_n));
    a.div_band_units = make_fastdiv((uint32_t)(a.group_m * a.tiles_n));
    a.div_band_h = make_fastdiv((uint32_t)a.group_m);
    const int bands = (a.tiles_m + a.group_m - 1) / a.group_m;
    a.div_band_h_last = make_fastdiv((uint32_t)(a.tiles_m - a.group_m * (bands - 1)));
    a.err = d->err;
    a.ws = nullptr;
    a.counters = nullptr;
    int64_t slots = (int64_t)cus * (jk ? jk->occupancy : d->occupancy[c.entry]);

    // Stream-K for the tiles after the last full round of whole tiles (dense 256-row tiles, which
    // take no K split): instead of a last, partly idle round, the leftover tiles' K blocks are
    // shared out evenly over the grid (sk_start in fp8gemm_args.h), and tiles shared by several
    // workgroups are summed by the exchange in the kernel.  On MI355X a partly empty round costs
    // as much as a full one (4096 x N x 16384 with 384, 448 and 512 tiles on 256 CUs: 464, 477
    // and 496 us), while the exchange and the stream-K phase's weaker L2 sharing cost several K
    // blocks' time.  So it is taken when it saves a workgroup at least stream_k_min_blocks K
    // blocks against whole tiles; measured (whole tiles -> stream-K, us, blocks saved):
    //   256 x 256: 4096x7168x2048 79.5 -> 87.0 (4), 2048x7168x7168 104.7 -> 111.1 (7),
    //     6144x2112x7168 104.4 -> 112.0 (8), 4096x7168x4096 130.0 -> 131.0 (8),
    //     4096x3072x7168 101.1 -> 99.6 (14), 4096x7168x7168 212.4 -> 202.5 (14),
    //     8192x7168x7168 411.3 -> 385.1 (28), 4096x7168x16384 465.1 -> 423.3 (32);
    //   256 x 192: 4096x2112x7168 94.6 -> 91.3 (17), 4096x1536x7168 90.7 -> 68.0 (28),
    //     4096x2112x16384 190.5 -> 165.3 (39); threshold 9, between its neighbours';
    //   256 x 160: 4096x2112x4096 57.7 -> 61.4 (4), 4096x2112x7168 95.5 -> 92.6 (7),
    //     4096x2112x16384 183.6 -> 171.1 (16), 3072x2112x7168 85.3 -> 78.8 (19).
    // Every gain measured had a workgroup take at least 0.43 of a tile's K blocks (at most three
    // segments per tile); a range shorter than a third of a tile keeps whole tiles, since each
    // further segment adds a partial that the last arrival reads.
    // FP8GEMM_STREAMK=0 turns it off, =1 on wherever leftover tiles exist.  Not for the run-time
    // specialised kernels (compiled without the exchange) nor for the allocation-free entry point.
    bool streamk = false;
    if (layout == kDense && e.kind == kKindTiled && e.bm == 256 && a.splits == 1 && !noalloc && !jk) {
        const int64_t P = slots, T = a.units;
        const int64_t full = T / P, R = T % P;
        int64_t per = 0, extra = 0, blocks = 0;
        const bool want = stream_k_plan(T, P, a.nkb, e.bn, &per, &extra, &blocks);
        const size_t need = (size_t)(2 * P) * e.bm * e.bn * sizeof(float);
        if (want && need <= workspace_partial_bytes(d->cus)) {
            // a stream with no workspace that is being captured keeps whole tiles (UNSUPPORTED
            // from workspace: nothing may be allocated during capture)
            Workspace* w = nullptr;
            st = workspace(d, stream, need, (size_t)R, &w);
            if (st != FP8GEMM_OK && st != FP8GEMM_ERR_UNSUPPORTED) return st;
            if (st == FP8GEMM_OK) {
                streamk = true;
                a.units = (int32_t)(full * P);
                a.sk_tiles = (int32_t)R;
                a.sk_per = (int32_t)per;
                a.sk_extra = (int32_t)extra;
                a.ws = w->partials;
                a.counters = w->counters;
            }
        }
    }
    if (a.splits > 1) {
        const int64_t tiles = (int64_t)a.units / a.splits;
        const size_t partial_bytes = (size_t)a.units * e.bm * e.bn * sizeof(float);
        if (noalloc) {
            if (partial_bytes > kScratchPartialBytes || (size_t)tiles > kScratchCounters)
                return FP8GEMM_ERR_UNSUPPORTED;
            a.ws = d->scratch.partials;
            a.counters = d->scratch.counters;
        } else {
            Workspace* w = nullptr;
            st = workspace(d, stream, partial_bytes, (size_t)tiles, &w);
            if (st != FP8GEMM_OK) return st;
            a.ws = w->partials;
            a.counters = w->counters;
        }
    }
    // a stream-K launch needs exactly `slots` workgroups (its schedule is cut for that many)
    int64_t grid = streamk ? slots : std::min<int64_t>(a.units, slots);
    if (grid <= 0) return FP8GEMM_OK;
    const char* lname = layout == kDense ? "nt" : (layout == kContiguous ? "contiguous" : (fp4 ? "masked fp8xfp4" : "masked"));
    if (e.kind == kKindStream)
        std::snprintf(g_last_config, sizeof g_last_config,
                      "%s stream tile=%dx%d waves=%d jn=%d phase=%d depth=%d split=%d kb_per_split=%d "
                      "units=%lld grid=%lld",
                      lname, e.bm, e.bn, e.waves_n, e.jn, e.kp, e.stages, a.splits, a.kb_per_split,
                      (long long)a.units, (long long)grid);
    else
        std::snprintf(g_last_config, sizeof g_last_config,
                      "%s%s tile=%dx%d waves=%dx%d stages=%d split=%d kb_per_split=%d units=%lld grid=%lld",
                      lname, jk ? " specialized" : "", e.bm, e.bn, e.waves_m, e.waves_n, e.stages, a.splits,
                      a.kb_per_split, (long long)a.units, (long long)grid);
    if (streamk) {
        const size_t n = std::strlen(g_last_config);
        std::snprintf(g_last_config + n, sizeof g_last_config - n, " streamk_tiles=%d blocks_per_wg=%d",
                      a.sk_tiles, a.sk_per);
    }
    if (std::getenv("FP8GEMM_LOG")) std::fprintf(stderr, "[fp8gemm] %s\n", g_last_config);
    if (jk) {
        // the argument block travels by value with its size stated: HIP copies the bytes into the
        // launch (or, under stream capture, into the graph's kernel node) before returning
        size_t arg_bytes = sizeof(KernelArgs);
        void* extra[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, &a, HIP_LAUNCH_PARAM_BUFFER_SIZE, &arg_bytes,
                         HIP_LAUNCH_PARAM_END};
        if (hipModuleLaunchKernel(jk->fn, (unsigned)grid, 1, 1, (unsigned)e.threads, 1, 1, 0, stream, nullptr,
                                  extra) != hipSuccess)
            return FP8GEMM_ERR_LAUNCH;
        return FP8GEMM_OK;
    }
    e.launch(dim3((unsigned)grid), a, stream);
    if (hipGetLastError() != hipSuccess) return FP8GEMM_ERR_LAUNCH;
    return FP8GEMM_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shared checks of the operand pointers (non-null, aligned).
int check_ptrs(const void* A, const float* sa, const void* B, const float* sb, const void* D) {
    if (!A || !sa || !B || !sb || !D) return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || !aligned(sa, 4) || !aligned(sb, 4))
        return FP8GEMM_ERR_MISALIGNED;
    return FP8GEMM_OK;
}

// Sizes the kernels index with 32-bit per-lane offsets: a tile row offset r*K (r < 256) must fit.
constexpr int64_t kMaxK = int64_t(1) << 24;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxBytes = int64_t(1) << 40;

int check_k(int64_t K) {
    if (K <= 0 || K % 128 != 0) return FP8GEMM_ERR_BAD_SHAPE;
    if (K > kMaxK) return FP8GEMM_ERR_UNSUPPORTED;
    return FP8GEMM_OK;
}

// Shared launch of the activation quantiser over G groups of `rows` rows; with `swiglu` the
// input rows hold 2K values (gate | up) and the quantised values are silu(gate) * up.
int quantize(const void* X, void* A, float* sa, const int32_t* masked_m, int32_t G, int64_t rows,
             int64_t K, bool swiglu, hipStream_t stream) {
    const int64_t nkb = K / 128;
    const int64_t blocks = (int64_t)G * rows * nkb;
    if (blocks >= (int64_t(1) << 31)) return FP8GEMM_ERR_UNSUPPORTED;  // block ids stay below 2^31
    DeviceState* d = nullptr;
    int st = device_state(&d);
    if (st != FP8GEMM_OK) return st;
    QuantArgs q{};
    q.X = static_cast<const uint16_t*>(X);
    q.A = static_cast<uint8_t*>(A);
    q.sa = sa;
    q.masked_m = masked_m;
    q.err = d->err;
    q.rows = (int32_t)rows;
    q.K = (int32_t)K;
    q.nkb = (int32_t)nkb;
    q.G = G;
    q.blocks = (uint32_t)blocks;
    q.div_nkb = make_fastdiv((uint32_t)nkb);
    q.div_rows = make_fastdiv((uint32_t)rows);
    const int64_t wgs = (blocks + kQuantBlocksPerWG - 1) / kQuantBlocksPerWG;
    const int64_t grid = (wgs + 7) / 8 * 8;
    std::snprintf(g_last_config, sizeof g_last_config, "%s blocks_per_wg=%d grid=%lld",
                  swiglu ? "swiglu_quantize_1x128" : "quantize_1x128", kQuantBlocksPerWG, (long long)grid);
    if (swiglu) launch_swiglu_quantize(q, dim3((unsigned)grid), stream);
    else launch_quantize_1x128(q, dim3((unsigned)grid), stream);
    if (hipGetLastError() != hipSuccess) return FP8GEMM_ERR_LAUNCH;
    return FP8GEMM_OK;
}

// Dense NT GEMM, from the table's kernel or its run-time specialisation.
int dense(const void* A, const float* sa, const void* B, const float* sb, void* D, int64_t M, int64_t N,
          int64_t K, void* stream, bool specialize, bool noalloc = false) {
    if (M < 0 || N < 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(K);
    if (st != FP8GEMM_OK) return st;
    if (M > kMaxRows || N > kMaxRows || M * K >= kMaxBytes || N * K >= kMaxBytes)
        return FP8GEMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8GEMM_OK;
    st = check_ptrs(A, sa, B, sb, D);
    if (st != FP8GEMM_OK) return st;
    KernelArgs a{};
    a.A = static_cast<const uint8_t*>(A);
    a.sa = sa;
    a.B = static_cast<const uint8_t*>(B);
    a.sb = sb;
    a.D = static_cast<uint16_t*>(D);
    a.rows = M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.G = 1;
    a.nkb = (int32_t)(K / 128);
    a.nnb = (int32_t)((N + 127) / 128);
    return launch(kDense, a, M, static_cast<hipStream_t>(stream), false, specialize, noalloc);
}

}  // namespace

extern "C" {

int fp8gemm_quantize_1x128(const void* X, void* A, float* sa, int64_t M, int64_t K, void* stream) {
    if (M < 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(K);
    if (st != FP8GEMM_OK) return st;
    if (M > kMaxRows || 2 * M * K >= kMaxBytes) return FP8GEMM_ERR_UNSUPPORTED;
    if (M == 0) return FP8GEMM_OK;
    if (!X || !A || !sa) return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(X, 16) || !aligned(A, 16) || !aligned(sa, 4)) return FP8GEMM_ERR_MISALIGNED;
    return quantize(X, A, sa, nullptr, 1, M, K, false, static_cast<hipStream_t>(stream));
}

int fp8gemm_quantize_1x128_masked(const void* X, void* A, float* sa, const int32_t* masked_m,
                                  int32_t G, int64_t M_max, int64_t K, void* stream) {
    if (G <= 0 || M_max < 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(K);
    if (st != FP8GEMM_OK) return st;
    if ((int64_t)G * M_max > kMaxRows || 2 * (int64_t)G * M_max * K >= kMaxBytes)
        return FP8GEMM_ERR_UNSUPPORTED;
    if (M_max == 0) return FP8GEMM_OK;
    if (!X || !A || !sa || !masked_m) return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(X, 16) || !aligned(A, 16) || !aligned(sa, 4) || !aligned(masked_m, 4))
        return FP8GEMM_ERR_MISALIGNED;
    return quantize(X, A, sa, masked_m, G, M_max, K, false, static_cast<hipStream_t>(stream));
}

int fp8gemm_swiglu_quantize_1x128(const void* X, void* A, float* sa, int64_t M, int64_t I, void* stream) {
    if (M < 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(I);
    if (st != FP8GEMM_OK) return st;
    if (M > kMaxRows || 4 * M * I >= kMaxBytes) return FP8GEMM_ERR_UNSUPPORTED;
    if (M == 0) return FP8GEMM_OK;
    if (!X || !A || !sa) return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(X, 16) || !aligned(A, 16) || !aligned(sa, 4)) return FP8GEMM_ERR_MISALIGNED;
    return quantize(X, A, sa, nullptr, 1, M, I, true, static_cast<hipStream_t>(stream));
}

int fp8gemm_swiglu_quantize_1x128_masked(const void* X, void* A, float* sa, const int32_t* masked_m,
                                         int32_t G, int64_t M_max, int64_t I, void* stream) {
    if (G <= 0 || M_max < 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(I);
    if (st != FP8GEMM_OK) return st;
    if ((int64_t)G * M_max > kMaxRows || 4 * (int64_t)G * M_max * I >= kMaxBytes) return FP8GEMM_ERR_UNSUPPORTED;
    if (M_max == 0) return FP8GEMM_OK;
    if (!X || !A || !sa || !masked_m) return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(X, 16) || !aligned(A, 16) || !aligned(sa, 4) || !aligned(masked_m, 4))
        return FP8GEMM_ERR_MISALIGNED;
    return quantize(X, A, sa, masked_m, G, M_max, I, true, static_cast<hipStream_t>(stream));
}

int fp8gemm_moe_expert_masked(const void* A, const float* sa, const void* W1, const float* s1,
                              const void* W2, const float* s2, const int32_t* masked_m, void* Y1,
                              void* Hq, float* sh, void* out, int32_t G, int64_t M_max, int64_t H,
                              int64_t I, int64_t expected_m, void* stream) {
    // every check of the three steps before anything is enqueued
    if (G <= 0 || M_max < 0 || expected_m < 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(H);
    if (st == FP8GEMM_OK) st = check_k(I);
    if (st != FP8GEMM_OK) return st;
    const int64_t rows = (int64_t)G * M_max;
    if (rows > kMaxRows || 2 * I > kMaxRows || rows * H >= kMaxBytes || 4 * rows * I >= kMaxBytes ||
        2 * (int64_t)G * I * H >= kMaxBytes || 2 * rows * H >= kMaxBytes)
        return FP8GEMM_ERR_UNSUPPORTED;
    if (M_max == 0) return FP8GEMM_OK;
    if (!A || !sa || !W1 || !s1 || !W2 || !s2 || !masked_m || !Y1 || !Hq || !sh || !out)
        return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(A, 16) || !aligned(W1, 16) || !aligned(W2, 16) || !aligned(Y1, 16) || !aligned(Hq, 16) ||
        !aligned(out, 16) || !aligned(sa, 4) || !aligned(s1, 4) || !aligned(s2, 4) || !aligned(sh, 4) ||
        !aligned(masked_m, 4))
        return FP8GEMM_ERR_MISALIGNED;
    st = fp8gemm_grouped_masked(A, sa, W1, s1, masked_m, Y1, G, M_max, 2 * I, H, expected_m, stream);
    if (st != FP8GEMM_OK) return st;
    st = fp8gemm_swiglu_quantize_1x128_masked(Y1, Hq, sh, masked_m, G, M_max, I, stream);
    if (st != FP8GEMM_OK) return st;
    return fp8gemm_grouped_masked(Hq, sh, W2, s2, masked_m, out, G, M_max, H, I, expected_m, stream);
}

int fp8gemm_nt(const void* A, const float* sa, const void* B, const float* sb, void* D, int64_t M,
               int64_t N, int64_t K, void* stream) {
    return dense(A, sa, B, sb, D, M, N, K, stream, false);
}

int fp8gemm_nt_noalloc(const void* A, const float* sa, const void* B, const float* sb, void* D, int64_t M,
                       int64_t N, int64_t K, void* stream) {
    return dense(A, sa, B, sb, D, M, N, K, stream, false, true);
}

int fp8gemm_nt_specialized(const void* A, const float* sa, const void* B, const float* sb, void* D, int64_t M,
                           int64_t N, int64_t K, void* stream) {
    return dense(A, sa, B, sb, D, M, N, K, stream, true);
}

int fp8gemm_specialize_nt(int64_t M, int64_t N, int64_t K, double* compile_ms) {
    if (M <= 0 || N <= 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(K);
    if (st != FP8GEMM_OK) return st;
    if (M > kMaxRows || N > kMaxRows || M * K >= kMaxBytes || N * K >= kMaxBytes) return FP8GEMM_ERR_UNSUPPORTED;
    DeviceState* d = nullptr;
    st = device_state(&d);
    if (st != FP8GEMM_OK) return st;
    int cap = g_cu_cap.load();
    int cus = (cap > 0 && cap < d->cus) ? cap : d->cus;
    Choice c = choose(kDense, M, N, (int)(K / 128), M, 1, cus, false);
    if (c.entry < 0) return FP8GEMM_ERR_UNSUPPORTED;
    const int before = jit_cache_size();
    const JitKernel* jk = nullptr;
    st = jit_kernel(d->id, kernels()[c.entry], c.entry, (int)N, (int)K, &jk);
    if (st != FP8GEMM_OK) return st;
    if (compile_ms) *compile_ms = jit_cache_size() > before ? jk->compile_ms : 0.0;
    return FP8GEMM_OK;
}

int fp8gemm_specialized_code_object(int layout, int bm, int bn, int waves_m, int waves_n, int stages, int64_t N,
                                    int64_t K, void* buf, size_t* size, char* log, int log_len) {
    if (!size) return FP8GEMM_ERR_NULL_PTR;
    if (N <= 0 || N > kMaxRows) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(K);
    if (st != FP8GEMM_OK) return st;
    const int idx = find_entry(layout, bm, bn, waves_m, waves_n, stages);
    if (idx < 0) return FP8GEMM_ERR_BAD_SHAPE;
    std::vector<char> code;
    std::string lowered, text;
    st = jit_compile(kernels()[idx], (int)N, (int)K, &code, &lowered, &text);
    if (log && log_len > 0) std::snprintf(log, (size_t)log_len, "%s", st == FP8GEMM_OK ? lowered.c_str() : text.c_str());
    if (st != FP8GEMM_OK) return st;
    const size_t cap = *size;
    *size = code.size();
    if (!buf) return FP8GEMM_OK;
    if (cap < code.size()) return FP8GEMM_ERR_BAD_SHAPE;
    std::memcpy(buf, code.data(), code.size());
    return FP8GEMM_OK;
}

int fp8gemm_specialized_count(void) { return jit_cache_size(); }

int fp8gemm_grouped_contiguous(const void* A, const float* sa, const void* B, const float* sb,
                               const int32_t* m_indices, void* D, int64_t M_total, int64_t N,
                               int64_t K, int32_t G, void* stream) {
    if (M_total < 0 || N < 0 || G <= 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(K);
    if (st != FP8GEMM_OK) return st;
    if (M_total > kMaxRows || N > kMaxRows || M_total * K >= kMaxBytes || (int64_t)G * N * K >= kMaxBytes)
        return FP8GEMM_ERR_UNSUPPORTED;
    if (M_total == 0 || N == 0) return FP8GEMM_OK;
    st = check_ptrs(A, sa, B, sb, D);
    if (st != FP8GEMM_OK) return st;
    if (!m_indices) return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(m_indices, 4)) return FP8GEMM_ERR_MISALIGNED;
    KernelArgs a{};
    a.A = static_cast<const uint8_t*>(A);
    a.sa = sa;
    a.B = static_cast<const uint8_t*>(B);
    a.sb = sb;
    a.D = static_cast<uint16_t*>(D);
    a.m_indices = m_indices;
    a.rows = M_total;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.G = G;
    a.nkb = (int32_t)(K / 128);
    a.nnb = (int32_t)((N + 127) / 128);
    return launch(kContiguous, a, M_total, static_cast<hipStream_t>(stream));
}

int fp8gemm_grouped_masked(const void* A, const float* sa, const void* B, const float* sb,
                           const int32_t* masked_m, void* D, int32_t G, int64_t M_max, int64_t N,
                           int64_t K, int64_t expected_m, void* stream) {
    if (G <= 0 || M_max < 0 || N < 0 || expected_m < 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(K);
    if (st != FP8GEMM_OK) return st;
    if ((int64_t)G * M_max > kMaxRows || N > kMaxRows || (int64_t)G * M_max * K >= kMaxBytes ||
        (int64_t)G * N * K >= kMaxBytes)
        return FP8GEMM_ERR_UNSUPPORTED;
    if (M_max == 0 || N == 0) return FP8GEMM_OK;
    st = check_ptrs(A, sa, B, sb, D);
    if (st != FP8GEMM_OK) return st;
    if (!masked_m) return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(masked_m, 4)) return FP8GEMM_ERR_MISALIGNED;
    KernelArgs a{};
    a.A = static_cast<const uint8_t*>(A);
    a.sa = sa;
    a.B = static_cast<const uint8_t*>(B);
    a.sb = sb;
    a.D = static_cast<uint16_t*>(D);
    a.masked_m = masked_m;
    a.rows = M_max;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.G = G;
    a.nkb = (int32_t)(K / 128);
    a.nnb = (int32_t)((N + 127) / 128);
    int64_t hint = expected_m > 0 ? std::min(expected_m, M_max) : M_max;
    return launch(kMasked, a, hint, static_cast<hipStream_t>(stream));
}

int fp8gemm_fp8fp4_grouped_masked(const void* A, const float* sa, const void* B, const uint8_t* sb,
                                  const int32_t* masked_m, void* D, int32_t G, int64_t M_max, int64_t N,
                                  int64_t K, int64_t expected_m, void* stream) {
    if (G <= 0 || M_max < 0 || N < 0 || expected_m < 0) return FP8GEMM_ERR_BAD_SHAPE;
    int st = check_k(K);
    if (st != FP8GEMM_OK) return st;
    if ((int64_t)G * M_max > kMaxRows || N > kMaxRows || (int64_t)G * M_max * K >= kMaxBytes ||
        (int64_t)G * N * K >= kMaxBytes || 257 * K / 2 >= (int64_t(1) << 31))
        return FP8GEMM_ERR_UNSUPPORTED;
    if (M_max == 0 || N == 0) return FP8GEMM_OK;
    if (!A || !sa || !B || !sb || !D || !masked_m) return FP8GEMM_ERR_NULL_PTR;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(D, 16) || !aligned(sa, 4) || !aligned(sb, 4) ||
        !aligned(masked_m, 4))
        return FP8GEMM_ERR_MISALIGNED;
    KernelArgs a{};
    a.A = static_cast<const uint8_t*>(A);
    a.sa = sa;
    a.B = static_cast<const uint8_t*>(B);
    a.sbe = sb;
    a.D = static_cast<uint16_t*>(D);
    a.masked_m = masked_m;
    a.rows = M_max;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.G = G;
    a.nkb = (int32_t)(K / 128);
    a.nnb = (int32_t)((N + 127) / 128);
    int64_t hint = expected_m > 0 ? std::min(expected_m, M_max) : M_max;
    return launch(kMasked, a, hint, static_cast<hipStream_t>(stream), true);
}

const char* fp8gemm_status_string(int status) {
    switch (status) {
        case FP8GEMM_OK: return "ok";
        case FP8GEMM_ERR_NULL_PTR: return "null pointer";
        case FP8GEMM_ERR_BAD_SHAPE: return "bad shape";
        case FP8GEMM_ERR_MISALIGNED: return "misaligned pointer";
        case FP8GEMM_ERR_UNSUPPORTED: return "unsupported size";
        case FP8GEMM_ERR_LAUNCH: return "kernel launch failed";
        case FP8GEMM_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int fp8gemm_init(void) {
    DeviceState* d = nullptr;
    return device_state(&d);
}

int fp8gemm_prepare_stream(void* stream) {
    DeviceState* d = nullptr;
    int st = device_state(&d);
    if (st != FP8GEMM_OK) return st;
    Workspace* w = nullptr;
    return workspace(d, static_cast<hipStream_t>(stream), 0, 0, &w);
}

int fp8gemm_set_num_cus(int n) {
    if (n < 0) return FP8GEMM_ERR_BAD_SHAPE;
    g_cu_cap.store(n);
    return FP8GEMM_OK;
}

int fp8gemm_last_config(char* buf, int len) {
    if (!buf || len <= 0) return FP8GEMM_ERR_NULL_PTR;
    std::snprintf(buf, (size_t)len, "%s", g_last_config);
    return FP8GEMM_OK;
}

int fp8gemm_read_device_error(void* stream, int32_t* err) {
    if (!err) return FP8GEMM_ERR_NULL_PTR;
    DeviceState* d = nullptr;
    int st = device_state(&d);
    if (st != FP8GEMM_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipStreamSynchronize(s) != hipSuccess) return FP8GEMM_ERR_HIP;
    int32_t v = 0;
    if (hipMemcpy(&v, d->err, sizeof v, hipMemcpyDeviceToHost) != hipSuccess) return FP8GEMM_ERR_HIP;
    if (hipMemset(d->err, 0, sizeof v) != hipSuccess) return FP8GEMM_ERR_HIP;
    *err = v;
    return FP8GEMM_OK;
}

}  // extern "C"
