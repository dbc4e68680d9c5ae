// Host-side logic of the NVFP4 GEMV library: argument validation, the launch
// plan (kernel variant, K split, grid, LDS and workspace sizes) and the order
// in which an entry point validates, plans, finds its workspace and launches.
//
// Plain C++17 with no HIP types, so that the same code is compiled into the
// library (nvfp4_gemv.hip) and into host-only checks built with g++ and the
// address and undefined-behaviour sanitizers.  The launch orchestration takes
// a "backend" with four calls (current device, library-owned workspace,
// fixed-size scratch of a device, launch of a plan): the library's backend
// calls HIP, a test backend can fail each of them on purpose.
//
// The operation the plans serve is the NVFP4 batched GEMV of "nvFP4 Batch
// GEMV算子系列(下)", section "NVFP4 Batched GEMV 概念阐述" (16-element scale
// blocks, so k must be a multiple of 16).
//
// Not part of the C ABI.
#ifndef NVFP4_GEMV_PLAN_H
#define NVFP4_GEMV_PLAN_H

#include <climits>
#include <cstddef>
#include <cstdint>

#include "nvfp4_gemv.h"

namespace nvfp4plan {

constexpr int kLanes = 64;               // lanes of a CDNA wave
constexpr int64_t kIterElems = 2048;     // K elements one wave covers per row per iteration
constexpr int64_t kMaxChunk = 16384;     // K elements staged in LDS per workgroup (32 KiB)
constexpr int64_t kMinSplitChunk = 2048;
constexpr int64_t kTargetGroups = 512;   // workgroups wanted before splitting K
constexpr int64_t kComputeUnits = 256;   // MI355X: 8 XCDs x 32 CUs
constexpr int kReduceThreads = 256;
constexpr int kGenericWaves = 4;
// The row-tile kernel addresses a tile's rows through one descriptor with
// 32-bit offsets; it takes K up to this bound.
constexpr int64_t kTileMaxK = int64_t(1) << 26;
// Largest split-K workspace the no-allocation entry point can use: the size
// of its fixed device array.
constexpr size_t kNoAllocScratchBytes = NVFP4_GEMV_NOALLOC_SCRATCH_BYTES;

// x staging of a fast variant: fp16 x~ in LDS (gemv_fast), packed codes in LDS
// (gemv_fastp), no staging (gemv_fastg, x read next to A every iteration), or
// row tiles (16, 8 or 4 rows) whose waves split K and keep x~ of their slice
// in registers (gemv_tile).
enum XForm { kXHalf = 0, kXPacked = 1, kXGlobal = 2, kXTile = 3 };

struct Variant {
    int R, U, W;
    int xform;
};
// Listed as {rows per wave, iterations in flight, waves, x staging}.
constexpr Variant kVariants[] = {
    {2, 4, 7, kXHalf},    {1, 8, 4, kXHalf},    {2, 4, 4, kXHalf},    {2, 2, 4, kXHalf},
    {4, 2, 4, kXHalf},    {2, 4, 8, kXHalf},    {1, 8, 8, kXHalf},    {4, 1, 4, kXHalf},
    {2, 1, 8, kXHalf},    {1, 4, 4, kXHalf},    {2, 2, 4, kXPacked},  {4, 1, 4, kXPacked},
    {4, 2, 4, kXPacked},  {2, 4, 8, kXPacked},  {4, 2, 8, kXPacked},  {1, 4, 8, kXPacked},
    {2, 4, 7, kXGlobal},  {2, 2, 7, kXGlobal},  {4, 2, 7, kXGlobal},  {2, 4, 4, kXGlobal},
    {1, 8, 7, kXGlobal},  {4, 1, 8, kXGlobal},  {16, 1, 8, kXTile},   {16, 1, 4, kXTile},
    {16, 1, 2, kXTile},   {16, 1, 1, kXTile},   {8, 1, 1, kXTile},    {8, 1, 2, kXTile},
    {4, 1, 1, kXTile},    {4, 1, 2, kXTile},    {4, 1, 8, kXTile},    {4, 1, 4, kXTile},
    {8, 1, 4, kXTile},
};
constexpr int kNumVariants = static_cast<int>(sizeof(kVariants) / sizeof(kVariants[0]));

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Default fast variant (0-based) by the number of 1 KiB K-iterations per row
// of one workgroup's K-range, from MI355X measurements on the decode, batched,
// Gaussian and short-K workloads.  Rows of 6 to 8 iterations (the decode
// weight's 8) are best read as 4-row tiles of 8 waves: each wave then holds
// one 1 KiB slice of 4 rows, all of it in flight at once, and a workgroup
// reads 16-32 KiB of A, the shape in which a plain read of such a weight is
// fastest (11.84 us against 12.23 for the staged {2, 4, 7} in an alternating
// A/B on one MI355X), as long as those tiles alone fill the GPU (at least 4
// per compute unit; a tile's 8 waves cannot split K any further).  Longer
// rows, and fewer rows, keep the staged {2, 4, 7}, which keeps every wave's
// rows in flight over any number of iterations and splits K across
// workgroups when its groups are few; with 3 to 5
// iterations x read next to A beats staging it; rows of one or two
// iterations are best read as row tiles, whose loads are all in flight at
// once: rows of one iteration as 4-row tiles of one wave (many small waves,
// little arithmetic left in each when its last load lands), rows of two as
// 16-row tiles of two waves.
inline int default_variant(int64_t l, int64_t m, int64_t k) {
    const int64_t nit = ceil_div(k < kMaxChunk ? k : kMaxChunk, kIterElems);
    const int64_t nit_all = ceil_div(k, kIterElems);
    if (nit_all > 8) return 0;   // {2, 4, 7} staged
    if (nit >= 6) return l * ceil_div(m, int64_t(4)) >= 4 * kComputeUnits ? 30 : 0;   // 4-row tile, 8 waves
    if (nit >= 3) return 19;     // {2, 4, 4} x read next to A
    if (nit == 2) return 24;     // 16-row tile, 2 waves
    return 28;                   // 4-row tile, 1 wave
}

struct Plan {
    int path;           // NVFP4_GEMV_PATH_FAST or _GENERIC
    int variant;        // 0-based fast-kernel variant
    int64_t ksplit;
    int64_t kchunk;
    int64_t row_blocks; // row blocks per batch
    int64_t groups;
    int threads;
    size_t lds_bytes;
    size_t ws_bytes;
};

inline int check_shape(int64_t l, int64_t m, int64_t k) {
    if (l < 1 || m < 1 || k < 16 || k % 16 != 0) return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (k >= (int64_t(1) << 31) || l > INT64_MAX / m || l * m >= (int64_t(1) << 31))
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (l * m > INT64_MAX / (k / 2)) return NVFP4_GEMV_ERR_BAD_SHAPE;
    return NVFP4_GEMV_OK;
}

// K split: one LDS stage (16384 elements) per workgroup at most for the
// staged fast kernels; an explicit split must leave every split at least one
// granule (32 elements for the fast kernel, 16 for the generic one) and fit
// one stage.
inline int split_k(int64_t k, int64_t ks_req, int64_t ks_auto, int64_t granule, bool staged,
                   int64_t *ks_out, int64_t *kchunk_out) {
    int64_t ks = ks_req > 0 ? ks_req : ks_auto;
    if (ks_req > 0 && ks > k / granule) return NVFP4_GEMV_ERR_BAD_TUNING;
    int64_t kchunk = ceil_div(ceil_div(k, ks), granule) * granule;
    if (staged && kchunk > kMaxChunk) {
        if (ks_req > 0) return NVFP4_GEMV_ERR_BAD_TUNING;
        kchunk = kMaxChunk;
    }
    *ks_out = ceil_div(k, kchunk);
    *kchunk_out = kchunk;
    return NVFP4_GEMV_OK;
}

// Resolves the launch plan; the shape must already be valid (check_shape).
inline int make_plan(int64_t l, int64_t m, int64_t k, bool aligned, const nvfp4_gemv_tuning_t *t,
                     Plan *p) {
    nvfp4_gemv_tuning_t tun = {NVFP4_GEMV_PATH_AUTO, 0, 0, 0};
    if (t) tun = *t;
    if (tun.reserved != 0 || tun.path < NVFP4_GEMV_PATH_AUTO || tun.path > NVFP4_GEMV_PATH_GENERIC ||
        tun.variant < 0 || tun.ksplit < 0)
        return NVFP4_GEMV_ERR_BAD_TUNING;
    const bool fast_ok = aligned && (k % 32 == 0);
    if (tun.path == NVFP4_GEMV_PATH_FAST && !fast_ok) return NVFP4_GEMV_ERR_BAD_TUNING;
    if (tun.path == NVFP4_GEMV_PATH_GENERIC && tun.variant != 0) return NVFP4_GEMV_ERR_BAD_TUNING;
    if (tun.variant > kNumVariants) return NVFP4_GEMV_ERR_BAD_TUNING;
    p->path = (tun.path == NVFP4_GEMV_PATH_GENERIC || !fast_ok) ? NVFP4_GEMV_PATH_GENERIC
                                                                  : NVFP4_GEMV_PATH_FAST;
    p->variant = tun.variant > 0 ? tun.variant - 1 : default_variant(l, m, k);

    int64_t rows_per_group;
    if (p->path == NVFP4_GEMV_PATH_FAST) {
        const Variant &v = kVariants[p->variant];
        if (v.xform == kXTile && k > kTileMaxK) return NVFP4_GEMV_ERR_BAD_TUNING;
        rows_per_group = v.xform == kXTile ? v.R : static_cast<int64_t>(v.R) * v.W;
        p->threads = v.W * kLanes;
    } else {
        p->variant = 0;
        rows_per_group = kGenericWaves;
        p->threads = kGenericWaves * kLanes;
    }
    p->row_blocks = ceil_div(m, rows_per_group);
    const int64_t groups1 = l * p->row_blocks;
    const bool fast = p->path == NVFP4_GEMV_PATH_FAST;
    const int64_t granule = fast ? 32 : 16;

    const int xform = fast ? kVariants[p->variant].xform : -1;
    const bool staged = xform == kXHalf || xform == kXPacked;
    int64_t ks_auto = staged ? ceil_div(k, kMaxChunk) : 1;
    // A tile's waves already split K: split it across workgroups only while
    // the tiles leave compute units idle, and only as far as every split
    // keeps a slice for each wave.
    const int64_t target = xform == kXTile ? kComputeUnits : kTargetGroups;
    if (groups1 * ks_auto < target) {
        const int64_t want = ceil_div(target, groups1);
        int64_t most = xform == kXTile ? ceil_div(k, kIterElems) / kVariants[p->variant].W
                                       : k / kMinSplitChunk;
        if (most < 1) most = 1;
        const int64_t pick = want < most ? want : most;
        if (pick > ks_auto) ks_auto = pick;
    }
    int64_t ks, kchunk;
    const int st = split_k(k, tun.ksplit, ks_auto, granule, staged, &ks, &kchunk);
    if (st != NVFP4_GEMV_OK) return st;
    p->ksplit = ks;
    p->kchunk = kchunk;
    p->groups = groups1 * ks;
    if (p->groups >= (int64_t(1) << 31)) return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (staged) {
        const Variant &v = kVariants[p->variant];
        const int64_t slots = ceil_div(ceil_div(kchunk, kIterElems), v.U) * v.U;
        // per slot and lane: 64 bytes of fp16 x~, or 16 bytes of codes + 4 of scales
        p->lds_bytes = static_cast<size_t>(slots) * kLanes * (v.xform == kXPacked ? 20 : 64);
    } else {
        p->lds_bytes = 0;
    }
    p->ws_bytes = ks > 1 ? static_cast<size_t>(ks) * static_cast<size_t>(l * m) * sizeof(float) : 0;
    return NVFP4_GEMV_OK;
}

inline bool aligned_for_fast(const void *A, const void *sfA, const void *x, const void *sfx) {
    auto a = [](const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; };
    return a(A, 16) && a(x, 16) && a(sfA, 2) && a(sfx, 2);
}

// Do the byte ranges [p, p + pn) and [q, q + qn) overlap?  Written without
// forming p + pn, which may wrap for addresses near the top.
inline bool overlaps(const void *p, size_t pn, const void *q, size_t qn) {
    if (!p || !q || pn == 0 || qn == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b ? b - a < pn : a - b < qn;
}

// The operands of one GEMV call (device pointers, never dereferenced here).
struct GemvArgs {
    const uint8_t *A, *sfA, *x, *sfx;
    const float *alpha;
    uint16_t *c;
    int64_t l, m, k;
};

inline int validate(const GemvArgs &a) {
    if (!a.A || !a.sfA || !a.x || !a.sfx || !a.c) return NVFP4_GEMV_ERR_NULL_POINTER;
    const int s = check_shape(a.l, a.m, a.k);
    if (s != NVFP4_GEMV_OK) return s;
    if (reinterpret_cast<uintptr_t>(a.c) % 2 != 0 || reinterpret_cast<uintptr_t>(a.alpha) % 4 != 0)
        return NVFP4_GEMV_ERR_ALIGNMENT;
    const size_t rows = static_cast<size_t>(a.l * a.m);
    const size_t cn = rows * 2;
    if (overlaps(a.c, cn, a.A, rows * static_cast<size_t>(a.k / 2)) ||
        overlaps(a.c, cn, a.sfA, rows * static_cast<size_t>(a.k / 16)) ||
        overlaps(a.c, cn, a.x, static_cast<size_t>(a.l) * static_cast<size_t>(a.k / 2)) ||
        overlaps(a.c, cn, a.sfx, static_cast<size_t>(a.l) * static_cast<size_t>(a.k / 16)) ||
        overlaps(a.c, cn, a.alpha, static_cast<size_t>(a.l) * 4))
        return NVFP4_GEMV_ERR_ALIAS;
    return NVFP4_GEMV_OK;
}

// ---- launch orchestration -------------------------------------------------
// Backend interface (all members return plain values, none throws):
//   bool  device(int *dev)                          current device, false if none
//   void *workspace(int dev, void *stream, size_t)  library-owned per-stream
//                                                   workspace, NULL on failure
//   void *scratch(int dev)                          the device's fixed scratch
//                                                   array, NULL on failure
//   int   run(const Plan &, const GemvArgs &, void *ws, void *stream)
//                                                   enqueues the plan's kernels;
//                                                   NVFP4_GEMV_OK or _ERR_LAUNCH

// nvfp4_gemv_launch: default plan, split-K partials in the library-owned
// workspace of (current device, stream).
template <class Backend>
int launch_owned_workspace(Backend &be, const GemvArgs &a, void *stream) {
    int s = validate(a);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(a.l, a.m, a.k, aligned_for_fast(a.A, a.sfA, a.x, a.sfx), nullptr, &p);
    if (s != NVFP4_GEMV_OK) return s;
    void *ws = nullptr;
    if (p.ws_bytes > 0) {
        int dev = -1;
        if (!be.device(&dev)) return NVFP4_GEMV_ERR_DEVICE;
        ws = be.workspace(dev, stream, p.ws_bytes);
        if (!ws) return NVFP4_GEMV_ERR_WORKSPACE;
    }
    return be.run(p, a, ws, stream);
}

// nvfp4_gemv_launch_tuned / _ws: the caller's plan request and workspace.
template <class Backend>
int launch_caller_workspace(Backend &be, const GemvArgs &a, const nvfp4_gemv_tuning_t *tuning,
                            void *workspace, size_t workspace_bytes, void *stream) {
    int s = validate(a);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(a.l, a.m, a.k, aligned_for_fast(a.A, a.sfA, a.x, a.sfx), tuning, &p);
    if (s != NVFP4_GEMV_OK) return s;
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes) return NVFP4_GEMV_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 4 != 0) return NVFP4_GEMV_ERR_ALIGNMENT;
        if (overlaps(workspace, p.ws_bytes, a.c, static_cast<size_t>(a.l * a.m) * 2))
            return NVFP4_GEMV_ERR_ALIAS;
    }
    return be.run(p, a, p.ws_bytes > 0 ? workspace : nullptr, stream);
}

// nvfp4_gemv_launch_noalloc: default plan, split-K partials in the current
// device's fixed scratch array; a plan needing more than the array holds is
// refused before anything else is asked of the backend.
template <class Backend>
int launch_fixed_scratch(Backend &be, const GemvArgs &a, void *stream) {
    int s = validate(a);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(a.l, a.m, a.k, aligned_for_fast(a.A, a.sfA, a.x, a.sfx), nullptr, &p);
    if (s != NVFP4_GEMV_OK) return s;
    void *ws = nullptr;
    if (p.ws_bytes > 0) {
        if (p.ws_bytes > kNoAllocScratchBytes) return NVFP4_GEMV_ERR_WORKSPACE;
        int dev = -1;
        if (!be.device(&dev)) return NVFP4_GEMV_ERR_DEVICE;
        ws = be.scratch(dev);
        if (!ws) return NVFP4_GEMV_ERR_WORKSPACE;
    }
    return be.run(p, a, ws, stream);
}

}  // namespace nvfp4plan

#endif  // NVFP4_GEMV_PLAN_H
