// Host-side plan of the small-N block-scaled GEMM and the grouped (MoE) GEMV:
// shape checks, the kernel variants and their defaults, and the launch plan
// (variant, K split, rows per workgroup, grid and workspace).  The products
// are the NVFP4 batched GEMV's scaled dot products ("nvFP4 Batch GEMV算子系列
// (下)", section "NVFP4 Batched GEMV 概念阐述") against several vectors, and
// the grouped form is the CuTeDSL bridge page's grouped GEMM (section "Kernel
// Launch") with one output column per token.
//
// Plain C++17 with no HIP types, so that the same code is compiled into the
// library (nvfp4_mma.hip) and into host-only checks built with g++ and the
// address and undefined-behaviour sanitizers.  Not part of the C ABI.
#ifndef NVFP4_MMA_PLAN_H
#define NVFP4_MMA_PLAN_H

#include <climits>
#include <cstddef>
#include <cstdint>

#include "nvfp4_gemv.h"
#include "nvfp4_mma.h"

namespace nvfp4mmaplan {

constexpr int kPlanWave = 64;        // lanes of a CDNA wave
constexpr int kTile = 16;            // MFMA tile: 16 weight rows x 16 vectors
constexpr int kWinElems = 256;       // K elements of one window: 128 bytes of every row
constexpr int kLaneElems = 64;       // K elements of one window in one lane (32 code bytes)
constexpr int64_t kMaxFastK = int64_t(1) << 26;   // keeps 32-row descriptors within 31 bits
constexpr int64_t kComputeUnits = 256;            // CUs of an MI355X (8 XCDs x 32)
constexpr int kReduceThreads = 256;
constexpr int kGenericWaves = 4;

enum Form { kMatrixCores = 0, kValuTiles = 1, kLdsStaged = 2, kLdsVectorRegs = 3 };
struct Variant {
    int R, U, W;
    int form;
};
// Matrix cores (mma_stream) and matrix cores fed through LDS (mma_lds): {row
// tiles of 16 per wave, windows in flight, waves per workgroup}.  VALU row
// tiles (vec_tile): {rows per tile, vectors per pass, waves per workgroup}.
constexpr Variant kVariants[] = {
    {1, 2, 4, kMatrixCores}, {1, 2, 8, kMatrixCores}, {2, 2, 4, kMatrixCores},
    {2, 1, 8, kMatrixCores}, {1, 3, 4, kMatrixCores}, {2, 2, 8, kMatrixCores},
    {4, 2, 4, kValuTiles},   {8, 2, 4, kValuTiles},   {4, 4, 4, kValuTiles},
    {8, 4, 4, kValuTiles},   {2, 2, 4, kLdsStaged},   {2, 4, 4, kLdsStaged},
    {1, 2, 4, kLdsStaged},   {2, 2, 6, kLdsStaged},   {2, 2, 8, kLdsStaged},
    {2, 2, 2, kLdsStaged},   {2, 4, 2, kLdsStaged},   {2, 2, 4, kLdsVectorRegs},
    {2, 2, 2, kLdsVectorRegs}, {4, 1, 4, kValuTiles},
};
constexpr int kNumVariants = static_cast<int>(sizeof(kVariants) / sizeof(kVariants[0]));
// Defaults from MI355X sweeps of every variant (graph replays, rotated
// operands).  Row-major weights, one 7168 x 16384 weight against n vectors:
// the VALU tiles {4, 1, 4} for n = 1 and {4, 2, 4} for n = 2 (11.8 and 14.0
// us; 12.7 for {4, 2, 4} with one vector, 17.8 and 18.0 on the matrix cores,
// which pad the vectors to 16); the LDS-staged {2, 2, 4}
// with the vectors in registers for 3 <= n <= 13 (14.6 / 14.7 / 15.2 / 15.4
// us at n = 4 / 8 / 12 / 13 against 15.3 / 15.3 / 15.4 / 15.4 for the all-LDS
// {2, 2, 4} and 15.3 / 15.4 / 15.6 / 15.6 for the all-LDS {2, 4, 4}); the
// all-LDS {2, 2, 4} above 13 (15.4 / 15.5 us at 14 / 16 against 15.6 / 16.1
// with the vectors in registers, whose 16 rows then cost more as register
// loads than as whole-line copies, and 15.7 / 15.8 for {2, 4, 4}).  Both
// {2, 2, 4} forms refill a window's slot before its decode and products.
// The grouped GEMV (64 experts of 2048 x 7168, 128 tokens): the LDS-staged {2, 2,
// 2} with the vectors in registers while the experts average at most 4
// tokens (78.1 us against 80.1 for the all-LDS {2, 2, 2}, 83-92 for {2, 2, 4}
// and 109 for the register-fed {2, 1, 8}); its 26 KiB of LDS let six
// workgroups share a compute unit.  Packed weights already load 1 KiB per
// instruction: {2, 2, 4} and {2, 1, 8} on the matrix cores.  The VALU tiles
// never split K, so they are the default only while their tiles fill the GPU.
constexpr int kDefaultSmallN = 10;
constexpr int kDefaultSmallNMid = 17;
constexpr int kDefaultSmallNPacked = 2;
constexpr int kDefaultSmallNFew = 6;
constexpr int kDefaultSmallNOne = 19;
constexpr int64_t kFewVectors = 2;
constexpr int64_t kMidVectors = 13;
constexpr int kDefaultGrouped = 15;
constexpr int kDefaultGroupedFew = 18;
constexpr int64_t kFewTokensPerExpert = 4;
constexpr int kDefaultGroupedPacked = 3;
static_assert(kVariants[kDefaultSmallN].form == kLdsStaged && kVariants[kDefaultSmallN].U == 2 &&
                  kVariants[kDefaultSmallN].W == 4 &&
                  kVariants[kDefaultSmallNMid].form == kLdsVectorRegs &&
                  kVariants[kDefaultSmallNMid].W == 4 &&
                  kVariants[kDefaultGrouped].form == kLdsStaged && kVariants[kDefaultGrouped].W == 2 &&
                  kVariants[kDefaultGroupedFew].form == kLdsVectorRegs &&
                  kVariants[kDefaultGroupedFew].W == 2 &&
                  kVariants[kDefaultSmallNPacked].form == kMatrixCores &&
                  kVariants[kDefaultGroupedPacked].form == kMatrixCores &&
                  kVariants[kDefaultSmallNFew].form == kValuTiles &&
                  kVariants[kDefaultSmallNOne].form == kValuTiles && kVariants[kDefaultSmallNOne].U == 1,
              "the defaults name the variants measured above");

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Plan {
    int path;
    int variant;
    int64_t ksplit, kchunk, row_blocks, rows_per_block, groups;
    int threads;
    size_t ws_bytes;
};

inline bool fits_int64_product(int64_t a, int64_t b) { return a == 0 || b <= INT64_MAX / a; }

// groups x rows x (k/2) and the other byte counts within int64, outputs < 2^31.
inline int check_dims(int64_t groups, int64_t rows, int64_t nvec, int64_t k, bool allow_zero_vec) {
    if (groups < 1 || rows < 1 || nvec < (allow_zero_vec ? 0 : 1) || k < 16 || k % 16 != 0)
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (k >= (int64_t(1) << 31)) return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (!fits_int64_product(groups, rows) || !fits_int64_product(groups * rows, k / 2))
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (!fits_int64_product(nvec, k / 2)) return NVFP4_GEMV_ERR_BAD_SHAPE;
    return NVFP4_GEMV_OK;
}

// Shape rules of a small-N call (l weight matrices of m x k against n vectors
// each) and of a grouped call (experts of n x k, tokens routed tokens), the
// same for the plan queries and the launches: every byte count within int64,
// outputs fewer than 2^31.
inline int check_smalln_shape(int64_t l, int64_t m, int64_t n, int64_t k) {
    int s = check_dims(l, m, n, k, false);
    if (s != NVFP4_GEMV_OK) return s;
    if (!fits_int64_product(l, n) || !fits_int64_product(l * n, k / 2) ||
        !fits_int64_product(l * m, n) || l * m * n >= (int64_t(1) << 31))
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    return NVFP4_GEMV_OK;
}

inline int check_grouped_shape(int64_t tokens, int64_t experts, int64_t n, int64_t k) {
    int s = check_dims(experts, n, tokens, k, true);
    if (s != NVFP4_GEMV_OK) return s;
    if (!fits_int64_product(tokens, n) || tokens * n >= (int64_t(1) << 31))
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    return NVFP4_GEMV_OK;
}

// Workgroups of the fast kernel: (split, group, row block).  Defaults:
//  * the small-N GEMM splits K (powers of two, at least one window per wave
//    and split) while there are fewer 16-row tiles than compute units;
//  * while the workgroups are few (under 8 per compute unit), the rows per
//    workgroup shrink so that the count becomes a multiple of the 256 compute
//    units of an MI355X: a workgroup's time is set by its rows, so equal rows
//    on every unit beat full tiles on some and idle units elsewhere.
inline int make_plan(int64_t groups, int64_t rows, int64_t nvec_per_group, int64_t k, bool aligned,
              bool grouped, const nvfp4_mma_tuning_t *t, Plan *p, bool packed = false) {
    nvfp4_mma_tuning_t tun = {NVFP4_GEMV_PATH_AUTO, 0, 0, 0};
    if (t) tun = *t;
    if (tun.path < NVFP4_GEMV_PATH_AUTO || tun.path > NVFP4_GEMV_PATH_GENERIC || tun.variant < 0 ||
        tun.variant > kNumVariants || tun.ksplit < 0 || tun.rows_per_block < 0)
        return NVFP4_GEMV_ERR_BAD_TUNING;
    const bool fast_ok = aligned && k % 64 == 0 && k <= kMaxFastK;
    if (tun.path == NVFP4_GEMV_PATH_FAST && !fast_ok) return NVFP4_GEMV_ERR_BAD_TUNING;
    if (tun.path == NVFP4_GEMV_PATH_GENERIC &&
        (tun.variant != 0 || tun.ksplit > 1 || tun.rows_per_block != 0))
        return NVFP4_GEMV_ERR_BAD_TUNING;
    if (grouped && tun.ksplit > 1) return NVFP4_GEMV_ERR_BAD_TUNING;
    // Packed weights: matrix-core variants only, whole tiles per workgroup,
    // K splits on window boundaries.
    if (packed && (!fast_ok || tun.path == NVFP4_GEMV_PATH_GENERIC ||
                   (tun.variant > 0 && kVariants[tun.variant - 1].form != kMatrixCores) ||
                   tun.rows_per_block % kTile != 0))
        return NVFP4_GEMV_ERR_BAD_TUNING;
    const bool fast = tun.path != NVFP4_GEMV_PATH_GENERIC && fast_ok;
    p->path = fast ? NVFP4_GEMV_PATH_FAST : NVFP4_GEMV_PATH_GENERIC;
    if (!fast) {
        // (with NVFP4_GEMV_PATH_AUTO, fast-kernel settings are ignored where the
        // shape or alignment rules the fast kernel out; an explicit K split is not)
        if (tun.ksplit > 1) return NVFP4_GEMV_ERR_BAD_TUNING;
        p->variant = 0;
        p->ksplit = 1;
        p->kchunk = k;
        p->rows_per_block = kGenericWaves;
        p->threads = kGenericWaves * kPlanWave;
    } else {
        if (tun.variant > 0) {
            p->variant = tun.variant - 1;
        } else if (grouped) {
            // nvec_per_group: the tokens per expert on average, rounded up
            p->variant = packed ? kDefaultGroupedPacked
                                : nvec_per_group <= kFewTokensPerExpert ? kDefaultGroupedFew
                                                                        : kDefaultGrouped;
        } else if (packed) {
            p->variant = kDefaultSmallNPacked;
        } else {
            const int64_t tiles = groups * ceil_div(rows, int64_t(kVariants[kDefaultSmallNFew].R));
            p->variant = (nvec_per_group <= kFewVectors && tiles >= 4 * kComputeUnits)
                             ? (nvec_per_group == 1 ? kDefaultSmallNOne : kDefaultSmallNFew)
                         : nvec_per_group <= kMidVectors ? kDefaultSmallNMid
                                                         : kDefaultSmallN;
        }
        const Variant &v = kVariants[p->variant];
        if (v.form == kValuTiles) {
            // a workgroup per tile of v.R rows (or fewer on request), no K split
            if (tun.rows_per_block > v.R || tun.ksplit > 1) return NVFP4_GEMV_ERR_BAD_TUNING;
            p->ksplit = 1;
            p->kchunk = k;
            p->rows_per_block = tun.rows_per_block > 0 ? tun.rows_per_block : v.R;
            p->threads = v.W * kPlanWave;
            p->row_blocks = ceil_div(rows, p->rows_per_block);
            p->groups = groups * p->row_blocks;
            if (p->groups >= (int64_t(1) << 31)) return NVFP4_GEMV_ERR_BAD_SHAPE;
            p->ws_bytes = 0;
            return NVFP4_GEMV_OK;
        }
        const int64_t tile_rows = int64_t(v.R) * kTile;
        if (tun.rows_per_block > tile_rows) return NVFP4_GEMV_ERR_BAD_TUNING;
        int64_t ks = 1;
        if (tun.ksplit > 0) {
            ks = tun.ksplit;
        } else if (!grouped) {
            const int64_t wg1 = groups * ceil_div(rows, int64_t(kTile));
            const int64_t most = k / (int64_t(v.W) * kWinElems);
            while (wg1 * ks < kComputeUnits && ks * 2 <= most) ks *= 2;
        }
        const int64_t granule = packed ? kWinElems : kLaneElems;
        if (ks > ceil_div(k, granule)) return NVFP4_GEMV_ERR_BAD_TUNING;
        const int64_t kchunk = ceil_div(ceil_div(k, ks), granule) * granule;
        p->ksplit = ceil_div(k, kchunk);
        p->kchunk = kchunk;
        int64_t rpb = tile_rows;
        if (tun.rows_per_block > 0) {
            rpb = tun.rows_per_block;
        } else if (!packed) {
            const int64_t wg = groups * ceil_div(rows, tile_rows) * p->ksplit;
            if (wg < 8 * kComputeUnits) {
                const int64_t target = ceil_div(wg, kComputeUnits) * kComputeUnits;
                const int64_t blocks = ceil_div(target, groups * p->ksplit);   // per group
                rpb = ceil_div(rows, blocks);
                if (rpb > tile_rows) rpb = tile_rows;
            }
        }
        p->rows_per_block = rpb;
        p->threads = v.W * kPlanWave;
    }
    p->row_blocks = ceil_div(rows, p->rows_per_block);
    p->groups = groups * p->row_blocks * p->ksplit;
    if (p->groups >= (int64_t(1) << 31)) return NVFP4_GEMV_ERR_BAD_SHAPE;
    p->ws_bytes = p->ksplit > 1
                      ? static_cast<size_t>(p->ksplit) * groups * rows * nvec_per_group * sizeof(float)
                      : 0;
    return NVFP4_GEMV_OK;
}

}  // namespace nvfp4mmaplan

#endif  // NVFP4_MMA_PLAN_H
