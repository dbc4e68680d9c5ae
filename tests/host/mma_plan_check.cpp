// Host-only checks of the small-N GEMM and grouped GEMV launch plan
// (precision_decode_amd/csrc/mma_plan.h), built with g++ and the address and
// undefined-behaviour sanitizers by tests/test_host_sanitized.py.  No GPU and
// no HIP.  Random shapes and tunings, from tiny to the edges of the shape
// rules, check that every accepted plan describes a launch the kernels can
// run (rows per workgroup within the variant's tile, whole K covered by the
// splits, workgroup count below 2^31, the workspace the splits need) and that
// the default variant follows the documented rules.
//
// Prints "mma_plan_check ok" and exits 0 when every check holds; otherwise
// prints the failed check and exits 1.
#include <cstdint>
#include <cstdio>

#include "mma_plan.h"

using namespace nvfp4mmaplan;

namespace {

int g_failures = 0;

#define CHECK(cond)                                                                   \
    do {                                                                              \
        if (!(cond)) {                                                                \
            std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);             \
            ++g_failures;                                                             \
        }                                                                             \
    } while (0)

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {   // splitmix64
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
int64_t pick(int64_t lo, int64_t hi) { return lo + static_cast<int64_t>(next() % uint64_t(hi - lo + 1)); }

// A dimension: mostly small and ragged, sometimes large, sometimes at a power of two.
int64_t dim(int64_t hi) {
    switch (next() % 4) {
    case 0: return pick(1, 40);
    case 1: return pick(1, hi);
    case 2: return int64_t(1) << pick(0, 63 - __builtin_clzll(uint64_t(hi)));   // powers of two up to hi
    default: return pick(1, 8192);
    }
}

// Every accepted plan, against what the kernels assume.
void check_plan(const Plan &p, int64_t groups, int64_t rows, int64_t nvec, int64_t k, bool grouped,
                bool packed) {
    CHECK(p.path == NVFP4_GEMV_PATH_FAST || p.path == NVFP4_GEMV_PATH_GENERIC);
    CHECK(p.ksplit >= 1 && p.kchunk >= 1);
    CHECK(p.rows_per_block >= 1);
    CHECK(p.row_blocks == ceil_div(rows, p.rows_per_block));
    CHECK(p.groups == groups * p.row_blocks * p.ksplit);
    CHECK(p.groups < (int64_t(1) << 31));
    // the splits cover K exactly once
    CHECK((p.ksplit - 1) * p.kchunk < k && p.ksplit * p.kchunk >= k);
    const unsigned __int128 need =
        p.ksplit > 1 ? static_cast<unsigned __int128>(p.ksplit) * uint64_t(groups) * uint64_t(rows) *
                           uint64_t(nvec) * sizeof(float)
                     : 0;
    CHECK(need == static_cast<unsigned __int128>(p.ws_bytes));
    if (grouped) CHECK(p.ksplit == 1);
    if (p.path == NVFP4_GEMV_PATH_GENERIC) {
        CHECK(!packed);
        CHECK(p.variant == 0 && p.ksplit == 1 && p.kchunk == k);
        CHECK(p.rows_per_block == kGenericWaves && p.threads == kGenericWaves * kPlanWave);
        return;
    }
    CHECK(p.variant >= 0 && p.variant < kNumVariants);
    if (p.variant < 0 || p.variant >= kNumVariants) return;
    const Variant &v = kVariants[p.variant];
    CHECK(p.threads == v.W * kPlanWave);
    CHECK(k % 64 == 0 && k <= kMaxFastK);
    if (v.form == kValuTiles) {
        CHECK(!packed);
        CHECK(p.ksplit == 1 && p.kchunk == k && p.rows_per_block <= v.R);
        return;
    }
    CHECK(p.rows_per_block <= int64_t(v.R) * kTile);
    CHECK(p.kchunk % (packed ? kWinElems : kLaneElems) == 0);
    if (packed) {
        CHECK(v.form == kMatrixCores);
        CHECK(p.rows_per_block % kTile == 0);
    }
}

// The default variant rules.
void check_default(const Plan &p, int64_t groups, int64_t rows, int64_t nvec, bool grouped, bool packed) {
    if (p.path != NVFP4_GEMV_PATH_FAST) return;
    const Variant &v = kVariants[p.variant];
    if (packed) {
        CHECK(v.form == kMatrixCores);
    } else if (grouped) {
        CHECK(v.form == (nvec <= kFewTokensPerExpert ? kLdsVectorRegs : kLdsStaged));
    } else if (nvec <= kFewVectors && groups * ceil_div(rows, 4) >= 4 * kComputeUnits) {
        CHECK(v.form == kValuTiles);
    } else {
        CHECK(v.form == (nvec <= kMidVectors ? kLdsVectorRegs : kLdsStaged));
    }
}

void random_plans(int iters) {
    int accepted = 0, fast = 0, split = 0, forms[4] = {0, 0, 0, 0};
    for (int i = 0; i < iters; ++i) {
        const bool grouped = next() % 3 == 0;
        const bool packed = next() % 4 == 0;
        const int64_t groups = dim(int64_t(1) << 20);
        const int64_t rows = dim(int64_t(1) << 24);
        const int64_t k = 16 * dim(int64_t(1) << 26);
        const int64_t nvec = grouped ? pick(0, 64) : dim(64);
        const int64_t tokens = grouped ? groups * nvec - pick(0, nvec > 0 ? nvec - 1 : 0) : 0;
        const int64_t per = grouped ? ceil_div(tokens, groups) : nvec;
        const int shape = grouped ? check_grouped_shape(tokens, groups, rows, k)
                                  : check_smalln_shape(groups, rows, nvec, k);
        if (shape != NVFP4_GEMV_OK) {
            CHECK(shape == NVFP4_GEMV_ERR_BAD_SHAPE);
            continue;
        }
        nvfp4_mma_tuning_t t = {NVFP4_GEMV_PATH_AUTO, 0, 0, 0};
        const int mode = static_cast<int>(next() % 3);
        if (mode >= 1) {
            t.variant = static_cast<int32_t>(next() % (kNumVariants + 1));
            if (next() % 2) t.ksplit = static_cast<int32_t>(next() % 9);
            if (next() % 2) t.rows_per_block = static_cast<int32_t>(next() % 40);
            if (mode == 2) t.path = static_cast<int32_t>(next() % 3);
        }
        Plan p{};
        const bool aligned = next() % 8 != 0;
        const int s = make_plan(groups, rows, per, k, aligned || packed, grouped, mode ? &t : nullptr,
                                &p, packed);
        CHECK(s == NVFP4_GEMV_OK || s == NVFP4_GEMV_ERR_BAD_TUNING || s == NVFP4_GEMV_ERR_BAD_SHAPE);
        if (s != NVFP4_GEMV_OK) continue;
        ++accepted;
        if (p.path == NVFP4_GEMV_PATH_FAST) {
            ++fast;
            ++forms[kVariants[p.variant].form];
        }
        if (p.ksplit > 1) ++split;
        check_plan(p, groups, rows, per, k, grouped, packed);
        if (mode == 0) check_default(p, groups, rows, per, grouped, packed);
        if (mode >= 1 && t.variant > 0 && p.path == NVFP4_GEMV_PATH_FAST) CHECK(p.variant == t.variant - 1);
        if (mode >= 1 && t.ksplit > 0 && p.path == NVFP4_GEMV_PATH_FAST) CHECK(p.ksplit <= t.ksplit);
    }
    // every kind of plan was reached
    CHECK(accepted > iters / 10 && fast > accepted / 4 && split > 100);
    for (int f = 0; f < 4; ++f) CHECK(forms[f] > 100);
    std::printf("%d plans accepted of %d: %d fast (forms %d %d %d %d), %d with a K split\n", accepted,
                iters, fast, forms[0], forms[1], forms[2], forms[3], split);
}

void fixed_cases() {
    Plan p{};
    // the decode weight against 1, 4, 16 vectors; moe_decode
    CHECK(make_plan(1, 7168, 1, 16384, true, false, nullptr, &p) == NVFP4_GEMV_OK);
    CHECK(kVariants[p.variant].form == kValuTiles);
    CHECK(make_plan(1, 7168, 4, 16384, true, false, nullptr, &p) == NVFP4_GEMV_OK);
    CHECK(kVariants[p.variant].form == kLdsVectorRegs && p.ksplit == 1);
    CHECK(p.groups % kComputeUnits == 0);
    CHECK(make_plan(1, 7168, 16, 16384, true, false, nullptr, &p) == NVFP4_GEMV_OK);
    CHECK(kVariants[p.variant].form == kLdsStaged && p.ws_bytes == 0);
    CHECK(make_plan(64, 2048, ceil_div(128, 64), 7168, true, true, nullptr, &p) == NVFP4_GEMV_OK);
    CHECK(kVariants[p.variant].form == kLdsVectorRegs && p.ksplit == 1);
    // few tiles: K split, workspace for every split
    CHECK(make_plan(1, 64, 3, 16384, true, false, nullptr, &p) == NVFP4_GEMV_OK);
    CHECK(p.ksplit > 1 && p.ws_bytes == size_t(p.ksplit) * 64 * 3 * 4);
    // shape edges
    CHECK(check_smalln_shape(1, 1, 1, 16) == NVFP4_GEMV_OK);
    CHECK(check_smalln_shape(1, 1, 1, 8) == NVFP4_GEMV_ERR_BAD_SHAPE);
    CHECK(check_smalln_shape(1, int64_t(1) << 16, int64_t(1) << 15, 64) == NVFP4_GEMV_ERR_BAD_SHAPE);
    CHECK(check_smalln_shape(int64_t(1) << 40, int64_t(1) << 40, 1, 64) == NVFP4_GEMV_ERR_BAD_SHAPE);
    CHECK(check_grouped_shape(-1, 4, 96, 128) == NVFP4_GEMV_ERR_BAD_SHAPE);
    CHECK(check_grouped_shape(0, 4, 96, 128) == NVFP4_GEMV_OK);
    CHECK(check_grouped_shape(int64_t(1) << 20, 4, int64_t(1) << 11, 128) == NVFP4_GEMV_ERR_BAD_SHAPE);
    // tunings outside the rules
    nvfp4_mma_tuning_t t = {NVFP4_GEMV_PATH_AUTO, kNumVariants + 1, 0, 0};
    CHECK(make_plan(1, 64, 4, 4096, true, false, &t, &p) == NVFP4_GEMV_ERR_BAD_TUNING);
    t = {NVFP4_GEMV_PATH_AUTO, 0, 2, 0};
    CHECK(make_plan(4, 64, 4, 4096, true, true, &t, &p) == NVFP4_GEMV_ERR_BAD_TUNING);   // grouped: no split
    for (int v = 0; v < kNumVariants; ++v) {
        t = {NVFP4_GEMV_PATH_AUTO, v + 1, 0, 0};
        const int s = make_plan(1, 64, 4, 4096, true, false, &t, &p, true);
        CHECK((s == NVFP4_GEMV_OK) == (kVariants[v].form == kMatrixCores));
    }
}

}  // namespace

int main() {
    fixed_cases();
    random_plans(200000);
    if (g_failures) {
        std::printf("%d checks failed\n", g_failures);
        return 1;
    }
    std::printf("mma_plan_check ok\n");
    return 0;
}
