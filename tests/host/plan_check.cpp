// Host-only checks of the GEMV library's validation, launch plan and launch
// orchestration (precision_decode_amd/csrc/gemv_plan.h), built with g++ and
// the address and undefined-behaviour sanitizers by tests/test_host_sanitized.py.
// No GPU and no HIP: a mock backend stands in for the device, the workspace
// allocator and the kernel launch, and can fail each of them on purpose.
//
// Prints "plan_check ok" and exits 0 when every check holds; otherwise prints
// the failed check and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "gemv_plan.h"

using namespace nvfp4plan;

namespace {

int g_failures = 0;

#define CHECK(cond)                                                                   \
    do {                                                                              \
        if (!(cond)) {                                                                \
            std::printf("FAILED %s:%d: %s\n", __FILE__, __LINE__, #cond);             \
            ++g_failures;                                                             \
        }                                                                             \
    } while (0)

// A backend whose every call can be made to fail; it counts what was called.
struct MockBackend {
    bool has_device = true;
    bool workspace_ok = true;
    bool scratch_ok = true;
    bool launch_ok = true;
    int device_calls = 0, workspace_calls = 0, scratch_calls = 0, run_calls = 0;
    size_t last_need = 0;
    void *last_ws = nullptr;
    Plan last_plan{};
    std::vector<unsigned char> ws_memory = std::vector<unsigned char>(1 << 20);

    bool device(int *dev) {
        ++device_calls;
        *dev = 0;
        return has_device;
    }
    void *workspace(int, void *, size_t need) {
        ++workspace_calls;
        last_need = need;
        if (!workspace_ok || need > ws_memory.size()) return nullptr;
        return ws_memory.data();
    }
    void *scratch(int) {
        ++scratch_calls;
        return scratch_ok ? ws_memory.data() : nullptr;
    }
    int run(const Plan &p, const GemvArgs &, void *ws, void *) {
        ++run_calls;
        last_plan = p;
        last_ws = ws;
        return launch_ok ? NVFP4_GEMV_OK : NVFP4_GEMV_ERR_LAUNCH;
    }
};

// Fake device addresses: never dereferenced, far apart, 256-byte aligned.
GemvArgs args(int64_t l, int64_t m, int64_t k) {
    GemvArgs a;
    a.A = reinterpret_cast<const uint8_t *>(uintptr_t(1) << 40);
    a.sfA = reinterpret_cast<const uint8_t *>(uintptr_t(2) << 40);
    a.x = reinterpret_cast<const uint8_t *>(uintptr_t(3) << 40);
    a.sfx = reinterpret_cast<const uint8_t *>(uintptr_t(4) << 40);
    a.alpha = reinterpret_cast<const float *>(uintptr_t(5) << 40);
    a.c = reinterpret_cast<uint16_t *>(uintptr_t(6) << 40);
    a.l = l;
    a.m = m;
    a.k = k;
    return a;
}

// The invariants every plan the library can make must satisfy.
void check_plan(int64_t l, int64_t m, int64_t k, bool aligned, const Plan &p) {
    CHECK(p.path == NVFP4_GEMV_PATH_FAST || p.path == NVFP4_GEMV_PATH_GENERIC);
    CHECK(p.variant >= 0 && p.variant < kNumVariants);
    CHECK(p.ksplit >= 1 && p.kchunk >= 16 && p.kchunk % 16 == 0);
    CHECK(p.ksplit * p.kchunk >= k);            // the splits cover K ...
    CHECK((p.ksplit - 1) * p.kchunk < k);       // ... and none is empty
    CHECK(p.groups >= 1 && p.groups < (int64_t(1) << 31));
    CHECK(p.groups == l * p.row_blocks * p.ksplit);
    CHECK(p.threads >= kLanes && p.threads <= 1024 && p.threads % kLanes == 0);
    CHECK(p.lds_bytes <= 160 * 1024);
    CHECK(p.ws_bytes == (p.ksplit > 1 ? size_t(p.ksplit) * size_t(l * m) * 4 : 0));
    if (p.path == NVFP4_GEMV_PATH_FAST) {
        CHECK(aligned && k % 32 == 0);
        CHECK(p.kchunk % 32 == 0);
        const Variant &v = kVariants[p.variant];
        const int64_t rows = v.xform == kXTile ? v.R : int64_t(v.R) * v.W;
        CHECK(p.row_blocks * rows >= m && (p.row_blocks - 1) * rows < m);
        if (v.xform == kXHalf || v.xform == kXPacked) CHECK(p.kchunk <= kMaxChunk);
        if (v.xform == kXTile) CHECK(k <= kTileMaxK);
        CHECK(p.threads == v.W * kLanes);
    } else {
        CHECK(p.row_blocks * kGenericWaves >= m);
    }
}

uint64_t g_rng = 0x9E3779B97F4A7C15ull;
uint64_t next() {   // xorshift64*
    g_rng ^= g_rng >> 12;
    g_rng ^= g_rng << 25;
    g_rng ^= g_rng >> 27;
    return g_rng * 0x2545F4914F6CDD1Dull;
}
int64_t pick(const std::vector<int64_t> &v) { return v[next() % v.size()]; }

void plans_over_many_shapes() {
    const std::vector<int64_t> ls = {1, 2, 3, 4, 8, 16, 64, 1000, 1 << 20};
    const std::vector<int64_t> ms = {1, 3, 4, 7, 14, 16, 100, 128, 896, 2048, 4096, 7168, 100000};
    const std::vector<int64_t> ks = {16,   32,    48,    64,    256,   2032,  2048,  2064,  4096,
                                     7168, 16384, 16400, 32768, 65536, 1 << 20, (1 << 26) + 32,
                                     (int64_t(1) << 31) - 16};
    int planned = 0;
    for (int it = 0; it < 20000; ++it) {
        const int64_t l = pick(ls), m = pick(ms), k = pick(ks);
        const bool aligned = next() & 1;
        nvfp4_gemv_tuning_t t = {0, 0, 0, 0};
        const int mode = static_cast<int>(next() % 4);
        if (mode >= 1) t.variant = static_cast<int32_t>(next() % (kNumVariants + 1));
        if (mode >= 2) t.ksplit = static_cast<int32_t>(next() % 9);
        if (mode == 3) t.path = static_cast<int32_t>(next() % 3);
        if (check_shape(l, m, k) != NVFP4_GEMV_OK) continue;
        Plan p;
        const int s = make_plan(l, m, k, aligned, mode ? &t : nullptr, &p);
        if (mode == 0) CHECK(s == NVFP4_GEMV_OK || s == NVFP4_GEMV_ERR_BAD_SHAPE);
        if (s == NVFP4_GEMV_OK) {
            check_plan(l, m, k, aligned, p);
            ++planned;
        } else {
            CHECK(s == NVFP4_GEMV_ERR_BAD_TUNING || s == NVFP4_GEMV_ERR_BAD_SHAPE);
        }
    }
    CHECK(planned > 5000);
}

void the_headline_workloads_plan_as_measured() {
    struct W { int64_t l, m, k; int variant; int64_t ksplit; };
    // decode, batched, short K, Gaussian: one kernel, no K split
    const W w[] = {{1, 7168, 16384, 30, 1}, {8, 4096, 7168, 19, 1}, {4, 7168, 2048, 28, 1},
                   {16, 2048, 4096, 24, 1}};
    for (const W &x : w) {
        Plan p;
        CHECK(make_plan(x.l, x.m, x.k, true, nullptr, &p) == NVFP4_GEMV_OK);
        CHECK(p.path == NVFP4_GEMV_PATH_FAST && p.variant == x.variant && p.ksplit == x.ksplit);
        CHECK(p.ws_bytes == 0);
    }
    // one GPU's eighth of the decode weight: too few 4-row tiles to fill the
    // GPU, so the staged kernel with K split across workgroups
    Plan p;
    CHECK(make_plan(1, 896, 16384, true, nullptr, &p) == NVFP4_GEMV_OK);
    CHECK(p.variant == 0 && p.ksplit > 1 && p.ws_bytes == size_t(p.ksplit) * 896 * 4);
}

void validation_comes_before_any_backend_call() {
    MockBackend be;
    GemvArgs a = args(1, 8, 64);
    a.A = nullptr;
    CHECK(launch_owned_workspace(be, a, nullptr) == NVFP4_GEMV_ERR_NULL_POINTER);
    a = args(1, 8, 40);   // k % 16 != 0
    CHECK(launch_owned_workspace(be, a, nullptr) == NVFP4_GEMV_ERR_BAD_SHAPE);
    a = args(0, 8, 64);
    CHECK(launch_owned_workspace(be, a, nullptr) == NVFP4_GEMV_ERR_BAD_SHAPE);
    a = args(int64_t(1) << 40, int64_t(1) << 40, 64);   // l * m overflows
    CHECK(launch_owned_workspace(be, a, nullptr) == NVFP4_GEMV_ERR_BAD_SHAPE);
    a = args(1, 8, 64);
    a.c = reinterpret_cast<uint16_t *>(reinterpret_cast<uintptr_t>(a.c) + 1);
    CHECK(launch_owned_workspace(be, a, nullptr) == NVFP4_GEMV_ERR_ALIGNMENT);
    a = args(1, 8, 64);
    a.alpha = reinterpret_cast<const float *>(reinterpret_cast<uintptr_t>(a.alpha) + 2);
    CHECK(launch_owned_workspace(be, a, nullptr) == NVFP4_GEMV_ERR_ALIGNMENT);
    a = args(1, 8, 64);
    a.c = reinterpret_cast<uint16_t *>(const_cast<uint8_t *>(a.A) + 100);   // inside A
    CHECK(launch_owned_workspace(be, a, nullptr) == NVFP4_GEMV_ERR_ALIAS);
    a = args(1, 8, 64);
    a.c = reinterpret_cast<uint16_t *>(const_cast<float *>(a.alpha)) - 1;   // reaches alpha
    CHECK(launch_owned_workspace(be, a, nullptr) == NVFP4_GEMV_ERR_ALIAS);
    nvfp4_gemv_tuning_t bad = {0, 0, 0, 1};   // reserved field set
    CHECK(launch_caller_workspace(be, args(1, 8, 64), &bad, nullptr, 0, nullptr) ==
          NVFP4_GEMV_ERR_BAD_TUNING);
    CHECK(be.device_calls == 0 && be.workspace_calls == 0 && be.run_calls == 0);
}

void workspace_and_launch_failures() {
    // a split-K shape: one GPU's eighth of the decode weight
    const GemvArgs split = args(1, 896, 16384);
    {
        MockBackend be;
        be.workspace_ok = false;
        CHECK(launch_owned_workspace(be, split, nullptr) == NVFP4_GEMV_ERR_WORKSPACE);
        CHECK(be.workspace_calls == 1 && be.run_calls == 0);
    }
    {
        MockBackend be;
        be.has_device = false;
        CHECK(launch_owned_workspace(be, split, nullptr) == NVFP4_GEMV_ERR_DEVICE);
        CHECK(be.workspace_calls == 0 && be.run_calls == 0);
    }
    {
        MockBackend be;
        be.launch_ok = false;
        CHECK(launch_owned_workspace(be, split, nullptr) == NVFP4_GEMV_ERR_LAUNCH);
        CHECK(be.run_calls == 1);
    }
    {
        MockBackend be;
        CHECK(launch_owned_workspace(be, split, nullptr) == NVFP4_GEMV_OK);
        CHECK(be.run_calls == 1 && be.last_ws == be.ws_memory.data());
        CHECK(be.last_need == be.last_plan.ws_bytes && be.last_plan.ksplit > 1);
    }
    {
        // no split: the workspace is never asked for, and no device either
        MockBackend be;
        be.workspace_ok = false;
        be.has_device = false;
        CHECK(launch_owned_workspace(be, args(1, 7168, 16384), nullptr) == NVFP4_GEMV_OK);
        CHECK(be.workspace_calls == 0 && be.device_calls == 0 && be.last_ws == nullptr);
        be.launch_ok = false;
        CHECK(launch_owned_workspace(be, args(1, 7168, 16384), nullptr) == NVFP4_GEMV_ERR_LAUNCH);
    }
    // caller-owned workspace
    Plan p;
    CHECK(make_plan(1, 896, 16384, true, nullptr, &p) == NVFP4_GEMV_OK);
    {
        MockBackend be;
        std::vector<float> ws(p.ws_bytes / 4 + 1);
        CHECK(launch_caller_workspace(be, split, nullptr, nullptr, p.ws_bytes, nullptr) ==
              NVFP4_GEMV_ERR_WORKSPACE);
        CHECK(launch_caller_workspace(be, split, nullptr, ws.data(), p.ws_bytes - 4, nullptr) ==
              NVFP4_GEMV_ERR_WORKSPACE);
        CHECK(launch_caller_workspace(be, split, nullptr,
                                      reinterpret_cast<char *>(ws.data()) + 2, p.ws_bytes,
                                      nullptr) == NVFP4_GEMV_ERR_ALIGNMENT);
        GemvArgs alias = split;
        alias.c = reinterpret_cast<uint16_t *>(ws.data());
        CHECK(launch_caller_workspace(be, alias, nullptr, ws.data(), p.ws_bytes, nullptr) ==
              NVFP4_GEMV_ERR_ALIAS);
        CHECK(be.run_calls == 0);
        CHECK(launch_caller_workspace(be, split, nullptr, ws.data(), p.ws_bytes, nullptr) ==
              NVFP4_GEMV_OK);
        CHECK(be.run_calls == 1 && be.last_ws == ws.data());
        be.launch_ok = false;
        CHECK(launch_caller_workspace(be, split, nullptr, ws.data(), p.ws_bytes, nullptr) ==
              NVFP4_GEMV_ERR_LAUNCH);
        CHECK(be.device_calls == 0 && be.workspace_calls == 0);
    }
}

void fixed_scratch_entry() {
    const GemvArgs split = args(1, 896, 16384);
    {
        MockBackend be;   // fits: the scratch array is used, nothing else
        CHECK(launch_fixed_scratch(be, split, nullptr) == NVFP4_GEMV_OK);
        CHECK(be.scratch_calls == 1 && be.workspace_calls == 0 && be.run_calls == 1);
        CHECK(be.last_ws == be.ws_memory.data() && be.last_plan.ksplit > 1);
    }
    {
        MockBackend be;   // no split: no scratch, no device query
        CHECK(launch_fixed_scratch(be, args(1, 7168, 16384), nullptr) == NVFP4_GEMV_OK);
        CHECK(be.scratch_calls == 0 && be.device_calls == 0 && be.last_ws == nullptr);
    }
    {
        // partial sums larger than the array: refused before the backend is asked
        MockBackend be;
        const GemvArgs big = args(1, 524352, 32768);
        Plan p;
        CHECK(make_plan(1, 524352, 32768, true, nullptr, &p) == NVFP4_GEMV_OK);
        CHECK(p.ws_bytes > kNoAllocScratchBytes);
        CHECK(launch_fixed_scratch(be, big, nullptr) == NVFP4_GEMV_ERR_WORKSPACE);
        CHECK(be.device_calls == 0 && be.scratch_calls == 0 && be.run_calls == 0);
        // the largest such shape that fits is accepted
        const GemvArgs fits = args(1, 524288, 32768);
        CHECK(make_plan(1, 524288, 32768, true, nullptr, &p) == NVFP4_GEMV_OK);
        CHECK(p.ws_bytes == kNoAllocScratchBytes);
        CHECK(launch_fixed_scratch(be, fits, nullptr) == NVFP4_GEMV_OK);
    }
    {
        MockBackend be;
        be.scratch_ok = false;
        CHECK(launch_fixed_scratch(be, split, nullptr) == NVFP4_GEMV_ERR_WORKSPACE);
        be.scratch_ok = true;
        be.has_device = false;
        CHECK(launch_fixed_scratch(be, split, nullptr) == NVFP4_GEMV_ERR_DEVICE);
        be.has_device = true;
        be.launch_ok = false;
        CHECK(launch_fixed_scratch(be, split, nullptr) == NVFP4_GEMV_ERR_LAUNCH);
        CHECK(be.workspace_calls == 0);
    }
    {
        MockBackend be;
        GemvArgs a = split;
        a.sfx = nullptr;
        CHECK(launch_fixed_scratch(be, a, nullptr) == NVFP4_GEMV_ERR_NULL_POINTER);
        CHECK(be.device_calls == 0 && be.scratch_calls == 0 && be.run_calls == 0);
    }
}

void overlap_near_the_top_of_the_address_space() {
    const void *top = reinterpret_cast<const void *>(UINTPTR_MAX - 15);
    const void *below = reinterpret_cast<const void *>(UINTPTR_MAX - 31);
    CHECK(!overlaps(top, 16, below, 16));
    CHECK(overlaps(top, 16, below, 17));
    CHECK(overlaps(below, 32, top, 1));
    CHECK(!overlaps(nullptr, 16, top, 16));
    CHECK(!overlaps(top, 0, top, 16));
}

}  // namespace

int main() {
    plans_over_many_shapes();
    the_headline_workloads_plan_as_measured();
    validation_comes_before_any_backend_call();
    workspace_and_launch_failures();
    fixed_scratch_entry();
    overlap_near_the_top_of_the_address_space();
    if (g_failures) {
        std::printf("plan_check: %d failed checks\n", g_failures);
        return 1;
    }
    std::printf("plan_check ok\n");
    return 0;
}
