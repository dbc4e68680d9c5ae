// NVFP4 block-scaled batched GEMV for MI355X (gfx950, CDNA4): host side.
//
//   c[b,r] = f16( f32( alpha[b] * sum_kk e2m1(A[b,r,kk]) e4m3(sfA[b,r,kk/16])
//                                      * e2m1(x[b,kk])   e4m3(sfx[b,kk/16]) ) )
//
// (the NVFP4 batched GEMV of "nvFP4 Batch GEMV算子系列(下)", section "NVFP4
// Batched GEMV 概念阐述").  The kernels and their design are in
// gemv_kernels.h; the validation and launch plan, shared with the host-only
// checks, in gemv_plan.h.  This file maps plans to kernel launches, owns the
// per-stream split-K workspaces and the fixed scratch array, and defines the
// C entry points of include/nvfp4_gemv.h.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "device_common.h"
#include "gemv_kernels.h"
#include "gemv_plan.h"
#include "nvfp4_gemv.h"
#include "probe_kernels.h"

namespace {

using namespace nvfp4dev;
using namespace nvfp4plan;

// ---------------------------------------------------------------- host side
typedef void (*FastKernel)(const uint8_t *, const uint8_t *, const uint8_t *, const uint8_t *,
                           const float *, uint16_t *, float *, int64_t, int64_t, int64_t,
                           int64_t, int64_t);

FastKernel fast_kernel(int v) {
    switch (v) {
    case 0: return gemv_fast<2, 4, 7>;
    case 1: return gemv_fast<1, 8, 4>;
    case 2: return gemv_fast<2, 4, 4>;
    case 3: return gemv_fast<2, 2, 4>;
    case 4: return gemv_fast<4, 2, 4>;
    case 5: return gemv_fast<2, 4, 8>;
    case 6: return gemv_fast<1, 8, 8>;
    case 7: return gemv_fast<4, 1, 4>;
    case 8: return gemv_fast<2, 1, 8>;
    case 9: return gemv_fast<1, 4, 4>;
    case 10: return gemv_fastp<2, 2, 4>;
    case 11: return gemv_fastp<4, 1, 4>;
    case 12: return gemv_fastp<4, 2, 4>;
    case 13: return gemv_fastp<2, 4, 8>;
    case 14: return gemv_fastp<4, 2, 8>;
    case 15: return gemv_fastp<1, 4, 8>;
    case 16: return gemv_fastg<2, 4, 7>;
    case 17: return gemv_fastg<2, 2, 7>;
    case 18: return gemv_fastg<4, 2, 7>;
    case 19: return gemv_fastg<2, 4, 4>;
    case 20: return gemv_fastg<1, 8, 7>;
    case 21: return gemv_fastg<4, 1, 8>;
    case 22: return gemv_tile<8, 16>;
    case 23: return gemv_tile<4, 16>;
    case 24: return gemv_tile<2, 16>;
    case 25: return gemv_tile<1, 16>;
    case 26: return gemv_tile<1, 8>;
    case 27: return gemv_tile<2, 8>;
    case 28: return gemv_tile<1, 4>;
    case 29: return gemv_tile<2, 4>;
    case 30: return gemv_tile<8, 4>;
    case 31: return gemv_tile<4, 4>;
    case 32: return gemv_tile<4, 8>;
    default: return nullptr;
    }
}

static_assert(kNumVariants == 33, "fast_kernel() covers every entry of kVariants");

// Enqueues the plan's kernels: the GEMV (or its partial sums) and, with a K
// split, the second pass.
int run(const Plan &p, const GemvArgs &g, void *ws, hipStream_t stream) {
    const uint8_t *A = g.A, *sfA = g.sfA, *x = g.x, *sfx = g.sfx;
    const float *alpha = g.alpha;
    uint16_t *c = g.c;
    int64_t l = g.l, m = g.m, k = g.k;
    float *part = p.ksplit > 1 ? static_cast<float *>(ws) : nullptr;
    int64_t kchunk = p.kchunk, row_blocks = p.row_blocks;
    void *args[] = {&A, &sfA, &x, &sfx, &alpha, &c, &part, &l, &m, &k, &kchunk, &row_blocks};
    const void *fn;
    if (p.path == NVFP4_GEMV_PATH_FAST)
        fn = reinterpret_cast<const void *>(fast_kernel(p.variant));
    else
        fn = reinterpret_cast<const void *>(gemv_generic);
    hipError_t e = hipLaunchKernel(fn, dim3(static_cast<uint32_t>(p.groups)), dim3(p.threads),
                                   args, p.lds_bytes, stream);
    if (e != hipSuccess) return NVFP4_GEMV_ERR_LAUNCH;
    if (p.ksplit > 1) {
        const float *cpart = part;
        int64_t ks = p.ksplit;
        void *rargs[] = {&cpart, &alpha, &c, &l, &m, &ks};
        const int64_t n = l * m;
        e = hipLaunchKernel(reinterpret_cast<const void *>(gemv_splitk_reduce),
                            dim3(static_cast<uint32_t>(ceil_div(n, kReduceThreads))),
                            dim3(kReduceThreads), rargs, 0, stream);
        if (e != hipSuccess) return NVFP4_GEMV_ERR_LAUNCH;
    }
    return NVFP4_GEMV_OK;
}

// Library-owned split-K workspaces, one per (device, stream).  A slot only
// grows.  Growing allocates a new buffer and retires the old one without
// freeing it: kernels enqueued earlier on the stream may still read it, and
// freeing it safely would need a synchronisation.  Retired buffers are kept
// until the process ends; each growth at least doubles the slot, so they add
// at most the slot's final size.  No allocation is made while the stream is
// being captured into a graph (the call fails instead).
std::mutex g_ws_mutex;
std::map<std::pair<int, void *>, std::pair<void *, size_t>> g_ws;
std::vector<void *> g_ws_retired;

bool stream_capturing(void *stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;   // cannot tell: do not allocate
    }
    return cs != hipStreamCaptureStatusNone;
}

// Device addresses of the fixed scratch array, one per device, taken once
// with that device current (each GPU holds its own copy of the array).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

void *scratch_address(int dev);

// The library's backend for the launch orchestration of gemv_plan.h.
struct HipBackend {
    bool device(int *dev) {
        if (hipGetDevice(dev) == hipSuccess) return true;
        (void)hipGetLastError();
        return false;
    }
    void *workspace(int dev, void *stream, size_t need) {
        return nvfp4_stream_workspace(dev, stream, need);
    }
    void *scratch(int dev) { return scratch_address(dev); }
    int run(const Plan &p, const GemvArgs &g, void *ws, void *stream) {
        return ::run(p, g, ws, static_cast<hipStream_t>(stream));
    }
};

GemvArgs gemv_args(const uint8_t *A, const uint8_t *sfA, const uint8_t *x, const uint8_t *sfx,
                   const float *alpha, uint16_t *c, int64_t l, int64_t m, int64_t k) {
    GemvArgs g;
    g.A = A;
    g.sfA = sfA;
    g.x = x;
    g.sfx = sfx;
    g.alpha = alpha;
    g.c = c;
    g.l = l;
    g.m = m;
    g.k = k;
    return g;
}

}  // namespace

// Split-K partial sums of nvfp4_gemv_launch_noalloc.  Host code never passes
// this name to a kernel or a copy: on the host it is only a stand-in for the
// symbol, and the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
void *scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}
}  // namespace

void *nvfp4_stream_workspace(int dev, void *stream, size_t need) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto &slot = g_ws[std::make_pair(dev, stream)];
    if (slot.second >= need) return slot.first;
    if (stream_capturing(stream)) return nullptr;
    size_t bytes = slot.second > need / 2 ? 2 * slot.second : need;
    bytes = (bytes + 255) & ~size_t(255);
    void *ptr = nullptr;
    if (hipMalloc(&ptr, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    if (slot.first) g_ws_retired.push_back(slot.first);
    slot = std::make_pair(ptr, bytes);
    return ptr;
}

extern "C" {

const char *nvfp4_gemv_status_string(int status) {
    switch (status) {
    case NVFP4_GEMV_OK: return "ok";
    case NVFP4_GEMV_ERR_NULL_POINTER: return "a required pointer is NULL";
    case NVFP4_GEMV_ERR_BAD_SHAPE:
        return "bad shape: need l, m >= 1, k >= 16, k % 16 == 0, l*m < 2^31, k < 2^31";
    case NVFP4_GEMV_ERR_WORKSPACE: return "workspace missing, too small or not allocatable";
    case NVFP4_GEMV_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case NVFP4_GEMV_ERR_ALIAS: return "the output c overlaps an input";
    case NVFP4_GEMV_ERR_ALIGNMENT: return "c must be 2-byte, alpha and workspace 4-byte aligned";
    case NVFP4_GEMV_ERR_DEVICE: return "no current HIP device";
    case NVFP4_GEMV_ERR_BAD_TUNING: return "invalid tuning request for this shape";
    case NVFP4_GEMV_ERR_BAD_ARGUMENT: return "an enumerated argument (rule, flag) is out of range";
    default: return "unknown status";
    }
}

int nvfp4_gemv_num_variants(void) { return kNumVariants; }

int nvfp4_gemv_variant_info(int v, int32_t *rows_per_wave, int32_t *iters_in_flight,
                            int32_t *waves_per_group, int32_t *x_staging) {
    if (!rows_per_wave || !iters_in_flight || !waves_per_group || !x_staging)
        return NVFP4_GEMV_ERR_NULL_POINTER;
    if (v < 1 || v > kNumVariants) return NVFP4_GEMV_ERR_BAD_TUNING;
    *rows_per_wave = kVariants[v - 1].R;
    *iters_in_flight = kVariants[v - 1].U;
    *waves_per_group = kVariants[v - 1].W;
    *x_staging = kVariants[v - 1].xform;
    return NVFP4_GEMV_OK;
}

int nvfp4_gemv_plan(int64_t l, int64_t m, int64_t k, int aligned, const nvfp4_gemv_tuning_t *in,
                    nvfp4_gemv_tuning_t *out, size_t *workspace_bytes) {
    if (!out || !workspace_bytes) return NVFP4_GEMV_ERR_NULL_POINTER;
    const int s = check_shape(l, m, k);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    const int st = make_plan(l, m, k, aligned != 0, in, &p);
    if (st != NVFP4_GEMV_OK) return st;
    out->path = p.path;
    out->variant = p.path == NVFP4_GEMV_PATH_GENERIC ? 0 : p.variant + 1;
    out->ksplit = static_cast<int32_t>(p.ksplit);
    out->reserved = 0;
    *workspace_bytes = p.ws_bytes;
    return NVFP4_GEMV_OK;
}

size_t nvfp4_gemv_workspace_size(int64_t l, int64_t m, int64_t k) {
    if (check_shape(l, m, k) != NVFP4_GEMV_OK) return 0;
    // the larger of the fast and generic plans, so the size holds whatever the
    // operands' alignment turns out to be
    Plan fast, generic;
    if (make_plan(l, m, k, true, nullptr, &fast) != NVFP4_GEMV_OK) return 0;
    if (make_plan(l, m, k, false, nullptr, &generic) != NVFP4_GEMV_OK) return 0;
    return fast.ws_bytes > generic.ws_bytes ? fast.ws_bytes : generic.ws_bytes;
}

int nvfp4_gemv_launch_tuned(const uint8_t *A_packed, const uint8_t *sfA, const uint8_t *x_packed,
                            const uint8_t *sfx, const float *alpha, uint16_t *c, int64_t l,
                            int64_t m, int64_t k, const nvfp4_gemv_tuning_t *tuning,
                            void *workspace, size_t workspace_bytes, void *stream) {
    HipBackend be;
    return launch_caller_workspace(be, gemv_args(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k),
                                   tuning, workspace, workspace_bytes, stream);
}

int nvfp4_gemv_launch_ws(const uint8_t *A_packed, const uint8_t *sfA, const uint8_t *x_packed,
                         const uint8_t *sfx, const float *alpha, uint16_t *c, int64_t l,
                         int64_t m, int64_t k, void *workspace, size_t workspace_bytes,
                         void *stream) {
    return nvfp4_gemv_launch_tuned(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k, nullptr,
                                   workspace, workspace_bytes, stream);
}

int nvfp4_gemv_launch(const uint8_t *A_packed, const uint8_t *sfA, const uint8_t *x_packed,
                      const uint8_t *sfx, const float *alpha, uint16_t *c, int64_t l, int64_t m,
                      int64_t k, void *stream) {
    HipBackend be;
    return launch_owned_workspace(be, gemv_args(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k),
                                  stream);
}

int nvfp4_gemv_launch_noalloc(const uint8_t *A_packed, const uint8_t *sfA,
                              const uint8_t *x_packed, const uint8_t *sfx, const float *alpha,
                              uint16_t *c, int64_t l, int64_t m, int64_t k, void *stream) {
    HipBackend be;
    return launch_fixed_scratch(be, gemv_args(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k),
                                stream);
}

int nvfp4_workspace_reserve(size_t bytes, void *stream) {
    if (bytes == 0) return NVFP4_GEMV_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return NVFP4_GEMV_ERR_DEVICE;
    }
    return nvfp4_stream_workspace(dev, stream, bytes) ? NVFP4_GEMV_OK : NVFP4_GEMV_ERR_WORKSPACE;
}

int nvfp4_hbm_read_probe(const void *buffer, size_t bytes, uint32_t *sink, void *stream) {
    if (!buffer || !sink) return NVFP4_GEMV_ERR_NULL_POINTER;
    if (bytes == 0 || bytes % 16 != 0 || bytes > static_cast<size_t>(INT64_MAX))
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (reinterpret_cast<uintptr_t>(buffer) % 16 != 0 || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return NVFP4_GEMV_ERR_ALIGNMENT;
    const int64_t nbytes = static_cast<int64_t>(bytes);
    // a workgroup per 16 KiB chunk, up to kProbeMaxGroups (each then takes several)
    int64_t groups = ceil_div(nbytes, kProbeChunk);
    if (groups > kProbeMaxGroups) groups = kProbeMaxGroups;
    const uint8_t *buf = static_cast<const uint8_t *>(buffer);
    void *args[] = {&buf, const_cast<int64_t *>(&nbytes), &sink};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(hbm_read_probe),
                                   dim3(static_cast<uint32_t>(groups)), dim3(kProbeThreads), args,
                                   0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_GEMV_OK : NVFP4_GEMV_ERR_LAUNCH;
}

int nvfp4_hbm_read_probe_rows(const uint8_t *A, const uint8_t *sfA, int64_t rows, int64_t k,
                              uint32_t *sink, void *stream) {
    if (!A || !sfA || !sink) return NVFP4_GEMV_ERR_NULL_POINTER;
    if (rows < 1 || k < 32 || k % 32 != 0 || k >= (int64_t(1) << 31) || rows > INT64_MAX / (k / 2))
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    const int64_t rows_per_group = int64_t(kRowProbeR) * kRowProbeW;
    const int64_t groups = ceil_div(rows, rows_per_group);
    if (groups >= (int64_t(1) << 31)) return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (reinterpret_cast<uintptr_t>(A) % 16 != 0 || reinterpret_cast<uintptr_t>(sfA) % 2 != 0 ||
        reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return NVFP4_GEMV_ERR_ALIGNMENT;
    void *args[] = {&A, &sfA, &rows, &k, &sink};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(hbm_read_rows),
                                         dim3(static_cast<uint32_t>(groups)),
                                         dim3(kRowProbeW * kWave), args, 0,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_GEMV_OK : NVFP4_GEMV_ERR_LAUNCH;
}

}  // extern "C"
