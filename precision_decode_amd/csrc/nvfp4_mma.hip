// NVFP4 block-scaled products of a weight matrix with several vectors on
// MI355X (gfx950): the small-N GEMM (n vectors per weight matrix) and the
// grouped (MoE) GEMV (the tokens of each expert against that expert's
// weights).  The scaled dot product is the NVFP4 batched GEMV's ("nvFP4 Batch
// GEMV算子系列(下)", section "NVFP4 Batched GEMV 概念阐述"); the grouped form is
// the 2D x 3D grouped GEMM of the CuTeDSL bridge page (section "Kernel
// Launch"), shrunk to one output column per token.
//
// With up to 16 vectors per weight row the VALU can no longer do every
// product (each weight element meets up to 16 vectors), while the bytes are
// still those of a GEMV: weights are read once and dominate the traffic.  So
// the products go to the matrix cores and the VALU only decodes:
//
//  * a weight element times its block scale, e2m1 * e4m3, has at most 5
//    significant bits and lies in 2^-10 .. 2688, so it is exact in fp16; the
//    same holds for the vectors.  Each lane decodes 32 codes (16 bytes) and
//    their two block scales into four 8-element fp16 operands with the gfx950
//    packed FP4 -> fp16 conversion and one packed fp16 multiply per pair;
//  * v_mfma_f32_16x16x32_f16 multiplies a 16-row tile of weights by 16
//    vectors over 32 K elements; products of two such values are exact in
//    fp32 and the matrix core accumulates in fp32.  Lane i + 16q holds row
//    (or vector) i, elements 8q .. 8q+7 of the 32; the contraction does not
//    care which K element sits where as long as both operands agree, so a
//    lane's 16-byte load covers 32 consecutive elements, split over four
//    MFMA steps;
//  * each wave streams its tile rows with 16-byte non-temporal buffer loads
//    (two instructions per 128-byte line of 16 rows), keeps several windows
//    in flight, and reads the vectors' codes with ordinary (cached) loads:
//    every workgroup reads the same vectors, so they stay in L2;
//  * the waves of a workgroup share the tile rows and take interleaved
//    windows of its K range; their fp32 tiles are added in wave order through
//    LDS, so the result does not depend on scheduling.  Few tiles are
//    balanced by splitting K across workgroups (small-N GEMM only), with fp32
//    partials added in split order by a second kernel.
//
// Three other forms sit beside it: the same products fed through LDS by
// whole-line direct-to-LDS copies (mma_lds, the default for row-major
// weights; with few vectors, only the weights, the vectors going straight to
// registers), weights packed once into the order the lanes read them
// (mma_pack_weight; every load instruction then reads 1 KiB contiguously
// instead of 16 rows x 64 bytes), and, for one or two vectors, VALU row tiles
// that read the row-major weights row-contiguously and take the few dot
// products themselves (vec_tile).
//
// Every accumulator starts at +0.0, so an exactly-zero result is +0.  With
// integer-coded inputs (E2M1 values times scales 0, 1, 2) every partial sum is
// a multiple of 1/4 below 2^22, exact in fp32 in any order.
//
// This file holds the host side (validation, launches, the C-ABI entry
// points); the device code is mma_kernels.h and the plan (shape rules,
// variants, defaults) mma_plan.h.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cstdint>
#include "device_common.h"
#include "mma_kernels.h"
#include "mma_plan.h"
#include "nvfp4_gemv.h"
#include "nvfp4_mma.h"

namespace {

using namespace nvfp4dev;
using namespace nvfp4mmaplan;

// ---------------------------------------------------------------- host side
// (shape rules, variants, defaults and the launch plan are in mma_plan.h)
typedef void (*MmaKernel)(const MmaArgs);

template <bool G, bool P, bool S16 = false>
MmaKernel fast_kernel(int v) {
    switch (v) {
    case 0: return mma_stream<1, 2, 4, G, P>;
    case 1: return mma_stream<1, 2, 8, G, P>;
    case 2: return mma_stream<2, 2, 4, G, P>;
    case 3: return mma_stream<2, 1, 8, G, P>;
    case 4: return mma_stream<1, 3, 4, G, P>;
    case 5: return mma_stream<2, 2, 8, G, P>;
    case 6: return P ? nullptr : vec_tile<4, 2, 4, G>;
    case 7: return P ? nullptr : vec_tile<8, 2, 4, G>;
    case 8: return P ? nullptr : vec_tile<4, 4, 4, G>;
    case 9: return P ? nullptr : vec_tile<8, 4, 4, G>;
    case 10: return P ? nullptr : mma_lds<2, 2, 4, G, S16, false, true>;
    case 11: return P ? nullptr : mma_lds<2, 4, 4, G, S16>;
    case 12: return P ? nullptr : mma_lds<1, 2, 4, G, S16>;
    case 13: return P ? nullptr : mma_lds<2, 2, 6, G, S16>;
    case 14: return P ? nullptr : mma_lds<2, 2, 8, G, S16>;
    case 15: return P ? nullptr : mma_lds<2, 2, 2, G, S16>;
    case 16: return P ? nullptr : mma_lds<2, 4, 2, G, S16>;
    case 17: return P ? nullptr : mma_lds<2, 2, 4, G, S16, true, true>;
    case 18: return P ? nullptr : mma_lds<2, 2, 2, G, S16, true>;
    case 19: return P ? nullptr : vec_tile<4, 1, 4, G>;
    default: return nullptr;
    }
}

bool overlaps(const void *p, size_t pn, const void *q, size_t qn) {
    if (!p || !q || pn == 0 || qn == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + qn && b < a + pn;
}

bool aligned_ptrs(const void *w, const void *sw, const void *v, const void *sv) {
    auto al = [](const void *p, uintptr_t n) { return reinterpret_cast<uintptr_t>(p) % n == 0; };
    return al(w, 16) && al(v, 16) && al(sw, 4) && al(sv, 4);
}

int launch(const Plan &p, bool grouped, MmaArgs a, hipStream_t stream, bool packed = false) {
    a.kchunk = p.kchunk;
    a.row_blocks = p.row_blocks;
    a.rows_per_block = p.rows_per_block;
    // LDS-staged variants copy block scales 16 bytes at a time when every
    // scale row, workgroup K range and window group starts 16-byte aligned
    const bool s16 = a.k % 256 == 0 && a.kchunk % 256 == 0 &&
                     reinterpret_cast<uintptr_t>(a.sW) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(a.sV) % 16 == 0;
    const void *fn;
    if (p.path == NVFP4_GEMV_PATH_FAST)
        fn = reinterpret_cast<const void *>(
            grouped ? (packed ? fast_kernel<true, true>(p.variant)
                              : s16 ? fast_kernel<true, false, true>(p.variant)
                                    : fast_kernel<true, false>(p.variant))
                    : (packed ? fast_kernel<false, true>(p.variant)
                              : s16 ? fast_kernel<false, false, true>(p.variant)
                                    : fast_kernel<false, false>(p.variant)));
    else
        fn = reinterpret_cast<const void *>(grouped ? mma_generic<true> : mma_generic<false>);
    void *args[] = {&a};
    hipError_t e = hipLaunchKernel(fn, dim3(static_cast<uint32_t>(p.groups)), dim3(p.threads), args,
                                   0, stream);
    if (e != hipSuccess) return NVFP4_GEMV_ERR_LAUNCH;
    if (a.part != nullptr) {
        const float *part = a.part;
        const float *alpha = a.alpha;
        uint16_t *c = a.c;
        int64_t total = a.groups * a.rows * a.nvec, per_group = a.rows * a.nvec, ks = p.ksplit;
        int32_t bf = a.out_bf16;
        void *rargs[] = {&part, &alpha, &c, &total, &per_group, &ks, &bf};
        e = hipLaunchKernel(reinterpret_cast<const void *>(mma_splitk_reduce),
                            dim3(static_cast<uint32_t>(ceil_div(total, kReduceThreads))),
                            dim3(kReduceThreads), rargs, 0, stream);
        if (e != hipSuccess) return NVFP4_GEMV_ERR_LAUNCH;
    }
    return NVFP4_GEMV_OK;
}

// Bytes of the packed codes and scales of `groups` matrices of rows x k
// (whole 16-row tiles and 256-element windows); false if they overflow.
bool packed_sizes(int64_t groups, int64_t rows, int64_t k, int64_t *codes, int64_t *scales) {
    const int64_t tiles = ceil_div(rows, int64_t(kTile)), wins = ceil_div(k, int64_t(kWinElems));
    if (!fits_int64_product(groups, tiles) || !fits_int64_product(groups * tiles, wins) ||
        !fits_int64_product(groups * tiles * wins, kPackedWinBytes))
        return false;
    *codes = groups * tiles * wins * kPackedWinBytes;
    *scales = groups * tiles * wins * kPackedWinScaleBytes;
    return true;
}

// Shape and pointer rules of the packed launches: the fast kernel's (k % 64,
// k <= 2^26, 16-byte codes, 4-byte scales), since packed weights have no
// generic path.
int check_packed(int64_t groups, int64_t rows, int64_t k, const void *Wp, const void *sWp,
                 const void *V, const void *sV, int64_t *codes, int64_t *scales) {
    if (k % 64 != 0 || k > kMaxFastK || !packed_sizes(groups, rows, k, codes, scales))
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (!aligned_ptrs(Wp, sWp, V, sV)) return NVFP4_GEMV_ERR_ALIGNMENT;
    return NVFP4_GEMV_OK;
}

int validate_smalln(const uint8_t *A, const uint8_t *sfA, const uint8_t *B, const uint8_t *sfB,
                    const float *alpha, uint16_t *c, int64_t l, int64_t m, int64_t n, int64_t k,
                    int32_t out_type, bool packed = false) {
    if (!A || !sfA || !B || !sfB || !c) return NVFP4_GEMV_ERR_NULL_POINTER;
    if (out_type != NVFP4_OUT_F16 && out_type != NVFP4_OUT_BF16) return NVFP4_GEMV_ERR_BAD_ARGUMENT;
    int s = check_smalln_shape(l, m, n, k);
    if (s != NVFP4_GEMV_OK) return s;
    if (reinterpret_cast<uintptr_t>(c) % 2 != 0 || reinterpret_cast<uintptr_t>(alpha) % 4 != 0)
        return NVFP4_GEMV_ERR_ALIGNMENT;
    int64_t ab = l * m * (k / 2), sb = l * m * (k / 16);
    if (packed) {
        s = check_packed(l, m, k, A, sfA, B, sfB, &ab, &sb);
        if (s != NVFP4_GEMV_OK) return s;
    }
    const size_t cn = static_cast<size_t>(l * m * n) * 2;
    if (overlaps(c, cn, A, static_cast<size_t>(ab)) || overlaps(c, cn, sfA, static_cast<size_t>(sb)) ||
        overlaps(c, cn, B, static_cast<size_t>(l * n) * (k / 2)) ||
        overlaps(c, cn, sfB, static_cast<size_t>(l * n) * (k / 16)) ||
        overlaps(c, cn, alpha, static_cast<size_t>(l) * 4))
        return NVFP4_GEMV_ERR_ALIAS;
    return NVFP4_GEMV_OK;
}

int validate_grouped(const uint8_t *X, const uint8_t *sfX, const uint8_t *W, const uint8_t *sfW,
                     const int32_t *offsets, const float *gs_x, const float *gs_w, uint16_t *c,
                     int64_t tokens, int64_t experts, int64_t n, int64_t k, int32_t out_type,
                     bool packed = false) {
    if (!X || !sfX || !W || !sfW || !offsets || !c) return NVFP4_GEMV_ERR_NULL_POINTER;
    if (out_type != NVFP4_OUT_F16 && out_type != NVFP4_OUT_BF16) return NVFP4_GEMV_ERR_BAD_ARGUMENT;
    int s = check_grouped_shape(tokens, experts, n, k);
    if (s != NVFP4_GEMV_OK) return s;
    auto mis = [](const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; };
    if (mis(c, 2) || mis(offsets, 4) || mis(gs_x, 4) || mis(gs_w, 4)) return NVFP4_GEMV_ERR_ALIGNMENT;
    int64_t wb = experts * n * (k / 2), swb = experts * n * (k / 16);
    if (packed) {
        s = check_packed(experts, n, k, W, sfW, X, sfX, &wb, &swb);
        if (s != NVFP4_GEMV_OK) return s;
    }
    const size_t cn = static_cast<size_t>(tokens * n) * 2;
    if (overlaps(c, cn, X, static_cast<size_t>(tokens) * (k / 2)) ||
        overlaps(c, cn, sfX, static_cast<size_t>(tokens) * (k / 16)) ||
        overlaps(c, cn, W, static_cast<size_t>(wb)) || overlaps(c, cn, sfW, static_cast<size_t>(swb)) ||
        overlaps(c, cn, offsets, static_cast<size_t>(experts) * 4) ||
        overlaps(c, cn, gs_x, static_cast<size_t>(experts) * 4) ||
        overlaps(c, cn, gs_w, static_cast<size_t>(experts) * 4))
        return NVFP4_GEMV_ERR_ALIAS;
    return NVFP4_GEMV_OK;
}

MmaArgs smalln_args(const uint8_t *A, const uint8_t *sfA, const uint8_t *B, const uint8_t *sfB,
                    const float *alpha, uint16_t *c, int64_t l, int64_t m, int64_t n, int64_t k,
                    int32_t out_type, float *part) {
    MmaArgs a = {};
    a.W = A;
    a.sW = sfA;
    a.V = B;
    a.sV = sfB;
    a.alpha = alpha;
    a.c = c;
    a.part = part;
    a.groups = l;
    a.rows = m;
    a.nvec = n;
    a.k = k;
    a.out_bf16 = out_type == NVFP4_OUT_BF16;
    return a;
}

}  // namespace

extern "C" {

int nvfp4_mma_num_variants(void) { return kNumVariants; }

int nvfp4_mma_variant_info(int v, int32_t *row_tiles_per_wave, int32_t *windows_in_flight,
                           int32_t *waves_per_group) {
    if (!row_tiles_per_wave || !windows_in_flight || !waves_per_group)
        return NVFP4_GEMV_ERR_NULL_POINTER;
    if (v < 1 || v > kNumVariants) return NVFP4_GEMV_ERR_BAD_TUNING;
    *row_tiles_per_wave = kVariants[v - 1].R;
    *windows_in_flight = kVariants[v - 1].U;
    *waves_per_group = kVariants[v - 1].W;
    return NVFP4_GEMV_OK;
}

int nvfp4_mma_variant_form(int v, int32_t *form) {
    if (!form) return NVFP4_GEMV_ERR_NULL_POINTER;
    if (v < 1 || v > kNumVariants) return NVFP4_GEMV_ERR_BAD_TUNING;
    *form = kVariants[v - 1].form;
    return NVFP4_GEMV_OK;
}

int nvfp4_gemm_smalln_plan(int64_t l, int64_t m, int64_t n, int64_t k, int aligned,
                           const nvfp4_mma_tuning_t *in, nvfp4_mma_tuning_t *out,
                           size_t *workspace_bytes) {
    if (!out || !workspace_bytes) return NVFP4_GEMV_ERR_NULL_POINTER;
    int s = check_smalln_shape(l, m, n, k);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(l, m, n, k, aligned != 0, false, in, &p);
    if (s != NVFP4_GEMV_OK) return s;
    out->path = p.path;
    out->variant = p.path == NVFP4_GEMV_PATH_FAST ? p.variant + 1 : 0;
    out->ksplit = static_cast<int32_t>(p.ksplit);
    out->rows_per_block = p.path == NVFP4_GEMV_PATH_FAST ? static_cast<int32_t>(p.rows_per_block) : 0;
    *workspace_bytes = p.ws_bytes;
    return NVFP4_GEMV_OK;
}

int nvfp4_grouped_gemv_plan(int64_t experts, int64_t n, int64_t k, int64_t tokens, int aligned,
                            int packed, const nvfp4_mma_tuning_t *in, nvfp4_mma_tuning_t *out) {
    if (!out) return NVFP4_GEMV_ERR_NULL_POINTER;
    int s = check_grouped_shape(tokens, experts, n, k);
    if (s != NVFP4_GEMV_OK) return s;
    if (packed && (k % 64 != 0 || k > kMaxFastK)) return NVFP4_GEMV_ERR_BAD_SHAPE;
    Plan p;
    s = make_plan(experts, n, ceil_div(tokens, experts), k, packed != 0 || aligned != 0, true, in, &p,
                  packed != 0);
    if (s != NVFP4_GEMV_OK) return s;
    out->path = p.path;
    out->variant = p.path == NVFP4_GEMV_PATH_FAST ? p.variant + 1 : 0;
    out->ksplit = static_cast<int32_t>(p.ksplit);
    out->rows_per_block = p.path == NVFP4_GEMV_PATH_FAST ? static_cast<int32_t>(p.rows_per_block) : 0;
    return NVFP4_GEMV_OK;
}

int nvfp4_gemm_smalln_launch_tuned(const uint8_t *A_packed, const uint8_t *sfA,
                                   const uint8_t *B_packed, const uint8_t *sfB,
                                   const float *alpha, uint16_t *c, int64_t l, int64_t m,
                                   int64_t n, int64_t k, int32_t out_type,
                                   const nvfp4_mma_tuning_t *tuning, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    int s = validate_smalln(A_packed, sfA, B_packed, sfB, alpha, c, l, m, n, k, out_type);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(l, m, n, k, aligned_ptrs(A_packed, sfA, B_packed, sfB), false, tuning, &p);
    if (s != NVFP4_GEMV_OK) return s;
    float *part = nullptr;
    if (p.ws_bytes > 0) {
        if (!workspace || workspace_bytes < p.ws_bytes) return NVFP4_GEMV_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(workspace) % 4 != 0) return NVFP4_GEMV_ERR_ALIGNMENT;
        part = static_cast<float *>(workspace);
    }
    return launch(p, false,
                  smalln_args(A_packed, sfA, B_packed, sfB, alpha, c, l, m, n, k, out_type, part),
                  static_cast<hipStream_t>(stream));
}

int nvfp4_gemm_smalln_launch(const uint8_t *A_packed, const uint8_t *sfA, const uint8_t *B_packed,
                             const uint8_t *sfB, const float *alpha, uint16_t *c, int64_t l,
                             int64_t m, int64_t n, int64_t k, int32_t out_type, void *stream) {
    int s = validate_smalln(A_packed, sfA, B_packed, sfB, alpha, c, l, m, n, k, out_type);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(l, m, n, k, aligned_ptrs(A_packed, sfA, B_packed, sfB), false, nullptr, &p);
    if (s != NVFP4_GEMV_OK) return s;
    float *part = nullptr;
    if (p.ws_bytes > 0) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return NVFP4_GEMV_ERR_DEVICE;
        part = static_cast<float *>(nvfp4_stream_workspace(dev, stream, p.ws_bytes));
        if (!part) return NVFP4_GEMV_ERR_WORKSPACE;
    }
    return launch(p, false,
                  smalln_args(A_packed, sfA, B_packed, sfB, alpha, c, l, m, n, k, out_type, part),
                  static_cast<hipStream_t>(stream));
}

int nvfp4_mma_packed_sizes(int64_t groups, int64_t rows, int64_t k, size_t *codes_bytes,
                           size_t *scales_bytes) {
    if (!codes_bytes || !scales_bytes) return NVFP4_GEMV_ERR_NULL_POINTER;
    int s = check_dims(groups, rows, 1, k, false);
    if (s != NVFP4_GEMV_OK) return s;
    int64_t cb, sb;
    if (k % 64 != 0 || k > kMaxFastK || !packed_sizes(groups, rows, k, &cb, &sb))
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    *codes_bytes = static_cast<size_t>(cb);
    *scales_bytes = static_cast<size_t>(sb);
    return NVFP4_GEMV_OK;
}

int nvfp4_mma_pack_weight(const uint8_t *W, const uint8_t *sW, int64_t groups, int64_t rows,
                          int64_t k, uint8_t *W_packed, uint8_t *sW_packed, void *stream) {
    if (!W || !sW || !W_packed || !sW_packed) return NVFP4_GEMV_ERR_NULL_POINTER;
    int s = check_dims(groups, rows, 1, k, false);
    if (s != NVFP4_GEMV_OK) return s;
    int64_t cb, sb;
    s = check_packed(groups, rows, k, W_packed, sW_packed, W, sW, &cb, &sb);
    if (s != NVFP4_GEMV_OK) return s;
    const size_t wb = static_cast<size_t>(groups * rows * (k / 2));
    const size_t swb = static_cast<size_t>(groups * rows * (k / 16));
    const void *outs[2] = {W_packed, sW_packed};
    const size_t outn[2] = {static_cast<size_t>(cb), static_cast<size_t>(sb)};
    for (int i = 0; i < 2; ++i)
        if (overlaps(outs[i], outn[i], W, wb) || overlaps(outs[i], outn[i], sW, swb))
            return NVFP4_GEMV_ERR_ALIAS;
    if (overlaps(W_packed, outn[0], sW_packed, outn[1])) return NVFP4_GEMV_ERR_ALIAS;
    const int64_t blocks = ceil_div(cb / 16, int64_t(kPackThreads));
    if (blocks >= (int64_t(1) << 31)) return NVFP4_GEMV_ERR_BAD_SHAPE;
    void *args[] = {&W, &sW, &W_packed, &sW_packed, &groups, &rows, &k};
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(mma_pack_weight),
                                         dim3(static_cast<uint32_t>(blocks)), dim3(kPackThreads),
                                         args, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NVFP4_GEMV_OK : NVFP4_GEMV_ERR_LAUNCH;
}

int nvfp4_gemm_smalln_launch_packed(const uint8_t *A_packed, const uint8_t *sfA_packed,
                                    const uint8_t *B_packed, const uint8_t *sfB,
                                    const float *alpha, uint16_t *c, int64_t l, int64_t m,
                                    int64_t n, int64_t k, int32_t out_type,
                                    const nvfp4_mma_tuning_t *tuning, void *stream) {
    int s = validate_smalln(A_packed, sfA_packed, B_packed, sfB, alpha, c, l, m, n, k, out_type,
                            true);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(l, m, n, k, true, false, tuning, &p, true);
    if (s != NVFP4_GEMV_OK) return s;
    float *part = nullptr;
    if (p.ws_bytes > 0) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return NVFP4_GEMV_ERR_DEVICE;
        part = static_cast<float *>(nvfp4_stream_workspace(dev, stream, p.ws_bytes));
        if (!part) return NVFP4_GEMV_ERR_WORKSPACE;
    }
    return launch(p, false,
                  smalln_args(A_packed, sfA_packed, B_packed, sfB, alpha, c, l, m, n, k, out_type,
                              part),
                  static_cast<hipStream_t>(stream), true);
}

int nvfp4_grouped_gemv_launch_packed(const uint8_t *X_packed, const uint8_t *sfX,
                                     const uint8_t *W_packed, const uint8_t *sfW_packed,
                                     const int32_t *offsets, const float *gs_x, const float *gs_w,
                                     uint16_t *c, int64_t tokens, int64_t experts, int64_t n,
                                     int64_t k, int32_t out_type, const nvfp4_mma_tuning_t *tuning,
                                     void *stream) {
    int s = validate_grouped(X_packed, sfX, W_packed, sfW_packed, offsets, gs_x, gs_w, c, tokens,
                             experts, n, k, out_type, true);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(experts, n, ceil_div(tokens, experts), k, true, true, tuning, &p, true);
    if (s != NVFP4_GEMV_OK) return s;
    if (tokens == 0) return NVFP4_GEMV_OK;
    MmaArgs a = {};
    a.W = W_packed;
    a.sW = sfW_packed;
    a.V = X_packed;
    a.sV = sfX;
    a.offsets = offsets;
    a.gs_v = gs_x;
    a.gs_w = gs_w;
    a.c = c;
    a.groups = experts;
    a.rows = n;
    a.nvec = tokens;
    a.k = k;
    a.out_bf16 = out_type == NVFP4_OUT_BF16;
    return launch(p, true, a, static_cast<hipStream_t>(stream), true);
}

int nvfp4_grouped_gemv_launch_tuned(const uint8_t *X_packed, const uint8_t *sfX,
                                    const uint8_t *W_packed, const uint8_t *sfW,
                                    const int32_t *offsets, const float *gs_x, const float *gs_w,
                                    uint16_t *c, int64_t tokens, int64_t experts, int64_t n,
                                    int64_t k, int32_t out_type, const nvfp4_mma_tuning_t *tuning,
                                    void *stream) {
    int s = validate_grouped(X_packed, sfX, W_packed, sfW, offsets, gs_x, gs_w, c, tokens, experts,
                             n, k, out_type);
    if (s != NVFP4_GEMV_OK) return s;
    Plan p;
    s = make_plan(experts, n, ceil_div(tokens, experts), k, aligned_ptrs(W_packed, sfW, X_packed, sfX),
                  true, tuning, &p);
    if (s != NVFP4_GEMV_OK) return s;
    if (tokens == 0) return NVFP4_GEMV_OK;
    MmaArgs a = {};
    a.W = W_packed;
    a.sW = sfW;
    a.V = X_packed;
    a.sV = sfX;
    a.offsets = offsets;
    a.gs_v = gs_x;
    a.gs_w = gs_w;
    a.c = c;
    a.groups = experts;
    a.rows = n;
    a.nvec = tokens;
    a.k = k;
    a.out_bf16 = out_type == NVFP4_OUT_BF16;
    return launch(p, true, a, static_cast<hipStream_t>(stream));
}

int nvfp4_grouped_gemv_launch(const uint8_t *X_packed, const uint8_t *sfX, const uint8_t *W_packed,
                              const uint8_t *sfW, const int32_t *offsets, const float *gs_x,
                              const float *gs_w, uint16_t *c, int64_t tokens, int64_t experts,
                              int64_t n, int64_t k, int32_t out_type, void *stream) {
    return nvfp4_grouped_gemv_launch_tuned(X_packed, sfX, W_packed, sfW, offsets, gs_x, gs_w, c,
                                           tokens, experts, n, k, out_type, nullptr, stream);
}

}  // extern "C"
