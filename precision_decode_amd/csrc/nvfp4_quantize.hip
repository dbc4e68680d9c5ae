// BF16 -> NVFP4 quantisation on the GPU (gfx950), and the GEMV fed by it.
//
// The quantiser follows the graph-safe activation quantiser of the CuTeDSL
// NVFP4 bridge page (section "Quantization"): the fp32 global scale is given
// (computed once, e.g. during warm-up) rather than taken from the tensor's
// amax, so the call needs no host synchronisation.  For every 16-element block
// along the last axis, all arithmetic in fp32 with IEEE rounding:
//
//   xn   = x / g                                (correctly rounded division)
//   am   = max(max_i |xn_i|, 1e-8)              (NaN propagates)
//   s    = e4m3_rne(am / 6)                     (past 464: the NaN pattern 0x7F)
//   v_i  = xn_i / max(e4m3(s), 1e-8)            (NaN propagates)
//   code = E2M1 magnitude index of |v_i| by the rounding rule, + 8 when v_i < 0
//
// Rounding rules: the page's activation quantiser doubles |v| (clamped to 6),
// rounds to the nearest integer (ties to even) and maps the result through its
// half-step table; its weight quantiser takes the argmin of the fp32 distances
// to the eight magnitudes (first index on ties); nearest-even rounds to the
// nearest magnitude with ties to the even code.  A NaN v gets code 0.
//
// Work mapping: one lane per 16-element block (32 bytes of bf16 in, 8 bytes of
// codes and 1 scale byte out), blocks numbered across rows so any row length
// that is a multiple of 16 keeps the wave's loads and stores contiguous.  A
// wave reads its 64 blocks (2 KiB) with two 16-byte loads per lane that each
// cover 1 KiB contiguously, and hands every lane its block through LDS.  The
// divisions round exactly as IEEE division does without its cost: x / g as
// an fp64 product with 1/g (the quotient of a bf16 by an fp32 never lies
// within 2^-49 of an fp32 rounding midpoint, the fp64 product with a
// reciprocal within one ulp is within 2^-51), x_n / s as one reciprocal and one fused residual correction (the
// block scale has 4 significant bits, so quotients stay 2^-29 away from
// midpoints); blocks outside the range this holds for take IEEE divisions.
// The E2M1 rounding of every rule runs on gfx950's FP4 conversion.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "device_common.h"
#include "nvfp4_gemv.h"
#include "nvfp4_quantize.h"
#include "quant_arith.h"

namespace {

using namespace nvfp4quant;
using nvfp4dev::kWave;
using nvfp4dev::u32x4;
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantThreads = 256;

// Codes of 16 values v[i] (element i at nibble i of the 64-bit result) under
// the rule, sign bit 8 for v < 0, NaN -> 0, all on the gfx950 FP4 conversion,
// which rounds to nearest even on the E2M1 grid and saturates at 6, with the
// sign of v.  It differs from the rules only at -0 (code 8, not 0) and NaN,
// which the caller rules out.
//  * nearest-even: the conversion itself;
//  * nearest-lower (argmin of fp32 distances, first on ties): the ties where
//    nearest-even goes up (0.75, 1.75, 3.5) are exactly the grid midpoints
//    whose fp32 pattern has mantissa bit 22 set and bits 20..0 clear; those
//    values, and only ever values whose rounding one ulp down cannot change
//    (grid points, non-midpoints), move one ulp towards zero first.  For
//    |v| <= 2^20, which every block satisfies (|v| <= 6.25, or < 6e5 when the
//    block scale rounds to zero), the fp32 distances are exact near every tie,
//    so the argmin is the nearest value with ties down, and 6 beyond the grid;
//  * half-step (the page's table on rint(2 min(|v|, 6))): below 2 the table is
//    nearest-even on the grid; from 2 its cut points 2.75, 3.75 and 5.25 sit
//    0.25 above the grid midpoints 2.5, 3.5 and 5, whose ties go to the even
//    codes (2, 4 and 4).  The table sends 3.75 up and 5.25 down, as those ties
//    do, but 2.75 up, against its tie.  So f(a) = RN(a (1 - 2^-24) - 0.25 +
//    5 2^-24), one fma, is rounded instead, clamped below at 2 (med3):
//    f(a) = a - 0.25 + (5 - a) 2^-24 before rounding, so f(2.75) lands
//    2.25 2^-24 above 2.5 and rounds to the float above it (half an ulp there
//    is 2 2^-24), f(3.75) and f(5.25) round onto 3.5 and 5 exactly, and every
//    float next to a cut rounds to the side it belongs to.  Checked against
//    the table for every finite fp32 |v| on the CPU.

template <int RULE>
__device__ __forceinline__ u32x2 block_codes(const float (&v)[16]) {
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if constexpr (RULE == NVFP4_ROUND_NEAREST_LOWER) {
            const uint32_t b = __float_as_uint(v[i]);
            t[i] = __uint_as_float(b - ((b & 0x005FFFFFu) == 0x00400000u ? 1u : 0u));
        } else if constexpr (RULE == NVFP4_ROUND_HALF_STEP) {
            const float a = __builtin_fabsf(v[i]);
            const float m = __builtin_amdgcn_fmed3f(
                __builtin_fmaf(a, kHalfStepScale, kHalfStepShift), a, 2.0f);
            t[i] = __builtin_copysignf(m, v[i]);
        } else {
            t[i] = v[i];
        }
    }
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        w[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j], t[8 * j + 0], t[8 * j + 1], 1.0f, 0);
        w[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j], t[8 * j + 2], t[8 * j + 3], 1.0f, 1);
        w[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j], t[8 * j + 4], t[8 * j + 5], 1.0f, 2);
        w[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j], t[8 * j + 6], t[8 * j + 7], 1.0f, 3);
    }
    return u32x2{w[0], w[1]};
}

// One 16-element block: bf16 words w0, w1 (elements 2i, 2i+1 in word i) with
// global scale g -> 8 bytes of codes and the E4M3 scale code.
//
// The block amax of |x/g| is RN(max|x| / |g|) (rounding is monotonic), taken
// on the bf16 magnitude patterns (NaN patterns sort above +Inf, so a NaN
// wins).  Fast path, for g in [2^-40, 2^30] and every nonzero |x| >= 2^-100:
// x/g through quot_f64 and, unless the block scale rounded to zero, v = x_n / s
// through quot_short, which round as IEEE division does here (a quotient too
// small for the fp32 normal range only ever counts by its sign, which both
// keep).  Other blocks (a subnormal input, an extreme or non-finite scale)
// take IEEE divisions.
template <int RULE>
__device__ __forceinline__ void quantize_one(u32x4 w0, u32x4 w1, float g, u32x2 *codes,
                                             uint32_t *scale) {
    const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    // largest magnitude pattern and smallest nonzero one (pattern - 1, zero
    // wraps to the top), two bf16 values per 16-bit lane pair
    u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const u16x2 m = __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu);
        mx = __builtin_elementwise_max(mx, m);
        mn = __builtin_elementwise_min(mn, static_cast<u16x2>(m - u16x2{1, 1}));
    }
    const uint32_t maxp = mx.x > mx.y ? mx.x : mx.y;
    const uint32_t tiny = mn.x < mn.y ? mn.x : mn.y;
    const bool fast = g >= 0x1p-40f && g <= 0x1p30f && tiny >= (27u << 7) - 1u;   // 2^-100

    float xn[16];
    float am;
    if (fast) {
        const double yg = recip_f64(static_cast<double>(g));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xn[2 * i] = quot_f64(bf16_to_f32(w[i] & 0xFFFFu), yg);
            xn[2 * i + 1] = quot_f64(__uint_as_float(w[i] & 0xFFFF0000u), yg);
        }
        am = quot_f64(bf16_to_f32(maxp), yg);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xn[2 * i] = bf16_to_f32(w[i] & 0xFFFFu) / g;
            xn[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) / g;
        }
        am = bf16_to_f32(maxp) / __builtin_fabsf(g);
    }
    am = am < 1e-8f ? 1e-8f : am;                  // NaN stays NaN
    // am / 6 with am >= 1e-8: quot_f64 is exact (6 has 2 significant bits)
    const uint32_t s = e4m3_code_pos(quot_f64(am, 1.0 / 6.0));
    const float sv = e4m3_value_pos(s);
    const float den = sv < 1e-8f ? 1e-8f : sv;     // NaN stays NaN

    float v[16];
    if (fast && s != 0u) {   // s == 0: den is the 1e-8 floor, not a 4-bit number
        const float yd = __builtin_amdgcn_rcpf(den);
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = quot_short(xn[i], den, yd);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = xn[i] / den + 0.0f;   // -0 -> +0: its code is 0
    }
    u32x2 out = block_codes<RULE>(v);
    if (s == 0x7Fu) out = u32x2{0u, 0u};           // a NaN block scale: every v is NaN, code 0
    *codes = out;
    *scale = s;
}

// One lane quantises one 16-element block; blocks are numbered across rows
// (block b is block b % bpr of row b / bpr).  A wave's 64 blocks are 2 KiB of
// x: each lane loads 16 bytes of each 1 KiB half (every load instruction
// reads 1 KiB contiguously), the wave stages them in LDS and every lane reads
// back the 32 bytes of its block.  `x` 16-byte aligned, `q` 8-byte aligned;
// gs_stride 0 (one scale) or 1 (one scale per row).  Lanes below `rows` also
// write alpha[row] = f32(other[row] * gs[row]) (or gs[row] when `other` is
// NULL) when `alpha` is not NULL.
template <int RULE>
__global__ __launch_bounds__(kQuantThreads) void quantize_blocks(
    const uint16_t *__restrict__ x, const float *__restrict__ gs, int64_t gs_stride,
    uint8_t *__restrict__ q, uint8_t *__restrict__ sf, int64_t nblocks, int64_t bpr,
    const float *__restrict__ other, float *__restrict__ alpha, int64_t rows) {
    __shared__ u32x4 stage[2 * kQuantThreads];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x;
    if (alpha != nullptr && b < rows) {
        const float g = gs[b * gs_stride];
        alpha[b] = other != nullptr ? other[b] * g : g;
    }
    const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kQuantThreads + wave * kWave;   // the wave's first block
    if (b0 >= nblocks) return;                     // wave-uniform
    const int nvalid = static_cast<int>(nblocks - b0 < kWave ? nblocks - b0 : kWave);
    // The lane's row, for a scale per row: the wave's first row and offset in
    // it once per wave (block numbers stay below 2^31, checked on the host),
    // then, when a row holds a wave's 64 blocks or more, at most one row
    // boundary inside the wave.  Lanes past the last block take the last row.
    uint32_t row = 0;
    if (gs_stride != 0) {
        const uint32_t ub0 = static_cast<uint32_t>(b0), ubpr = static_cast<uint32_t>(bpr);
        const uint32_t r0 = ub0 / ubpr;
        const uint32_t off = ub0 - r0 * ubpr + static_cast<uint32_t>(lane);
        row = r0 + (ubpr >= static_cast<uint32_t>(kWave) ? (off >= ubpr ? 1u : 0u) : off / ubpr);
        const uint32_t last = static_cast<uint32_t>(rows - 1);
        row = row < last ? row : last;
    }
    // the wave's blocks (loads past the last block read zeros), then the
    // block's global scale, all in flight together
    const __amdgpu_buffer_rsrc_t xr = nvfp4dev::buffer_of(
        reinterpret_cast<const uint8_t *>(x + b0 * 16), nvalid * 32);
    nvfp4dev::phase_fence();
    const u32x4 h0 = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, 16 * lane, 0, nvfp4dev::kNonTemporal));
    const u32x4 h1 = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, 1024 + 16 * lane, 0, nvfp4dev::kNonTemporal));
    const float g = gs[row * gs_stride];
    nvfp4dev::phase_fence();
    __asm__ volatile("" ::"v"(g));                 // keeps the load here, not after the staging
    u32x4 *st = stage + 2 * kWave * wave;          // the wave's 2 KiB
    st[lane] = h0;
    st[kWave + lane] = h1;
    // LDS operations of one wave complete in order; the fences keep the
    // compiler from moving the reads above the other lanes' writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 w0 = st[2 * lane];
    const u32x4 w1 = st[2 * lane + 1];
    if (b >= nblocks) return;
    u32x2 codes;
    uint32_t s;
    quantize_one<RULE>(w0, w1, g, &codes, &s);
    *reinterpret_cast<u32x2 *>(q + b * 8) = codes;
    sf[b] = static_cast<uint8_t>(s);
}

// ---------------------------------------------------------------- tensor amax
// Global scale of each of `groups` tensors of `per_group` bf16 elements, as
// the bridge page's weight quantiser computes it (section "Quantization"):
// g = max(max |T|, 1e-8) / (6 * 448) in fp32.  Pass 1: workgroup j of group
// e reads every kAmaxGroups-th 16-byte chunk of the group's tensor and
// writes the largest bf16 magnitude pattern it saw (NaN patterns sort above
// +Inf, so a NaN wins) to part[e][j].  Pass 2: one workgroup per group
// reduces the partials, writes g[e], and g[e] for each of the group's rows
// into the per-row scale array that the quantiser then reads.
constexpr int kAmaxThreads = 256;
constexpr int kAmaxGroups = 64;        // pass-1 workgroups per tensor

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
        const uint32_t t = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, kWave));
        v = t > v ? t : v;
    }
    return v;
}

__global__ __launch_bounds__(kAmaxThreads) void amax_partial(const uint16_t *__restrict__ x,
                                                             int64_t per_group,
                                                             uint32_t *__restrict__ part) {
    __shared__ uint32_t wmax[kAmaxThreads / kWave];
    const int64_t e = blockIdx.x / kAmaxGroups;
    const int64_t j = blockIdx.x % kAmaxGroups;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x + e * per_group);
    const int64_t nchunks = per_group / 8;   // 16-byte chunks (per_group % 16 == 0)
    u16x2 mx = {0, 0};
    for (int64_t i = j * kAmaxThreads + threadIdx.x; i < nchunks; i += kAmaxGroups * kAmaxThreads) {
        const u32x4 w = __builtin_nontemporal_load(src + i);
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
            mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, wd[t] & 0x7FFF7FFFu));
    }
    uint32_t m = mx.x > mx.y ? mx.x : mx.y;
    m = wave_max_u32(m);
    if ((threadIdx.x & (kWave - 1)) == 0) wmax[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t all = 0u;
        for (int w = 0; w < kAmaxThreads / kWave; ++w) all = wmax[w] > all ? wmax[w] : all;
        part[e * kAmaxGroups + j] = all;
    }
}

__global__ __launch_bounds__(kWave) void amax_finalize(const uint32_t *__restrict__ part,
                                                       int64_t rows_per_group,
                                                       float *__restrict__ g_out,
                                                       float *__restrict__ row_scale) {
    const int64_t e = blockIdx.x;
    uint32_t m = 0u;
    for (int j = threadIdx.x; j < kAmaxGroups; j += kWave) {
        const uint32_t v = part[e * kAmaxGroups + j];
        m = v > m ? v : m;
    }
    m = wave_max_u32(m);
    float amax = __uint_as_float(m << 16);
    amax = amax < 1e-8f ? 1e-8f : amax;          // NaN stays NaN
    const float g = amax / 2688.0f;              // 6 * 448, one fp32 division
    if (threadIdx.x == 0) g_out[e] = g;
    for (int64_t r = threadIdx.x; r < rows_per_group; r += kWave) row_scale[e * rows_per_group + r] = g;
}

typedef void (*QuantKernel)(const uint16_t *, const float *, int64_t, uint8_t *, uint8_t *,
                            int64_t, int64_t, const float *, float *, int64_t);

QuantKernel quant_kernel(int rule) {
    switch (rule) {
    case NVFP4_ROUND_HALF_STEP: return quantize_blocks<NVFP4_ROUND_HALF_STEP>;
    case NVFP4_ROUND_NEAREST_EVEN: return quantize_blocks<NVFP4_ROUND_NEAREST_EVEN>;
    default: return quantize_blocks<NVFP4_ROUND_NEAREST_LOWER>;
    }
}

bool misaligned(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) != 0; }

bool overlaps(const void *p, size_t pn, const void *q, size_t qn) {
    if (!p || !q || pn == 0 || qn == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + qn && b < a + pn;
}

constexpr int64_t kMaxBlocks = (int64_t(1) << 31) - 1 - kQuantThreads;

int check_quant(const uint16_t *x, const float *gs, int32_t per_row, const uint8_t *q,
                const uint8_t *sf, int64_t rows, int64_t d, int32_t rule) {
    if (!x || !gs || !q || !sf) return NVFP4_GEMV_ERR_NULL_POINTER;
    if (rule < NVFP4_ROUND_HALF_STEP || rule > NVFP4_ROUND_NEAREST_LOWER || per_row < 0 ||
        per_row > 1)
        return NVFP4_GEMV_ERR_BAD_ARGUMENT;
    if (rows < 1 || d < 16 || d % 16 != 0 || rows > kMaxBlocks || d / 16 > kMaxBlocks / rows)
        return NVFP4_GEMV_ERR_BAD_SHAPE;
    if (misaligned(x, 16) || misaligned(q, 8) || misaligned(gs, 4)) return NVFP4_GEMV_ERR_ALIGNMENT;
    const size_t n = static_cast<size_t>(rows) * static_cast<size_t>(d);
    const size_t gsn = (per_row ? static_cast<size_t>(rows) : 1) * 4;
    const void *outs[2] = {q, sf};
    const size_t outn[2] = {n / 2, n / 16};
    for (int i = 0; i < 2; ++i)
        if (overlaps(outs[i], outn[i], x, n * 2) || overlaps(outs[i], outn[i], gs, gsn))
            return NVFP4_GEMV_ERR_ALIAS;
    if (overlaps(q, n / 2, sf, n / 16)) return NVFP4_GEMV_ERR_ALIAS;
    return NVFP4_GEMV_OK;
}

int launch_quant(const uint16_t *x, const float *gs, int64_t gs_stride, uint8_t *q, uint8_t *sf,
                 int64_t rows, int64_t d, int32_t rule, const float *other, float *alpha,
                 hipStream_t stream) {
    int64_t nblocks = rows * (d / 16), bpr = d / 16;
    const int64_t lanes = nblocks > rows ? nblocks : rows;
    const int64_t groups = (lanes + kQuantThreads - 1) / kQuantThreads;
    void *args[] = {&x, &gs, &gs_stride, &q, &sf, &nblocks, &bpr, &other, &alpha, &rows};
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void *>(quant_kernel(rule)),
                        dim3(static_cast<uint32_t>(groups)), dim3(kQuantThreads), args, 0, stream);
    return e == hipSuccess ? NVFP4_GEMV_OK : NVFP4_GEMV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int nvfp4_quantize_activation(const uint16_t *x_bf16, const float *global_scale,
                              int32_t scale_per_row, uint8_t *x_packed, uint8_t *sf, int64_t rows,
                              int64_t d, int32_t rule, void *stream) {
    const int s = check_quant(x_bf16, global_scale, scale_per_row, x_packed, sf, rows, d, rule);
    if (s != NVFP4_GEMV_OK) return s;
    return launch_quant(x_bf16, global_scale, scale_per_row, x_packed, sf, rows, d, rule, nullptr,
                        nullptr, static_cast<hipStream_t>(stream));
}

int nvfp4_gemv_bf16x_launch(const uint8_t *A_packed, const uint8_t *sfA, const float *A_scale,
                            const uint16_t *x_bf16, const float *x_scale, int32_t rule,
                            uint8_t *x_packed, uint8_t *sfx, float *alpha, uint16_t *c,
                            int64_t l, int64_t m, int64_t k, void *stream) {
    if (!A_packed || !sfA || !alpha || !c) return NVFP4_GEMV_ERR_NULL_POINTER;
    int s = check_quant(x_bf16, x_scale, 1, x_packed, sfx, l, k, rule);
    if (s != NVFP4_GEMV_OK) return s;
    nvfp4_gemv_tuning_t plan;
    size_t ws = 0;
    s = nvfp4_gemv_plan(l, m, k, 1, nullptr, &plan, &ws);
    if (s != NVFP4_GEMV_OK) return s;
    if (misaligned(c, 2) || misaligned(alpha, 4) || misaligned(A_scale, 4))
        return NVFP4_GEMV_ERR_ALIGNMENT;
    // every output against every input and against each other
    const size_t lm = static_cast<size_t>(l) * static_cast<size_t>(m);
    const size_t lk = static_cast<size_t>(l) * static_cast<size_t>(k);
    const void *in[5] = {A_packed, sfA, A_scale, x_bf16, x_scale};
    const size_t inn[5] = {lm * static_cast<size_t>(k / 2), lm * static_cast<size_t>(k / 16),
                           A_scale ? static_cast<size_t>(l) * 4 : 0, lk * 2,
                           static_cast<size_t>(l) * 4};
    const void *out[4] = {x_packed, sfx, alpha, c};
    const size_t outn[4] = {lk / 2, lk / 16, static_cast<size_t>(l) * 4, lm * 2};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(out[i], outn[i], in[j], inn[j])) return NVFP4_GEMV_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlaps(out[i], outn[i], out[j], outn[j])) return NVFP4_GEMV_ERR_ALIAS;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    s = launch_quant(x_bf16, x_scale, 1, x_packed, sfx, l, k, rule, A_scale, alpha, st);
    if (s != NVFP4_GEMV_OK) return s;
    return nvfp4_gemv_launch(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k, stream);
}

int nvfp4_quantize_weight(const uint16_t *w_bf16, int64_t groups, int64_t rows, int64_t d,
                          int32_t rule, uint8_t *w_packed, uint8_t *sf, float *global_scale,
                          void *stream) {
    if (!global_scale) return NVFP4_GEMV_ERR_NULL_POINTER;
    if (groups < 1 || rows < 1 || groups > kMaxBlocks / rows) return NVFP4_GEMV_ERR_BAD_SHAPE;
    const int64_t total_rows = groups * rows;
    // shape, rule, alignment of x / packed output and the aliasing of the
    // outputs with the input are the quantiser's rules over all rows
    int s = check_quant(w_bf16, global_scale, 0, w_packed, sf, total_rows, d, rule);
    if (s != NVFP4_GEMV_OK) return s;
    if (misaligned(global_scale, 4)) return NVFP4_GEMV_ERR_ALIGNMENT;
    const size_t n = static_cast<size_t>(total_rows) * static_cast<size_t>(d);
    const size_t gn = static_cast<size_t>(groups) * 4;
    if (overlaps(global_scale, gn, w_bf16, n * 2) || overlaps(global_scale, gn, w_packed, n / 2) ||
        overlaps(global_scale, gn, sf, n / 16))
        return NVFP4_GEMV_ERR_ALIAS;
    if (groups > (int64_t(1) << 31) / kAmaxGroups) return NVFP4_GEMV_ERR_BAD_SHAPE;
    // workspace: the pass-1 partials, then one fp32 scale per row
    const size_t part_bytes = static_cast<size_t>(groups) * kAmaxGroups * sizeof(uint32_t);
    const size_t ws_bytes = part_bytes + static_cast<size_t>(total_rows) * sizeof(float);
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return NVFP4_GEMV_ERR_DEVICE;
    uint8_t *ws = static_cast<uint8_t *>(nvfp4_stream_workspace(dev, stream, ws_bytes));
    if (!ws) return NVFP4_GEMV_ERR_WORKSPACE;
    uint32_t *part = reinterpret_cast<uint32_t *>(ws);
    float *row_scale = reinterpret_cast<float *>(ws + part_bytes);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    int64_t per_group = rows * d;
    void *a1[] = {&w_bf16, &per_group, &part};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(amax_partial),
                                   dim3(static_cast<uint32_t>(groups * kAmaxGroups)),
                                   dim3(kAmaxThreads), a1, 0, st);
    if (e != hipSuccess) return NVFP4_GEMV_ERR_LAUNCH;
    const uint32_t *cpart = part;
    int64_t rpg = rows;
    void *a2[] = {&cpart, &rpg, &global_scale, &row_scale};
    e = hipLaunchKernel(reinterpret_cast<const void *>(amax_finalize),
                        dim3(static_cast<uint32_t>(groups)), dim3(kWave), a2, 0, st);
    if (e != hipSuccess) return NVFP4_GEMV_ERR_LAUNCH;
    return launch_quant(w_bf16, row_scale, 1, w_packed, sf, total_rows, d, rule, nullptr, nullptr, st);
}

}  // extern "C"
