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
// that is a multiple of 16 keeps the wave's loads and stores contiguous.  Divisions by the global and block scales use one
// reciprocal per block and fused residual corrections, which round exactly as
// IEEE division does in the range the kernel checks for; the E2M1 rounding
// uses gfx950's FP4 conversion where a rule allows.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "nvfp4_gemv.h"
#include "nvfp4_quantize.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQuantThreads = 256;

// The page's half-step table (doubled, rounded magnitude 0..12 -> E2M1 index),
// four bits per entry.
constexpr uint64_t half_step_table() {
    constexpr uint8_t t[13] = {0, 1, 2, 3, 4, 4, 5, 5, 6, 6, 6, 7, 7};
    uint64_t r = 0;
    for (int i = 0; i < 13; ++i) r |= static_cast<uint64_t>(t[i]) << (4 * i);
    return r;
}
constexpr uint64_t kHalfStep = half_step_table();

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> E4M3 (float8_e4m3fn) code for v > 0, or NaN / +Inf: round to
// nearest even; values from 464 up (halfway to the first step past 448, whose
// pattern is NaN), infinities and NaN give 0x7F.
__device__ __forceinline__ uint32_t e4m3_code_pos(float v) {
    if (!(v <= 464.0f)) return 0x7Fu;
    if (v < 0.015625f) {                         // below 2^-6: subnormal steps of 2^-9
        return static_cast<uint32_t>(__builtin_rintf(v * 512.0f));   // exact scaling, 0..8
    }
    // normal: keep 3 mantissa bits with round-to-nearest-even on the fp32 pattern
    const uint32_t b = __float_as_uint(v);
    const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;     // (exp << 3 | mant), rounded
    return r - (120u << 3);                       // rebias 127 -> 7
}

// E4M3 code (0..0x7F, sign clear) -> float; 0x7F is NaN.
__device__ __forceinline__ float e4m3_value_pos(uint32_t s) {
    if (s == 0x7Fu) return __uint_as_float(0x7FC00000u);
    if (s < 8u) return static_cast<float>(s) * 0.001953125f;          // s * 2^-9, exact
    return __uint_as_float((((s >> 3) + 120u) << 23) | ((s & 7u) << 20));
}

template <int RULE>
__device__ __forceinline__ uint32_t e2m1_index(float v) {
    float a = __builtin_fabsf(v);
    if (a != a) a = 0.0f;                          // NaN -> index 0
    if constexpr (RULE == NVFP4_ROUND_HALF_STEP) {
        const float h = __builtin_rintf((a < 6.0f ? a : 6.0f) * 2.0f);   // 0..12, exact
        const uint32_t hi = static_cast<uint32_t>(h);
        return static_cast<uint32_t>(kHalfStep >> (4 * hi)) & 7u;
    } else if constexpr (RULE == NVFP4_ROUND_NEAREST_EVEN) {
        // count the midpoints below a; on a midpoint take the even neighbour
        return static_cast<uint32_t>(a > 0.25f) + static_cast<uint32_t>(a >= 0.75f) +
               static_cast<uint32_t>(a > 1.25f) + static_cast<uint32_t>(a >= 1.75f) +
               static_cast<uint32_t>(a > 2.5f) + static_cast<uint32_t>(a >= 3.5f) +
               static_cast<uint32_t>(a > 5.0f);
    } else {
        // argmin over fp32 distances, first index on ties
        constexpr float g[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
        uint32_t best = 0;
        float bd = a;
#pragma unroll
        for (int j = 1; j < 8; ++j) {
            const float d = __builtin_fabsf(a - g[j]);
            if (d < bd) {
                bd = d;
                best = static_cast<uint32_t>(j);
            }
        }
        return best;
    }
}

// a / b rounded to nearest even, given y = RN(1/b): q = a*y, then two
// residual corrections q += (a - b*q)*y with exact fused residuals.  After the
// first correction q is within an ulp of a/b, so the second one rounds
// correctly (Markstein's theorem for round-to-nearest).  The caller keeps b,
// 1/b and the quotient inside the normal range (see `fast` below); a zero
// quotient comes out as +0.
__device__ __forceinline__ float div_rn(float a, float b, float y) {
    float q = a * y;
    float e = __builtin_fmaf(-b, q, a);
    q = __builtin_fmaf(e, y, q);
    e = __builtin_fmaf(-b, q, a);
    return __builtin_fmaf(e, y, q);
}

// Codes of 16 values v[i] (element i at nibble i of the 64-bit result) under
// the rule, sign bit 8 for v < 0, NaN -> 0.
//  * nearest-even: the gfx950 FP4 conversion rounds to nearest even on the
//    E2M1 grid and saturates at 6, with the sign of v; only -0 (code 8, not 0)
//    and NaN differ from the rule, and the caller removes both;
//  * nearest-lower (argmin of fp32 distances, first on ties): the same
//    conversion, one step down at the three ties whose even neighbour is the
//    upper one (0.75, 1.75, 3.5).  For |v| <= 2^20, which every block here
//    satisfies (|v| <= 6.25, or < 6e5 when the block scale rounds to zero),
//    the fp32 distances are exact near every tie, so the argmin is the nearest
//    value with ties down, and 6 beyond the grid;
//  * half-step: the page's table on rint(2 min(|v|, 6)).
template <int RULE>
__device__ __forceinline__ u32x2 block_codes(const float (&v)[16]) {
    u32x2 out;
    if constexpr (RULE == NVFP4_ROUND_HALF_STEP) {
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t code = e2m1_index<RULE>(v[i]) | (v[i] < 0.0f ? 8u : 0u);
            packed[i >> 3] |= code << (4 * (i & 7));
        }
        out.x = packed[0];
        out.y = packed[1];
    } else {
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            w[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j], v[8 * j + 0], v[8 * j + 1], 1.0f, 0);
            w[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j], v[8 * j + 2], v[8 * j + 3], 1.0f, 1);
            w[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j], v[8 * j + 4], v[8 * j + 5], 1.0f, 2);
            w[j] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[j], v[8 * j + 6], v[8 * j + 7], 1.0f, 3);
        }
        if constexpr (RULE == NVFP4_ROUND_NEAREST_LOWER) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float a = __builtin_fabsf(v[i]);
                const bool down = a == 0.75f || a == 1.75f || a == 3.5f;
                w[i >> 3] -= down ? (1u << (4 * (i & 7))) : 0u;   // index >= 2 there: no borrow
            }
        }
        out.x = w[0];
        out.y = w[1];
    }
    return out;
}

// One 16-element block: bf16 words w0, w1 (elements 2i, 2i+1 in word i) with
// global scale g -> 8 bytes of codes and the E4M3 scale code.
//
// Fast path: with the global scale in [2^-40, 2^30] and every nonzero input
// at least 2^-100 in magnitude, x/g and xn/den stay inside the range where
// div_rn rounds correctly (a tiny quotient's exact value never changes its
// code: only its sign counts there), so both divisions take one reciprocal
// per block and five fused operations per element.  Other blocks (rare: a
// subnormal input, an extreme or non-finite scale) take IEEE divisions.
template <int RULE>
__device__ __forceinline__ void quantize_one(u32x4 w0, u32x4 w1, float g, u32x2 *codes,
                                             uint32_t *scale) {
    const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    // smallest nonzero magnitude pattern (bf16 bits - 1, zero wraps to the top)
    uint32_t tiny = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t lo = (w[i] & 0x7FFFu) - 1u, hi = ((w[i] >> 16) & 0x7FFFu) - 1u;
        tiny = lo < tiny ? lo : tiny;
        tiny = hi < tiny ? hi : tiny;
    }
    const bool fast = g >= 0x1p-40f && g <= 0x1p30f && tiny >= (27u << 7) - 1u;   // 2^-100

    float xn[16];
    if (fast) {
        const float yg = 1.0f / g;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xn[2 * i] = div_rn(bf16_to_f32(w[i] & 0xFFFFu), g, yg);
            xn[2 * i + 1] = div_rn(bf16_to_f32(w[i] >> 16), g, yg);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            xn[2 * i] = bf16_to_f32(w[i] & 0xFFFFu) / g;
            xn[2 * i + 1] = bf16_to_f32(w[i] >> 16) / g;
        }
    }
    // max |xn| on the bit patterns: NaN patterns sort above +Inf, so a NaN wins
    uint32_t amb = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t a = __float_as_uint(xn[i]) & 0x7FFFFFFFu;
        amb = a > amb ? a : amb;
    }
    float am = __uint_as_float(amb);
    am = am < 1e-8f ? 1e-8f : am;                  // NaN stays NaN
    const uint32_t s = e4m3_code_pos(am / 6.0f);
    const float sv = e4m3_value_pos(s);
    const float den = sv < 1e-8f ? 1e-8f : sv;     // NaN stays NaN

    float v[16];
    if (fast) {
        const float yd = 1.0f / den;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = div_rn(xn[i], den, yd);
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
// (block b is block b % bpr of row b / bpr).  `x` 16-byte aligned, `q` 8-byte
// aligned; gs_stride 0 (one scale) or 1 (one scale per row).  Lanes below
// `rows` also write alpha[row] = f32(other[row] * gs[row]) (or gs[row] when
// `other` is NULL) when `alpha` is not NULL.
template <int RULE>
__global__ __launch_bounds__(kQuantThreads) void quantize_blocks(
    const uint16_t *__restrict__ x, const float *__restrict__ gs, int64_t gs_stride,
    uint8_t *__restrict__ q, uint8_t *__restrict__ sf, int64_t nblocks, int64_t bpr,
    const float *__restrict__ other, float *__restrict__ alpha, int64_t rows) {
    const int64_t b = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x;
    if (alpha != nullptr && b < rows) {
        const float g = gs[b * gs_stride];
        alpha[b] = other != nullptr ? other[b] * g : g;
    }
    if (b >= nblocks) return;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(x) + 2 * b;
    const u32x4 w0 = __builtin_nontemporal_load(src);
    const u32x4 w1 = __builtin_nontemporal_load(src + 1);
    // block numbers stay below 2^31 (checked on the host): a 32-bit division
    const uint32_t row = static_cast<uint32_t>(b) / static_cast<uint32_t>(bpr);
    u32x2 codes;
    uint32_t s;
    quantize_one<RULE>(w0, w1, gs[row * gs_stride], &codes, &s);
    *reinterpret_cast<u32x2 *>(q + b * 8) = codes;
    sf[b] = static_cast<uint8_t>(s);
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

}  // extern "C"
