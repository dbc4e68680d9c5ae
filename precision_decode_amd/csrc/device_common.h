// Device helpers shared by the HIP sources of the NVFP4 library (gfx950).
//
// Formats (the NVFP4 layout of "nvFP4 Batch GEMV算子系列(下)", section "NVFP4
// Batched GEMV 概念阐述", with the E2M1 magnitudes of the CuTeDSL bridge page's
// constants): E2M1 codes are packed two per byte, element 2i in bits 3:0 and
// element 2i+1 in bits 7:4, bit 3 of a code is the sign; block scales are OCP
// float8_e4m3fn codes, one per 16 consecutive elements.
//
// Not part of the C ABI.
#ifndef NVFP4_DEVICE_COMMON_H
#define NVFP4_DEVICE_COMMON_H

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace nvfp4dev {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Two E2M1 codes (byte SEL of w) -> two fp16, exact.  The scale operand of the
// gfx950 conversion is a power of two carried in a float; 1.0 leaves values
// unscaled.
template <int SEL>
__device__ __forceinline__ f16x2 e2m1x2_f16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// Two E4M3 codes (bytes 0 and 1 of w) -> two fp32, exact.
__device__ __forceinline__ f32x2 e4m3x2_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
}

// Two E4M3 codes (bytes 0 and 1 of w) -> two fp16.  Exact: E4M3 values are
// 2^-9 .. 448 with 4 significant bits, all normal fp16 numbers; NaN stays NaN.
__device__ __forceinline__ f16x2 e4m3x2_f16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
}

__device__ __forceinline__ uint32_t bits(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ f16x2 halves(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

// fp16 bits of f16(f32(al * v)): the product is rounded to fp32 first.  The
// empty asm keeps that rounding: without it the compiler folds the multiply
// and the conversion into one mixed-precision FMA that rounds only once, to
// fp16, which differs on a few outputs.
__device__ __forceinline__ uint16_t f16_of_product(float al, float v) {
    float p = al * v;
    __asm__ volatile("" : "+v"(p));
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(p));
}

// bf16 bits of a float by IEEE round-to-nearest-even on the bit pattern
// (overflow rounds to infinity); NaN gives a quiet NaN of the same sign.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// bf16 bits of bf16(f32(al * v)).
__device__ __forceinline__ uint16_t bf16_of_product(float al, float v) {
    float p = al * v;
    __asm__ volatile("" : "+v"(p));
    return bf16_rne(p);
}

// Word 3 of a buffer descriptor: 32-bit data format, untyped (raw) access.
constexpr int kRawBufferFlags = 0x00020000;
// Cache-policy operand of a buffer load: non-temporal (streamed, read once).
constexpr int kNonTemporal = 2;
// A buffer offset past any descriptor's range: the load returns zeros and
// touches no memory.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Raw buffer descriptor over [base, base + bytes).  Loads at offsets whose
// access reaches past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const uint8_t *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), 0, bytes, kRawBufferFlags);
}

// Keeps the compiler's scheduler from moving any instruction across this
// point (kernels rely on issue order for the load counters).
__device__ __forceinline__ void phase_fence() { __builtin_amdgcn_sched_barrier(0); }

// Sum over the 64 lanes, the same value in every lane, without LDS: DPP
// exchanges inside 16-lane rows (neighbour, pair, mirror of 8, mirror of 16),
// then swaps of 16-lane rows and of 32-lane halves.  Each step adds two values
// that every lane of a pair adds in the same order, so all lanes agree bit
// for bit.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL,
                                                              0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __builtin_bit_cast(float, static_cast<unsigned>(r16[0])) +
        __builtin_bit_cast(float, static_cast<unsigned>(r16[1]));
    const unsigned w = __builtin_bit_cast(unsigned, v);
    const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
    return __builtin_bit_cast(float, static_cast<unsigned>(r32[0])) +
           __builtin_bit_cast(float, static_cast<unsigned>(r32[1]));
}

}  // namespace nvfp4dev

// Library-owned workspace, one per (device, stream), grown on demand and kept
// until the process ends (defined in nvfp4_gemv.hip).  Returns NULL when the
// slot must grow and cannot: allocation failed, or the stream is being
// captured into a graph.  Never synchronises and never frees a buffer that
// enqueued work may still read.
__attribute__((visibility("hidden"))) void *nvfp4_stream_workspace(int dev, void *stream,
                                                                    size_t need);

#endif  // NVFP4_DEVICE_COMMON_H
