// Device check of the quantiser's division-free quotients (quant_arith.h)
// against IEEE division, over the whole range in which the quantiser's fast
// path relies on them:
//  1. recip_f64(g) against RN64(1 / g) for every fp32 g in [2^-40, 2^30];
//  2. quot_f64(x, recip_f64(g)) against RN32(x / g) for every bf16 significand
//     of x against every fp32 significand of g, both signs (exponents only
//     shift a normal quotient), and quot_f64(am, RN64(1/6)) against RN32(am / 6)
//     for every fp32 significand of am;
//  3. quot_short(x, s, rcp(s)) against RN32(x / s) for every nonzero E4M3
//     scale value s and every fp32 x with x / s in [1/8, 8), where the E2M1
//     codes are decided.
// Prints one line per check and "quant_arith_check ok" when nothing differs;
// the exit status is 0 then, 3 on a difference, 1 on a HIP error.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "quant_arith.h"

using namespace nvfp4quant;

namespace {

__global__ void check_recip(uint32_t lo, uint32_t n, unsigned long long *bad) {
    const uint32_t stride = gridDim.x * blockDim.x;
    unsigned long long nb = 0;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const double d = static_cast<double>(__uint_as_float(lo + i));
        if (__double_as_longlong(recip_f64(d)) != __double_as_longlong(1.0 / d)) ++nb;
    }
    if (nb) atomicAdd(bad, nb);
}

__global__ void check_xg(unsigned long long *bad) {
    const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;   // fp32 significand of g (and of am)
    if (t >= (1u << 23)) return;
    const float g = __uint_as_float(0x3F800000u | t);
    const double yg = recip_f64(static_cast<double>(g));
    unsigned long long nb = 0;
    for (uint32_t sx = 0; sx < 128; ++sx) {
        const float x = bf16_to_f32(0x3F80u | sx);
        if (__float_as_uint(quot_f64(x, yg)) != __float_as_uint(x / g)) ++nb;
        if (__float_as_uint(quot_f64(-x, yg)) != __float_as_uint(-x / g)) ++nb;
    }
    if (__float_as_uint(quot_f64(g, 1.0 / 6.0)) != __float_as_uint(g / 6.0f)) ++nb;
    if (nb) atomicAdd(bad, nb);
}

__global__ void check_short(uint32_t code, uint32_t lo, uint32_t n, unsigned long long *bad) {
    const float den = e4m3_value_pos(code);
    const float yd = __builtin_amdgcn_rcpf(den);
    const uint32_t stride = gridDim.x * blockDim.x;
    unsigned long long nb = 0;
    for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = __uint_as_float(lo + i);
        if (__float_as_uint(quot_short(x, den, yd)) != __float_as_uint(x / den)) ++nb;
    }
    if (nb) atomicAdd(bad, nb);
}

float e4m3_host(uint32_t code) {
    if (code < 8) return static_cast<float>(code) * 0.001953125f;
    const uint32_t b = (((code >> 3) + 120u) << 23) | ((code & 7u) << 20);
    float v;
    std::memcpy(&v, &b, 4);
    return v;
}

uint32_t bits_of(float v) {
    uint32_t b;
    std::memcpy(&b, &v, 4);
    return b;
}

}  // namespace

int main() {
    unsigned long long *d = nullptr;
    if (hipMalloc(&d, 3 * sizeof(unsigned long long)) != hipSuccess) return 1;
    if (hipMemset(d, 0, 3 * sizeof(unsigned long long)) != hipSuccess) return 1;

    const uint32_t rlo = bits_of(0x1p-40f), rhi = bits_of(0x1p30f);
    const unsigned long long n_recip = rhi - rlo + 1ull;
    hipLaunchKernelGGL(check_recip, dim3(4096), dim3(256), 0, 0, rlo, rhi - rlo + 1u, d);
    hipLaunchKernelGGL(check_xg, dim3((1u << 23) / 256), dim3(256), 0, 0, d + 1);
    const unsigned long long n_xg = 2ull * 128ull * (1ull << 23) + (1ull << 23);
    unsigned long long n_short = 0;
    for (uint32_t code = 1; code <= 0x7E; ++code) {
        const float den = e4m3_host(code);
        const uint32_t lo = bits_of(den * 0.125f), hi = bits_of(den * 8.0f);   // exact scalings
        n_short += hi - lo;
        hipLaunchKernelGGL(check_short, dim3(2048), dim3(256), 0, 0, code, lo, hi - lo, d + 2);
    }
    if (hipGetLastError() != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
        std::printf("HIP error\n");
        return 1;
    }
    unsigned long long h[3] = {0, 0, 0};
    if (hipMemcpy(h, d, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return 1;
    (void)hipFree(d);
    std::printf("recip_f64: %llu fp32 g in [2^-40, 2^30], %llu differ from RN64(1/g)\n", n_recip, h[0]);
    std::printf("quot_f64: %llu quotients x/g and am/6, %llu differ from IEEE division\n", n_xg, h[1]);
    std::printf("quot_short: %llu quotients x/s over the 126 nonzero E4M3 scales, %llu differ\n", n_short, h[2]);
    if (h[0] || h[1] || h[2]) return 3;
    std::printf("quant_arith_check ok\n");
    return 0;
}
