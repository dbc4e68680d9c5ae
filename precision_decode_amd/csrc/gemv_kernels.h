// NVFP4 block-scaled batched GEMV for MI355X (gfx950, CDNA4).
//
//   c[b,r] = f16( f32( alpha[b] * sum_kk e2m1(A[b,r,kk]) e4m3(sfA[b,r,kk/16])
//                                      * e2m1(x[b,kk])   e4m3(sfx[b,kk/16]) ) )
//
// The operation is the NVFP4 batched GEMV of "nvFP4 Batch GEMV算子系列(下)"
// (section "NVFP4 Batched GEMV 概念阐述"): blocks of 16 K-elements share an FP8
// E4M3 scale, E2M1 elements are packed two per byte with the even element in
// the low nibble (as the CuTeDSL bridge page's quantisers pack them).
//
// A GEMV reads every weight byte once and does 2 flops per 9/16 byte, so the
// kernel is bound by HBM bandwidth, not by compute; it uses no MFMA.  Design:
//
//  * the workgroup first decodes its K-range of x into x~ = e2m1(x) * e4m3(sfx)
//    as fp16 in LDS (exact: 2 + 4 significant bits, |x~| <= 2688, smallest
//    nonzero 2^-10 is a normal fp16), laid out so that each lane's reads are
//    consecutive across lanes (no bank conflicts);
//  * each wave streams R rows at once, lanes along K: one 16-byte
//    non-temporal load per lane per row covers 32 elements (two scale blocks),
//    a wave instruction reads 1 KiB of one row; U such iterations are kept in
//    flight per row;
//  * A is decoded with gfx950's packed E2M1 -> fp16 conversion (2 elements
//    per instruction, exact), multiplied by x~ with v_dot2_f32_f16 (2 products
//    per instruction, fp32 accumulate), each 16-element block sum is scaled by
//    its E4M3 sfA once (fp32 FMA);
//  * lane partial sums are reduced across the wave; the epilogue is one fp32
//    multiply by alpha and one fp32 -> fp16 round-to-nearest-even conversion;
//  * when there are too few rows to fill the GPU, or K is longer than one
//    workgroup's LDS staging, K is split across workgroups: they write fp32
//    partial sums to a workspace and a second kernel adds them in split order.
//
// Every accumulator starts at +0.0, so an exactly-zero result is +0.  With the
// integer-coded inputs (E2M1 values times scales 0, 1, 2) every partial sum is
// a multiple of 1/4 below 2^22 and therefore exact in fp32, whatever the
// summation order.
//
// This header holds the GEMV's device code (kernels and their helpers); the
// read probes are in probe_kernels.h, and the host side (plans, entry points,
// workspaces) is nvfp4_gemv.hip, the only includer of both.
#ifndef NVFP4_GEMV_KERNELS_H
#define NVFP4_GEMV_KERNELS_H

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "device_common.h"
#include "gemv_plan.h"

namespace {

using namespace nvfp4dev;
using namespace nvfp4plan;

// ---------------------------------------------------------------- decode
// acc + sum over the 8 codes of `a` of e2m1(code) * x~ (8 fp16 in xq).
__device__ __forceinline__ float dot8(uint32_t a, u32x4 xq, float acc) {
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<0>(a), halves(xq.x), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<1>(a), halves(xq.y), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<2>(a), halves(xq.z), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<3>(a), halves(xq.w), acc, false);
    return acc;
}

// One lane's 32 elements (two scale blocks): 16 bytes of A, their two sfA
// codes in the low half of s2, and x~ for the same 32 positions.
__device__ __forceinline__ float chunk32(u32x4 a, uint32_t s2, const u32x4 (&xq)[4], float acc) {
    float b0 = dot8(a.x, xq[0], 0.0f);
    b0 = dot8(a.y, xq[1], b0);
    float b1 = dot8(a.z, xq[2], 0.0f);
    b1 = dot8(a.w, xq[3], b1);
    const f32x2 s = e4m3x2_f32(s2);
    acc = __builtin_fmaf(b0, s.x, acc);
    acc = __builtin_fmaf(b1, s.y, acc);
    return acc;
}

// x~ for 32 elements: 16 bytes of x and their two sfx codes -> 32 fp16.
__device__ __forceinline__ void decode_x32(u32x4 xv, uint32_t s2, u32x4 (&out)[4]) {
    const f32x2 s = e4m3x2_f32(s2);
    const _Float16 h0 = static_cast<_Float16>(s.x);
    const _Float16 h1 = static_cast<_Float16>(s.y);
    const f16x2 v0 = {h0, h0};
    const f16x2 v1 = {h1, h1};
    out[0] = u32x4{bits(e2m1x2_f16<0>(xv.x) * v0), bits(e2m1x2_f16<1>(xv.x) * v0),
                   bits(e2m1x2_f16<2>(xv.x) * v0), bits(e2m1x2_f16<3>(xv.x) * v0)};
    out[1] = u32x4{bits(e2m1x2_f16<0>(xv.y) * v0), bits(e2m1x2_f16<1>(xv.y) * v0),
                   bits(e2m1x2_f16<2>(xv.y) * v0), bits(e2m1x2_f16<3>(xv.y) * v0)};
    out[2] = u32x4{bits(e2m1x2_f16<0>(xv.z) * v1), bits(e2m1x2_f16<1>(xv.z) * v1),
                   bits(e2m1x2_f16<2>(xv.z) * v1), bits(e2m1x2_f16<3>(xv.z) * v1)};
    out[3] = u32x4{bits(e2m1x2_f16<0>(xv.w) * v1), bits(e2m1x2_f16<1>(xv.w) * v1),
                   bits(e2m1x2_f16<2>(xv.w) * v1), bits(e2m1x2_f16<3>(xv.w) * v1)};
}

// (row block, batch, split) of this workgroup, row block fastest.  The plan
// keeps the workgroup count below 2^31, so 32-bit division suffices (much
// shorter than 64-bit division, which every workgroup would run first).
__device__ __forceinline__ void group_index(int64_t row_blocks, int64_t l, int64_t *rb,
                                            int64_t *b, int64_t *split) {
    const uint32_t g = blockIdx.x;
    const uint32_t rbs = static_cast<uint32_t>(row_blocks), ls = static_cast<uint32_t>(l);
    const uint32_t q = g / rbs;
    *rb = g - q * rbs;
    *b = q % ls;
    *split = q / ls;
}

// ---------------------------------------------------------------- fast kernel
// Workgroup = W waves; wave w streams rows rb*W*R + w*R .. +R-1 of batch b over
// the K-range [split*kchunk, min(k, (split+1)*kchunk)).  blockIdx.x enumerates
// (split, batch, row block) with the row block fastest.
//
// LDS holds x~ of the K-range: for iteration `it` (2048 elements) and lane i,
// the 32 fp16 of elements it*2048 + 32*i .. +31 sit in four 16-byte slots
// xs[(it*4 + j)*64 + i], j = 0..3, so a wave's reads of slot j are 1 KiB
// contiguous.  The iteration count is rounded up to a multiple of U and the
// slots past the end of K hold zeros.
//
// All global reads are buffer loads through a descriptor that covers exactly
// one row's K-range (or x's): a lane whose offset lies past the end gets
// zeros from the hardware range check (E2M1 code 0, E4M3 code 0), which
// contributes +0.  So no load sits under a per-lane branch, the compiler can
// count outstanding loads, and U iterations of every row stay in flight.
constexpr int kMaxIters = static_cast<int>(kMaxChunk / kIterElems);   // 8

// Makes a loaded value available here, so its load cannot be sunk into a
// later branch.
__device__ __forceinline__ void keep(u32x4 v) {
    __asm__ volatile("" ::"v"(v.x), "v"(v.y), "v"(v.z), "v"(v.w));
}
__device__ __forceinline__ void keep(uint16_t v) { __asm__ volatile("" ::"v"(v)); }

template <int R, int U, int W>
__global__ void __launch_bounds__(W * kWave)
gemv_fast(const uint8_t *__restrict__ A, const uint8_t *__restrict__ sfA,
          const uint8_t *__restrict__ x, const uint8_t *__restrict__ sfx,
          const float *__restrict__ alpha, uint16_t *__restrict__ c,
          float *__restrict__ part, int64_t l, int64_t m, int64_t k,
          int64_t kchunk, int64_t row_blocks) {
    static_assert(kMaxIters % U == 0, "U must divide the staged iteration count");
    constexpr int kXPerThread = (kMaxIters + W - 1) / W;   // x chunks of 32 elements per thread
    extern __shared__ u32x4 xs[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

    int64_t rb, b, split;
    group_index(row_blocks, l, &rb, &b, &split);

    const int64_t kb0 = split * kchunk;
    const int klen = static_cast<int>((k - kb0 < kchunk) ? (k - kb0) : kchunk);
    const int nit = (klen + static_cast<int>(kIterElems) - 1) / static_cast<int>(kIterElems);
    const int nstage = (nit + U - 1) / U;
    const int nslot = nstage * U;
    const int64_t row0 = rb * (W * R) + wave * R;

    // x and its scales for the K-range, issued before the A stream.
    const __amdgpu_buffer_rsrc_t xbuf = buffer_of(x + b * (k / 2) + kb0 / 2, klen / 2);
    const __amdgpu_buffer_rsrc_t sxbuf = buffer_of(sfx + b * (k / 16) + kb0 / 16, klen / 16);
    u32x4 xv[kXPerThread];
    uint16_t xs2[kXPerThread];
#pragma unroll
    for (int i = 0; i < kXPerThread; ++i) {
        const int q = tid + i * W * kWave;
        xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xbuf, 16 * q, 0, 0));
        xs2[i] = __builtin_amdgcn_raw_buffer_load_b16(sxbuf, 2 * q, 0, 0);
    }

    __amdgpu_buffer_rsrc_t abuf_rs[R], sbuf_rs[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = (row0 + r < m) ? row0 + r : m - 1;   // rows past m: read row m-1, never written
        abuf_rs[r] = buffer_of(A + (b * m + row) * (k / 2) + kb0 / 2, klen / 2);
        sbuf_rs[r] = buffer_of(sfA + (b * m + row) * (k / 16) + kb0 / 16, klen / 16);
    }

    u32x4 abuf[U][R];
    uint16_t sbuf[U][R];   // widened only where used, so no instruction touches it early
    auto issue = [&](int it, int u) {
        const int off = it * static_cast<int>(kIterElems / 2) + lane * 16;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            abuf[u][r] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(abuf_rs[r], off, 0, kNonTemporal));
            sbuf[u][r] = __builtin_amdgcn_raw_buffer_load_b16(sbuf_rs[r], off / 8, 0, kNonTemporal);
        }
    };
    auto consume = [&](int it, int u, float (&acc)[R]) {
        u32x4 xq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xq[j] = xs[(it * 4 + j) * kWave + lane];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = chunk32(abuf[u][r], sbuf[u][r], xq, acc[r]);
    };

    phase_fence();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        issue(u, u);
        phase_fence();   // same issue order as the refills in the loop below
    }

    // Decode the x chunks (waiting only for the x loads, which were issued
    // first) and store the slots that exist.
#pragma unroll
    for (int i = 0; i < kXPerThread; ++i) {
        keep(xv[i]);
        keep(xs2[i]);
    }
#pragma unroll
    for (int i = 0; i < kXPerThread; ++i) {
        const int q = tid + i * W * kWave;
        u32x4 out[4];
        decode_x32(xv[i], xs2[i], out);
        if (q < nslot * kWave) {
            const int it = q / kWave, li = q % kWave;
#pragma unroll
            for (int j = 0; j < 4; ++j) xs[(it * 4 + j) * kWave + li] = out[j];
        }
    }
    __syncthreads();
    phase_fence();

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;

    for (int st = 0; st + 1 < nstage; ++st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int it = st * U + u;
            consume(it, u, acc);
            issue(it + U, u);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int it = (nstage - 1) * U + u;
        if (it < nit) consume(it, u, acc);   // wave-uniform: skip iterations past K
    }

    float sum[R];
#pragma unroll
    for (int r = 0; r < R; ++r) sum[r] = wave_sum(acc[r]);

    if (lane < R) {
        float v = sum[0];
#pragma unroll
        for (int r = 1; r < R; ++r)
            if (lane == r) v = sum[r];
        const int64_t row = row0 + lane;
        if (row < m) {
            if (part != nullptr) {
                part[(split * l + b) * m + row] = v;
            } else {
                const float al = alpha ? alpha[b] : 1.0f;
                c[b * m + row] = f16_of_product(al, v);
            }
        }
    }
}

// ---------------------------------------------------------------- packed-x fast kernel
// The fast kernel with x staged raw: LDS holds x's packed codes (16 bytes per
// 32 elements) and its scale pairs, about 10 KiB for a 16384-element K-range
// instead of 32 KiB of fp16 x~, so staging is a copy, LDS reads per step are
// 18 bytes per lane instead of 64, and LDS no longer limits how many
// workgroups a compute unit holds.  Each wave decodes x's codes once per step
// for its R rows and applies the combined scale sA*sx once per 16-element
// block: Σ e2m1(a)·e2m1(x) over a block is exact, and sA*sx (4 + 4
// significant bits) is exact, so the fp32 FMA rounds exactly as the fp16-x~
// kernel does and the results are bit-identical.
//
// One lane's 32 elements: block sums of raw E2M1 products, then the scales.
__device__ __forceinline__ float dot8_raw(uint32_t a, uint32_t xw, float acc) {
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<0>(a), e2m1x2_f16<0>(xw), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<1>(a), e2m1x2_f16<1>(xw), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<2>(a), e2m1x2_f16<2>(xw), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<3>(a), e2m1x2_f16<3>(xw), acc, false);
    return acc;
}
__device__ __forceinline__ float chunk32_raw(u32x4 a, uint32_t sa2, u32x4 xr, f32x2 sx, float acc) {
    float b0 = dot8_raw(a.x, xr.x, 0.0f);
    b0 = dot8_raw(a.y, xr.y, b0);
    float b1 = dot8_raw(a.z, xr.z, 0.0f);
    b1 = dot8_raw(a.w, xr.w, b1);
    const f32x2 sa = e4m3x2_f32(sa2);
    acc = __builtin_fmaf(b0, sa.x * sx.x, acc);
    acc = __builtin_fmaf(b1, sa.y * sx.y, acc);
    return acc;
}

template <int R, int U, int W>
__global__ void __launch_bounds__(W * kWave)
gemv_fastp(const uint8_t *__restrict__ A, const uint8_t *__restrict__ sfA,
           const uint8_t *__restrict__ x, const uint8_t *__restrict__ sfx,
           const float *__restrict__ alpha, uint16_t *__restrict__ c,
           float *__restrict__ part, int64_t l, int64_t m, int64_t k,
           int64_t kchunk, int64_t row_blocks) {
    static_assert(kMaxIters % U == 0, "U must divide the staged iteration count");
    constexpr int kXPerThread = (kMaxIters + W - 1) / W;   // x chunks of 32 elements per thread
    // LDS: codes as xr[it*64 + lane] (16 bytes), scale pairs as xsc[it*64 + lane]
    extern __shared__ u32x4 xr[];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);

    int64_t rb, b, split;
    group_index(row_blocks, l, &rb, &b, &split);

    const int64_t kb0 = split * kchunk;
    const int klen = static_cast<int>((k - kb0 < kchunk) ? (k - kb0) : kchunk);
    const int nit = (klen + static_cast<int>(kIterElems) - 1) / static_cast<int>(kIterElems);
    const int nstage = (nit + U - 1) / U;
    const int nslot = nstage * U;
    uint32_t *xsc = reinterpret_cast<uint32_t *>(xr + nslot * kWave);
    const int64_t row0 = rb * (W * R) + wave * R;

    const __amdgpu_buffer_rsrc_t xbuf = buffer_of(x + b * (k / 2) + kb0 / 2, klen / 2);
    const __amdgpu_buffer_rsrc_t sxbuf = buffer_of(sfx + b * (k / 16) + kb0 / 16, klen / 16);
    u32x4 xv[kXPerThread];
    uint16_t xs2[kXPerThread];
#pragma unroll
    for (int i = 0; i < kXPerThread; ++i) {
        const int q = tid + i * W * kWave;
        xv[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xbuf, 16 * q, 0, 0));
        xs2[i] = __builtin_amdgcn_raw_buffer_load_b16(sxbuf, 2 * q, 0, 0);
    }

    __amdgpu_buffer_rsrc_t abuf_rs[R], sbuf_rs[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = (row0 + r < m) ? row0 + r : m - 1;   // rows past m: read row m-1, never written
        abuf_rs[r] = buffer_of(A + (b * m + row) * (k / 2) + kb0 / 2, klen / 2);
        sbuf_rs[r] = buffer_of(sfA + (b * m + row) * (k / 16) + kb0 / 16, klen / 16);
    }

    u32x4 abuf[U][R];
    uint16_t sbuf[U][R];
    auto issue = [&](int it, int u) {
        const int off = it * static_cast<int>(kIterElems / 2) + lane * 16;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            abuf[u][r] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(abuf_rs[r], off, 0, kNonTemporal));
            sbuf[u][r] = __builtin_amdgcn_raw_buffer_load_b16(sbuf_rs[r], off / 8, 0, kNonTemporal);
        }
    };
    auto consume = [&](int it, int u, float (&acc)[R]) {
        const u32x4 xq = xr[it * kWave + lane];
        const f32x2 sx = e4m3x2_f32(xsc[it * kWave + lane]);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = chunk32_raw(abuf[u][r], sbuf[u][r], xq, sx, acc[r]);
    };

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;

    // One loop for the whole K-range.  Its first pass only issues loads and
    // then stages x (waiting only for the x loads, which were issued before
    // any A), so every pass issues the same loads in the same order and the
    // load counter waits only for the oldest step.  `first` is 0, taken from
    // an argument so the compiler cannot peel the first pass off the loop.
    const int first = static_cast<int>(kchunk >> 62);
    for (int t = first - U; t < first + nslot; t += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int it = t - first + u;
            if (t >= first && it < nit) consume(it, u, acc);   // wave-uniform, no global memory
            issue(it + U, u);   // past the K-range: zeros, no traffic
            phase_fence();
        }
#pragma unroll
        for (int i = 0; i < kXPerThread; ++i) {
            __asm__ volatile("" : "+v"(xv[i].x), "+v"(xv[i].y), "+v"(xv[i].z), "+v"(xv[i].w),
                             "+v"(xs2[i]));
        }
        if (t == first - U) {
#pragma unroll
            for (int i = 0; i < kXPerThread; ++i) {
                const int q = tid + i * W * kWave;
                if (q < nslot * kWave) {
                    xr[q] = xv[i];
                    xsc[q] = xs2[i];
                }
            }
            __syncthreads();
        }
    }

    float sum[R];
#pragma unroll
    for (int r = 0; r < R; ++r) sum[r] = wave_sum(acc[r]);

    if (lane < R) {
        float v = sum[0];
#pragma unroll
        for (int r = 1; r < R; ++r)
            if (lane == r) v = sum[r];
        const int64_t row = row0 + lane;
        if (row < m) {
            if (part != nullptr) {
                part[(split * l + b) * m + row] = v;
            } else {
                const float al = alpha ? alpha[b] : 1.0f;
                c[b * m + row] = f16_of_product(al, v);
            }
        }
    }
}

// ---------------------------------------------------------------- unstaged fast kernel
// The packed-x arithmetic with no LDS at all: every wave loads x's codes and
// scale pair for its iteration straight from memory (ordinary cached loads:
// all workgroups read the same x, which stays in L2) next to its R rows of A.
// No staging, no barrier: a wave starts consuming as soon as its first loads
// land, and K needs no split for LDS capacity.  The x decode is shared by the
// wave's R rows.
template <int R, int U, int W>
__global__ void __launch_bounds__(W * kWave)
gemv_fastg(const uint8_t *__restrict__ A, const uint8_t *__restrict__ sfA,
           const uint8_t *__restrict__ x, const uint8_t *__restrict__ sfx,
           const float *__restrict__ alpha, uint16_t *__restrict__ c,
           float *__restrict__ part, int64_t l, int64_t m, int64_t k,
           int64_t kchunk, int64_t row_blocks) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    int64_t rb, b, split;
    group_index(row_blocks, l, &rb, &b, &split);

    const int64_t kb0 = split * kchunk;
    const int klen = static_cast<int>((k - kb0 < kchunk) ? (k - kb0) : kchunk);
    const int nit = (klen + static_cast<int>(kIterElems) - 1) / static_cast<int>(kIterElems);
    const int nstage = (nit + U - 1) / U;
    const int64_t row0 = rb * (W * R) + wave * R;

    const __amdgpu_buffer_rsrc_t xbuf = buffer_of(x + b * (k / 2) + kb0 / 2, klen / 2);
    const __amdgpu_buffer_rsrc_t sxbuf = buffer_of(sfx + b * (k / 16) + kb0 / 16, klen / 16);
    __amdgpu_buffer_rsrc_t abuf_rs[R], sbuf_rs[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = (row0 + r < m) ? row0 + r : m - 1;   // rows past m: read row m-1, never written
        abuf_rs[r] = buffer_of(A + (b * m + row) * (k / 2) + kb0 / 2, klen / 2);
        sbuf_rs[r] = buffer_of(sfA + (b * m + row) * (k / 16) + kb0 / 16, klen / 16);
    }

    u32x4 abuf[U][R], xq[U];
    uint16_t sbuf[U][R], xs[U];
    auto issue = [&](int it, int u) {
        const int off = it * static_cast<int>(kIterElems / 2) + lane * 16;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            abuf[u][r] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(abuf_rs[r], off, 0, kNonTemporal));
            sbuf[u][r] = __builtin_amdgcn_raw_buffer_load_b16(sbuf_rs[r], off / 8, 0, kNonTemporal);
        }
        xq[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xbuf, off, 0, 0));
        xs[u] = __builtin_amdgcn_raw_buffer_load_b16(sxbuf, off / 8, 0, 0);
    };
    auto consume = [&](int u, float (&acc)[R]) {
        const f32x2 sx = e4m3x2_f32(xs[u]);
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = chunk32_raw(abuf[u][r], sbuf[u][r], xq[u], sx, acc[r]);
    };

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;

    phase_fence();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        issue(u, u);
        phase_fence();
    }
    for (int st = 0; st + 1 < nstage; ++st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            consume(u, acc);
            issue(st * U + u + U, u);
            phase_fence();
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if ((nstage - 1) * U + u < nit) consume(u, acc);   // wave-uniform: skip iterations past K
    }

    float sum[R];
#pragma unroll
    for (int r = 0; r < R; ++r) sum[r] = wave_sum(acc[r]);

    if (lane < R) {
        float v = sum[0];
#pragma unroll
        for (int r = 1; r < R; ++r)
            if (lane == r) v = sum[r];
        const int64_t row = row0 + lane;
        if (row < m) {
            if (part != nullptr) {
                part[(split * l + b) * m + row] = v;
            } else {
                const float al = alpha ? alpha[b] : 1.0f;
                c[b * m + row] = f16_of_product(al, v);
            }
        }
    }
}

// ---------------------------------------------------------------- row-tile kernel
// A workgroup owns a tile of TR rows (16, 8 or 4) of one batch and the
// K-range of its split; its W waves share the tile and take K slices of 2048
// elements (1 KiB of every row) in turn: wave w takes slices w, w + W, ...
// For one slice a wave issues, back to back, x's 16 bytes and scale pair per
// lane and then one 16-byte load per lane for each of the TR rows (1 KiB of
// a row per instruction) with the row's scale pair, so TR KiB of A per wave
// are in flight at once and every load is row-contiguous.  x~ of the lane's
// 32 elements is decoded once into registers and serves all TR rows; no LDS
// holds x, and nothing waits at a barrier before the arithmetic.  A row is
// consumed as soon as its load lands, in issue order.  Fewer rows per tile
// mean more waves for the same rows and less arithmetic left per wave when
// its last load lands.
//
// Reduction: the TR per-lane partial sums are halved twice by swapping the
// 32-lane halves and then the 16-lane rows of the wave (each lane keeps the
// rows its half or row is responsible for and adds its partner's values),
// then the TR/4 values left are summed inside each 16-lane row by DPP.  The
// waves' row sums meet in LDS and wave 0 adds them in wave order, so the
// result does not depend on timing; a one-wave tile writes its rows from the
// lanes that hold them.
constexpr int kTileMaxWaves = 8;

template <int W, int TR>
__global__ void __launch_bounds__(W * kWave)
gemv_tile(const uint8_t *__restrict__ A, const uint8_t *__restrict__ sfA,
          const uint8_t *__restrict__ x, const uint8_t *__restrict__ sfx,
          const float *__restrict__ alpha, uint16_t *__restrict__ c,
          float *__restrict__ part, int64_t l, int64_t m, int64_t k,
          int64_t kchunk, int64_t row_blocks) {
    static_assert(W >= 1 && W <= kTileMaxWaves, "waves per tile");
    static_assert(TR == 16 || TR == 8 || TR == 4, "rows per tile");
    __shared__ float red[W * TR];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    int64_t rb, b, split;
    group_index(row_blocks, l, &rb, &b, &split);

    const int64_t kb0 = split * kchunk;
    const int klen = static_cast<int>((k - kb0 < kchunk) ? (k - kb0) : kchunk);
    const int nsl = (klen + static_cast<int>(kIterElems) - 1) / static_cast<int>(kIterElems);
    const int64_t row0 = rb * TR;
    const int nrows = static_cast<int>((m - row0 < TR) ? (m - row0) : TR);
    const int half = static_cast<int>(k / 2), sixteenth = static_cast<int>(k / 16);

    // One descriptor per operand over the tile's rows, from the split's first
    // element: row r's bytes start at r * half (codes) and r * sixteenth
    // (scales).  Offsets of rows past the tile's end, and of lanes past the
    // K-range, are past the descriptor's range and read zeros.
    const __amdgpu_buffer_rsrc_t ad = buffer_of(A + (b * m + row0) * half + kb0 / 2, nrows * half);
    const __amdgpu_buffer_rsrc_t sd =
        buffer_of(sfA + (b * m + row0) * sixteenth + kb0 / 16, nrows * sixteenth);
    const __amdgpu_buffer_rsrc_t xbuf = buffer_of(x + b * half + kb0 / 2, klen / 2);
    const __amdgpu_buffer_rsrc_t sxbuf = buffer_of(sfx + b * sixteenth + kb0 / 16, klen / 16);

    float acc[TR];
#pragma unroll
    for (int r = 0; r < TR; ++r) acc[r] = 0.0f;

    for (int s = wave; s < nsl; s += W) {
        const int e0 = s * static_cast<int>(kIterElems) + 32 * lane;   // lane's first element
        const int xo = e0 / 2;
        const uint32_t lo = e0 < klen ? static_cast<uint32_t>(xo) : kOutOfRange;
        const uint32_t lso = e0 < klen ? static_cast<uint32_t>(e0 / 16) : kOutOfRange;

        phase_fence();
        const u32x4 xv = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xbuf, xo, 0, 0));
        const uint16_t xs2 = __builtin_amdgcn_raw_buffer_load_b16(sxbuf, e0 / 16, 0, 0);
        u32x4 av[TR];
        uint16_t sv[TR];
#pragma unroll
        for (int r = 0; r < TR; ++r) {
            av[r] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(ad, lo + r * half, 0, kNonTemporal));
            sv[r] = __builtin_amdgcn_raw_buffer_load_b16(sd, lso + r * sixteenth, 0, kNonTemporal);
            phase_fence();   // row by row, in the order the rows are consumed
        }

        u32x4 xq[4];
        decode_x32(xv, xs2, xq);
#pragma unroll
        for (int r = 0; r < TR; ++r) acc[r] = chunk32(av[r], sv[r], xq, acc[r]);
    }

    // Halve across the 32-lane halves: the low half keeps rows 0 .. TR/2 - 1,
    // the high half the rest.
    constexpr int H = TR / 2, Q = TR / 4;
    float h2[H];
#pragma unroll
    for (int r = 0; r < H; ++r) {
        const auto t = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, acc[r]),
                                                        __builtin_bit_cast(unsigned, acc[r + H]),
                                                        false, false);
        h2[r] = __builtin_bit_cast(float, static_cast<unsigned>(t[0])) +
                __builtin_bit_cast(float, static_cast<unsigned>(t[1]));
    }
    // Halve across 16-lane rows: even rows keep values 0 .. TR/4 - 1, odd rows the rest.
    float h4[Q];
#pragma unroll
    for (int r = 0; r < Q; ++r) {
        const auto t = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, h2[r]),
                                                        __builtin_bit_cast(unsigned, h2[r + Q]),
                                                        false, false);
        h4[r] = __builtin_bit_cast(float, static_cast<unsigned>(t[0])) +
                __builtin_bit_cast(float, static_cast<unsigned>(t[1]));
    }
    // Sum inside each 16-lane row.
#pragma unroll
    for (int r = 0; r < Q; ++r) {
        float v = h4[r];
        v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
        v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
        v += dpp<0x141>(v);   // row_half_mirror
        v += dpp<0x140>(v);   // row_mirror
        h4[r] = v;
    }
    // Lane j < TR/4 of 16-lane row q (q = lane / 16) holds tile row
    // j + (TR/4) (q & 1) + (TR/2) (q >> 1).
    const int j = lane & 15, q = lane >> 4;
    const int trow = j + Q * (q & 1) + H * (q >> 1);
    float tv = h4[0];
#pragma unroll
    for (int r = 1; r < Q; ++r)
        if (j == r) tv = h4[r];
    if constexpr (W == 1) {
        // one wave: those lanes write their rows themselves (no LDS round trip
        // before the kernel's last stores)
        if (j < Q && trow < nrows) {
            const int64_t row = row0 + trow;
            if (part != nullptr) {
                part[(split * l + b) * m + row] = tv;
            } else {
                const float al = alpha ? alpha[b] : 1.0f;
                c[b * m + row] = f16_of_product(al, tv);
            }
        }
        return;
    }
    if (j < Q) red[wave * TR + trow] = tv;
    __syncthreads();
    if (wave == 0 && lane < nrows) {
        float v = red[lane];
#pragma unroll
        for (int w = 1; w < W; ++w) v += red[w * TR + lane];
        const int64_t row = row0 + lane;
        if (part != nullptr) {
            part[(split * l + b) * m + row] = v;
        } else {
            const float al = alpha ? alpha[b] : 1.0f;
            c[b * m + row] = f16_of_product(al, v);
        }
    }
}

// ---------------------------------------------------------------- generic kernel
// Any k % 16 == 0 and any byte alignment of A, sfA, x, sfx.  One wave per
// (split, batch, row); lanes take 16-element blocks; bytes are loaded singly
// and x~ is decoded on the fly.
__device__ __forceinline__ uint32_t load_u32_bytes(const uint8_t *p) {
    return static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 8) |
           (static_cast<uint32_t>(p[2]) << 16) | (static_cast<uint32_t>(p[3]) << 24);
}

__device__ __forceinline__ float dot8_generic(uint32_t a, uint32_t xw, f16x2 sx, float acc) {
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<0>(a), e2m1x2_f16<0>(xw) * sx, acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<1>(a), e2m1x2_f16<1>(xw) * sx, acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<2>(a), e2m1x2_f16<2>(xw) * sx, acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<3>(a), e2m1x2_f16<3>(xw) * sx, acc, false);
    return acc;
}

__global__ void __launch_bounds__(kGenericWaves * kWave)
gemv_generic(const uint8_t *__restrict__ A, const uint8_t *__restrict__ sfA,
             const uint8_t *__restrict__ x, const uint8_t *__restrict__ sfx,
             const float *__restrict__ alpha, uint16_t *__restrict__ c,
             float *__restrict__ part, int64_t l, int64_t m, int64_t k, int64_t kchunk,
             int64_t row_blocks) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int64_t rb, b, split;
    group_index(row_blocks, l, &rb, &b, &split);
    const int64_t row = rb * kGenericWaves + wave;
    if (row >= m) return;

    const int64_t kb0 = split * kchunk;
    const int64_t klen = (k - kb0 < kchunk) ? (k - kb0) : kchunk;
    const uint8_t *arow = A + (b * m + row) * (k / 2) + kb0 / 2;
    const uint8_t *srow = sfA + (b * m + row) * (k / 16) + kb0 / 16;
    const uint8_t *xrow = x + b * (k / 2) + kb0 / 2;
    const uint8_t *sxrow = sfx + b * (k / 16) + kb0 / 16;

    float acc = 0.0f;
    for (int64_t blk = lane; blk < klen / 16; blk += kWave) {
        const uint32_t a0 = load_u32_bytes(arow + blk * 8);
        const uint32_t a1 = load_u32_bytes(arow + blk * 8 + 4);
        const uint32_t x0 = load_u32_bytes(xrow + blk * 8);
        const uint32_t x1 = load_u32_bytes(xrow + blk * 8 + 4);
        const float sa = e4m3x2_f32(srow[blk]).x;
        const _Float16 hs = static_cast<_Float16>(e4m3x2_f32(sxrow[blk]).x);
        const f16x2 sx = {hs, hs};
        float bs = dot8_generic(a0, x0, sx, 0.0f);
        bs = dot8_generic(a1, x1, sx, bs);
        acc = __builtin_fmaf(bs, sa, acc);
    }
    const float v = wave_sum(acc);
    if (lane == 0) {
        if (part != nullptr) {
            part[(split * l + b) * m + row] = v;
        } else {
            const float al = alpha ? alpha[b] : 1.0f;
            c[b * m + row] = f16_of_product(al, v);
        }
    }
}

// ---------------------------------------------------------------- split-K second pass
// c[i] = f16(alpha * (((0 + p[0][i]) + p[1][i]) + ...)), splits in order.
__global__ void __launch_bounds__(kReduceThreads)
gemv_splitk_reduce(const float *__restrict__ part, const float *__restrict__ alpha,
                   uint16_t *__restrict__ c, int64_t l, int64_t m, int64_t ksplit) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kReduceThreads + threadIdx.x;
    const int64_t n = l * m;
    if (i >= n) return;
    float s = 0.0f;
    for (int64_t j = 0; j < ksplit; ++j) s += part[j * n + i];
    const float al = alpha ? alpha[i / m] : 1.0f;
    c[i] = f16_of_product(al, s);
}

}  // namespace

#endif  // NVFP4_GEMV_KERNELS_H
