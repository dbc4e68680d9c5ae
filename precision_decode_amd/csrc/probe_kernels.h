// Read probes of the NVFP4 GEMV library (gfx950): plain streaming reads, no
// arithmetic, whose run times are the read ceilings the GEMV is measured
// against on the same GPU in the same run.  Device code only; the entry
// points are nvfp4_hbm_read_probe and nvfp4_hbm_read_probe_rows in
// nvfp4_gemv.hip, this header's only includer.
#ifndef NVFP4_PROBE_KERNELS_H
#define NVFP4_PROBE_KERNELS_H

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "device_common.h"
#include "gemv_plan.h"

namespace {

using namespace nvfp4dev;
using namespace nvfp4plan;

constexpr int kProbeThreads = 256;
constexpr int kProbeMaxGroups = 4096;

// ---------------------------------------------------------------- read probe
// Reads `bytes` once in contiguous 16 KiB chunks, one chunk per workgroup of
// 4 waves at a time (workgroup g takes chunks g, g + G, ... for a grid of G):
// each thread issues its 4 16-byte non-temporal loads of the chunk together,
// so every wave instruction reads 1 KiB contiguously and the whole chunk is
// in flight at once.  Of the read orders measured (chunks of 16 KiB to 1 MiB,
// 4 to 16 waves, 4 or 8 loads per thread, cached or non-temporal), this one
// read 33-132 MB operands fastest and 1 GiB within 1% of the best.  A
// descriptor over each chunk turns loads past the end into zeros.
constexpr int kProbeLoads = 4;
constexpr int64_t kProbeChunk = int64_t(kProbeThreads) * kProbeLoads * 16;   // 16 KiB

__global__ void __launch_bounds__(kProbeThreads)
hbm_read_probe(const uint8_t *__restrict__ buf, int64_t bytes, uint32_t *__restrict__ sink) {
    const int64_t nchunks = (bytes + kProbeChunk - 1) / kProbeChunk;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
        const int64_t base = ch * kProbeChunk;
        const int len = static_cast<int>((bytes - base < kProbeChunk) ? bytes - base : kProbeChunk);
        const __amdgpu_buffer_rsrc_t rs = buffer_of(buf + base, len);
        u32x4 v[kProbeLoads];
#pragma unroll
        for (int j = 0; j < kProbeLoads; ++j)
            v[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rs, (j * kProbeThreads + threadIdx.x) * 16u, 0,
                                                 kNonTemporal));
#pragma unroll
        for (int j = 0; j < kProbeLoads; ++j) acc ^= v[j];
    }
    uint32_t w = acc.x ^ acc.y ^ acc.z ^ acc.w;
    for (int o = kWave / 2; o >= 1; o >>= 1) w ^= __shfl_xor(w, o, kWave);
    __shared__ uint32_t per_wave[kProbeThreads / kWave];
    if ((threadIdx.x & (kWave - 1)) == 0) per_wave[threadIdx.x / kWave] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t all = 0u;
        for (int i = 0; i < kProbeThreads / kWave; ++i) all ^= per_wave[i];
        sink[blockIdx.x] = all;
    }
}

// ---------------------------------------------------------------- row read probe
// Reads `rows` rows of codes (k/2 bytes each) and of scales (k/16 bytes each)
// with the load pattern of gemv_fast<2, 4, 7>, the GEMV's kernel for long
// rows, and no arithmetic: a workgroup of 7 waves owns 14 consecutive rows,
// each wave streams 2 rows with 4 iterations of 1 KiB per row in flight,
// 16-byte non-temporal loads of the codes and 2-byte loads of the scales,
// one buffer descriptor per row (loads past a row's end, and rows past the
// last, read zeros without touching memory).  Its time is the read ceiling of
// that pattern for a matrix of this shape.  Each workgroup stores the XOR of
// everything it read in sink[blockIdx.x].
constexpr int kRowProbeR = 2, kRowProbeU = 4, kRowProbeW = 7;

__global__ void __launch_bounds__(kRowProbeW * kWave)
hbm_read_rows(const uint8_t *__restrict__ A, const uint8_t *__restrict__ sfA, int64_t rows,
              int64_t k, uint32_t *__restrict__ sink) {
    constexpr int R = kRowProbeR, U = kRowProbeU, W = kRowProbeW;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t row0 = (static_cast<int64_t>(blockIdx.x) * W + wave) * R;
    const int nit = static_cast<int>((k + kIterElems - 1) / kIterElems);
    const int nstage = (nit + U - 1) / U;

    __amdgpu_buffer_rsrc_t ad[R], sd[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool in = row0 + r < rows;
        const int64_t row = in ? row0 + r : 0;
        ad[r] = buffer_of(A + row * (k / 2), in ? static_cast<int>(k / 2) : 0);
        sd[r] = buffer_of(sfA + row * (k / 16), in ? static_cast<int>(k / 16) : 0);
    }
    u32x4 v[U][R];
    uint16_t sv[U][R];
    auto issue = [&](int it, int u) {
        const int off = it * static_cast<int>(kIterElems / 2) + lane * 16;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            v[u][r] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(ad[r], off, 0, kNonTemporal));
            sv[u][r] = __builtin_amdgcn_raw_buffer_load_b16(sd[r], off / 8, 0, kNonTemporal);
        }
    };
    u32x4 acc = {0u, 0u, 0u, 0u};
    uint32_t sacc = 0u;
    phase_fence();
#pragma unroll
    for (int u = 0; u < U; ++u) {
        issue(u, u);
        phase_fence();
    }
    for (int st = 0; st + 1 < nstage; ++st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                acc ^= v[u][r];
                sacc ^= sv[u][r];
            }
            issue((st + 1) * U + u, u);   // past the last iteration: zeros, no traffic
            phase_fence();
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            acc ^= v[u][r];
            sacc ^= sv[u][r];
        }
    }
    uint32_t w = acc.x ^ acc.y ^ acc.z ^ acc.w ^ sacc;
    for (int o = kWave / 2; o >= 1; o >>= 1) w ^= __shfl_xor(w, o, kWave);
    __shared__ uint32_t per_wave[W];
    if (lane == 0) per_wave[wave] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t all = 0u;
        for (int i = 0; i < W; ++i) all ^= per_wave[i];
        sink[blockIdx.x] = all;
    }
}

}  // namespace

#endif  // NVFP4_PROBE_KERNELS_H
