// Device code of the small-N GEMM and the grouped GEMV (kernels and their
// helpers); the design is described at the top of nvfp4_mma.hip, the only
// includer, which holds the host side (launches and entry points).  The plan
// (shape rules, variants, defaults) is mma_plan.h.
#ifndef NVFP4_MMA_KERNELS_H
#define NVFP4_MMA_KERNELS_H

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "mma_plan.h"

namespace {

using namespace nvfp4dev;
using namespace nvfp4mmaplan;

constexpr int64_t kSliceElems = 2048;   // VALU tiles: K elements of one slice, 1 KiB of a row
// Packed weights (nvfp4_mma_pack_weight): one window of one 16-row tile is
// 2 KiB of codes (two 1 KiB halves, 16 bytes per lane) and 256 bytes of
// scales (4 per lane), in the order the lanes of mma_stream read them.
constexpr int kPackedWinBytes = 2048;
constexpr int kPackedWinScaleBytes = 256;
constexpr int kPackThreads = 256;

struct MmaArgs {
    const uint8_t *W, *sW;      // weights [groups][rows][k/2], scales [groups][rows][k/16]
    const uint8_t *V, *sV;      // vectors [.][k/2], scales [.][k/16]
    const float *alpha;         // small-N: [groups] or NULL
    const int32_t *offsets;     // grouped: [groups] cumulative token ends
    const float *gs_v, *gs_w;   // grouped: [groups] or NULL
    uint16_t *c;
    float *part;                // small-N split-K partials, or NULL
    int64_t groups, rows, nvec, k;   // nvec: n (small-N) or tokens (grouped)
    int64_t kchunk;             // K elements per workgroup
    int64_t row_blocks;         // workgroups along the rows of one group
    int64_t rows_per_block;     // weight rows per workgroup (at most 16 per row tile)
    int32_t out_bf16;
};

// Vectors [v0, v1) that group g multiplies: n per batch for the small-N GEMM,
// the expert's token range for the grouped GEMV (offsets clamped to the
// token count, so any offsets stay inside the arrays).
template <bool GROUPED>
__device__ __forceinline__ void vector_range(const MmaArgs &a, int64_t g, int64_t *v0, int64_t *v1) {
    if (GROUPED) {
        auto clampt = [&](int64_t v) { return v < 0 ? int64_t(0) : (v > a.nvec ? a.nvec : v); };
        *v0 = g > 0 ? clampt(a.offsets[g - 1]) : 0;
        *v1 = clampt(a.offsets[g]);
    } else {
        *v0 = g * a.nvec;
        *v1 = *v0 + a.nvec;
    }
}

__device__ __forceinline__ uint16_t round_out(float al, float v, int32_t bf16) {
    return bf16 ? bf16_of_product(al, v) : f16_of_product(al, v);
}

__device__ __forceinline__ float group_alpha(const MmaArgs &a, int64_t g, bool grouped) {
    if (grouped) {
        const float gv = a.gs_v ? a.gs_v[g] : 1.0f;
        const float gw = a.gs_w ? a.gs_w[g] : 1.0f;
        return gv * gw;   // one fp32 rounding
    }
    return a.alpha ? a.alpha[g] : 1.0f;
}

// ---------------------------------------------------------------- decode
__device__ __forceinline__ f16x8 join(f16x2 p, f16x2 q, f16x2 r, f16x2 s) {
    return f16x8{p.x, p.y, q.x, q.y, r.x, r.y, s.x, s.y};
}

// 32 codes (16 bytes, element 2i in the low nibble of byte i) and their two
// block-scale codes (bytes 0 and 1 of s2) -> four MFMA operands holding
// e2m1 * e4m3 for elements 0-7, 8-15, 16-23, 24-31.  Exact in fp16.
__device__ __forceinline__ void decode32(u32x4 q, uint32_t s2, f16x8 (&o)[4]) {
    const f16x2 s = e4m3x2_f16(s2);
    const f16x2 s0 = {s.x, s.x};
    const f16x2 s1 = {s.y, s.y};
    o[0] = join(e2m1x2_f16<0>(q.x) * s0, e2m1x2_f16<1>(q.x) * s0, e2m1x2_f16<2>(q.x) * s0,
                e2m1x2_f16<3>(q.x) * s0);
    o[1] = join(e2m1x2_f16<0>(q.y) * s0, e2m1x2_f16<1>(q.y) * s0, e2m1x2_f16<2>(q.y) * s0,
                e2m1x2_f16<3>(q.y) * s0);
    o[2] = join(e2m1x2_f16<0>(q.z) * s1, e2m1x2_f16<1>(q.z) * s1, e2m1x2_f16<2>(q.z) * s1,
                e2m1x2_f16<3>(q.z) * s1);
    o[3] = join(e2m1x2_f16<0>(q.w) * s1, e2m1x2_f16<1>(q.w) * s1, e2m1x2_f16<2>(q.w) * s1,
                e2m1x2_f16<3>(q.w) * s1);
}

// ---------------------------------------------------------------- fast kernel
// blockIdx.x enumerates (split, group, row block) with the row block fastest.
// A workgroup owns rows_per_block (at most R*16) weight rows of one group,
// their MFMA tiles padded with rows that read zeros, and the K range
// [split*kchunk, min(k, (split+1)*kchunk)); wave w takes windows w, w+W, ...
// of it.  A window is 256 elements, 128 bytes of every row: one whole cache
// line, read by two back-to-back load instructions of the same wave, so no
// line is shared between waves.  Lane i + 16q loads, per window, the 64
// elements at window offset 64q (32 code bytes, two 16-byte loads) and their
// four scale codes (one 4-byte load) of weight row i of each row tile and of
// vector i of the current pass of 16 vectors.  The scale lines are read 16
// bytes per row and window, so they are loaded through the cache rather than
// as streamed data.
//
// All global reads are buffer loads: a descriptor covers the workgroup's
// valid weight rows (or the pass's vectors) over the whole K, and a lane
// whose row or vector does not exist, or whose elements lie past the K range,
// gets zeros from the hardware range check without touching memory.  No load
// sits under a branch, so the compiler can count outstanding loads and keep U
// windows in flight.
//
// Small-N: the A operand of the MFMA is the weight tile, the B operand the
// vectors, so lane i + 16q ends with rows 4q .. 4q+3, vector i.  Grouped: the
// operands swap, so lane i + 16q ends with tokens 4q .. 4q+3, row i, and the
// 16 lanes of a quarter write 16 consecutive outputs of a token.
template <int R, int U, int W, bool GROUPED, bool PACKED>
__global__ void __launch_bounds__(W * kWave) mma_stream(const MmaArgs a) {
    __shared__ f32x4 red[(W > 1 ? W - 1 : 1) * R * kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int li = lane & (kTile - 1);
    const int kq = lane >> 4;

    // the plan keeps the workgroup count below 2^31: 32-bit division
    const uint32_t gi = blockIdx.x;
    const uint32_t rbs = static_cast<uint32_t>(a.row_blocks), gs = static_cast<uint32_t>(a.groups);
    const uint32_t q = gi / rbs;
    const int64_t rb = gi - q * rbs;
    const int64_t grp = q % gs;
    const int64_t split = q / gs;

    int64_t v0, v1;
    vector_range<GROUPED>(a, grp, &v0, &v1);
    if (v1 <= v0) return;   // workgroup-uniform: an expert without tokens

    const int64_t k = a.k;
    const uint32_t half = static_cast<uint32_t>(k / 2);
    const uint32_t sixteenth = static_cast<uint32_t>(k / 16);
    const int64_t kb0 = split * a.kchunk;
    const int64_t kend = (k - kb0 < a.kchunk) ? k : kb0 + a.kchunk;
    const int nwin = static_cast<int>((kend - kb0 + kWinElems - 1) / kWinElems);
    const int niter = nwin > wave ? (nwin - wave + W - 1) / W : 0;

    const int64_t row0 = rb * a.rows_per_block;
    const int64_t nrows = (a.rows - row0 < a.rows_per_block) ? a.rows - row0 : a.rows_per_block;
    // Packed weights: the group's 16-row tiles one after another, each as its
    // windows one after another (2 KiB of codes, 256 bytes of scales each);
    // rows_per_block is a multiple of 16, so the workgroup starts on a tile.
    const int64_t pwin = (k + kWinElems - 1) / kWinElems;           // windows per tile
    const int64_t ptiles = (a.rows + kTile - 1) / kTile;            // tiles per group
    const int64_t tile0 = grp * ptiles + row0 / kTile;
    const int ntile = static_cast<int>((nrows + kTile - 1) / kTile);
    const __amdgpu_buffer_rsrc_t wdesc =
        PACKED ? buffer_of(a.W + tile0 * pwin * kPackedWinBytes,
                           static_cast<int>(ntile * pwin * kPackedWinBytes))
               : buffer_of(a.W + (grp * a.rows + row0) * (k / 2), static_cast<int>(nrows * (k / 2)));
    const __amdgpu_buffer_rsrc_t swdesc =
        PACKED ? buffer_of(a.sW + tile0 * pwin * kPackedWinScaleBytes,
                           static_cast<int>(ntile * pwin * kPackedWinScaleBytes))
               : buffer_of(a.sW + (grp * a.rows + row0) * (k / 16),
                           static_cast<int>(nrows * (k / 16)));
    const float al = group_alpha(a, grp, GROUPED);

    for (int64_t vp = v0; vp < v1; vp += kTile) {
        const int64_t nv = (v1 - vp < kTile) ? v1 - vp : kTile;
        const __amdgpu_buffer_rsrc_t vdesc =
            buffer_of(a.V + vp * (k / 2), static_cast<int>(nv * (k / 2)));
        const __amdgpu_buffer_rsrc_t svdesc =
            buffer_of(a.sV + vp * (k / 16), static_cast<int>(nv * (k / 16)));

        u32x4 wq[U][R][2], vq[U][2];
        uint32_t ws[U][R], vs[U];
        auto issue = [&](int i, int u) {
            const int64_t kk = kb0 + static_cast<int64_t>(wave + W * i) * kWinElems + kq * kLaneElems;
            const bool in = kk < kend;
            const uint32_t ko = static_cast<uint32_t>(kk / 2);
            const uint32_t so = static_cast<uint32_t>(kk / 16);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                uint32_t o, os, hstep;
                if (PACKED) {
                    // window kk / 256 of tile r: the lane's 16-byte pieces at
                    // 16 lane and 1024 + 16 lane, its scale word at 4 lane
                    const uint32_t wi = static_cast<uint32_t>(r * pwin + kk / kWinElems);
                    o = in ? wi * kPackedWinBytes + 16 * lane : kOutOfRange;
                    os = in ? wi * kPackedWinScaleBytes + 4 * lane : kOutOfRange;
                    hstep = kPackedWinBytes / 2;
                } else {
                    const uint32_t row = static_cast<uint32_t>(r * kTile + li);
                    o = in ? row * half + ko : kOutOfRange;
                    os = in ? row * sixteenth + so : kOutOfRange;
                    hstep = 16;
                }
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wq[u][r][h] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(wdesc, o + hstep * h, 0, kNonTemporal));
                ws[u][r] = __builtin_amdgcn_raw_buffer_load_b32(swdesc, os, 0, 0);
            }
            const uint32_t o = in ? static_cast<uint32_t>(li) * half + ko : kOutOfRange;
            const uint32_t os = in ? static_cast<uint32_t>(li) * sixteenth + so : kOutOfRange;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                vq[u][h] = __builtin_bit_cast(u32x4,
                                              __builtin_amdgcn_raw_buffer_load_b128(vdesc, o + 16 * h, 0, 0));
            vs[u] = __builtin_amdgcn_raw_buffer_load_b32(svdesc, os, 0, 0);
        };

        f32x4 acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        auto consume = [&](int u) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f16x8 vo[4];
                decode32(vq[u][h], vs[u] >> (16 * h), vo);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    f16x8 wo[4];
                    decode32(wq[u][r][h], ws[u][r] >> (16 * h), wo);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        if (GROUPED)
                            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vo[s], wo[s], acc[r], 0,
                                                                            0, 0);
                        else
                            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wo[s], vo[s], acc[r], 0,
                                                                            0, 0);
                    }
                }
            }
        };

        phase_fence();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            issue(u, u);
            phase_fence();
        }
        for (int i = 0; i < niter; i += U) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (i + u < niter) consume(u);   // wave-uniform
                issue(i + u + U, u);             // past the wave's windows: zeros, no traffic
                phase_fence();
            }
        }

        // Tiles of waves 1..W-1 through LDS, added to wave 0's in wave order.
        if (W > 1) {
            if (wave > 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) red[((wave - 1) * R + r) * kWave + lane] = acc[r];
            }
            __syncthreads();
        }
        if (wave == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                f32x4 s = acc[r];
                for (int w = 1; w < W; ++w) s += red[((w - 1) * R + r) * kWave + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (GROUPED) {
                        const int64_t t = vp + kq * 4 + e;
                        const int rr = r * kTile + li;
                        if (t < v1 && rr < nrows)
                            a.c[t * a.rows + row0 + rr] = round_out(al, s[e], a.out_bf16);
                    } else {
                        const int rr = r * kTile + kq * 4 + e;
                        const int64_t col = vp - v0 + li;
                        if (rr < nrows && col < a.nvec) {
                            const int64_t o = (grp * a.rows + row0 + rr) * a.nvec + col;
                            if (a.part != nullptr)
                                a.part[split * a.groups * a.rows * a.nvec + o] = s[e];
                            else
                                a.c[o] = round_out(al, s[e], a.out_bf16);
                        }
                    }
                }
            }
        }
        if (W > 1 && vp + kTile < v1) __syncthreads();   // before the next pass reuses `red`
    }
}

// ---------------------------------------------------------------- LDS-staged operands
// vmcnt wait with lgkmcnt and expcnt left at their maximum (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint32_t lds_address(const uint8_t *p) {
    return static_cast<uint32_t>(
        reinterpret_cast<size_t>((__attribute__((address_space(3))) const uint8_t *)(p)));
}

constexpr int kGroupWins = 4;   // windows per staged scale group (64 scale bytes per row)

// Loads issued after the last load of window j + 1, once window j + NS has
// been issued, where j sits at position u of its group: windows j + 2 ..
// j + NS, each with WL loads (its copies, and its vector loads into registers
// when the vectors skip LDS), plus SL scale copies where one starts a group.
template <int NS, int WL, int SL>
constexpr int loads_after_next(int u) {
    int n = 0;
    for (int t = 2; t <= NS; ++t) n += WL + ((u + t) % kGroupWins == 0 ? SL : 0);
    return n;
}

// Position of 16-byte chunk c (0..7) of staged row rho in its 128-byte LDS
// row.  The 16 rows that one quarter of a wave reads at the same chunk land
// on 16 distinct positions, and so do the two halves of 8 rows.
__device__ __forceinline__ int chunk_pos(int rho, int c) { return c ^ ((rho & 7) ^ ((rho >> 3) & 1)); }
// Position of 4-byte scale word w (0..15: window w / 4 of the group, lane
// piece w % 4) in the 64-byte scale row of staged row rho.  The 16 rows that
// one quarter reads at the same word land in 16 distinct banks, and a whole
// wave's read in 64.
__device__ __forceinline__ int scale_pos(int rho, int w) { return w ^ (4 * ((rho >> 2) & 3)); }

// One window's operands from LDS, in one asm block that waits for its own
// reads (the outputs are early-clobber: a read that returns while later ones
// are still being issued must not land in a register that holds one of their
// addresses): the weight codes of row li of the R tiles and of vector li
// (chunks 2kq and 2kq + 1, at addresses aw0, aw1 for tile 0; the next tile
// and the vectors 2 KiB apart) and the matching scale words (address as,
// tiles and vectors 1 KiB apart).  The compiler does not relate these reads to the
// direct-to-LDS loads (the kernel orders them with explicit vmcnt waits);
// with plain C++ reads it placed a full vmcnt(0) drain at the loop head.
template <int R>
__device__ __forceinline__ void lds_read_weights(uint32_t aw0, uint32_t aw1, uint32_t as,
                                                 u32x4 (&wq)[R][2], uint32_t (&ws)[R]) {
    static_assert(R == 2, "two row tiles per wave");
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b128 %2, %6 offset:2048\n\t"
        "ds_read_b128 %3, %7 offset:2048\n\t"
        "ds_read_b32 %4, %8\n\t"
        "ds_read_b32 %5, %8 offset:1024\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(wq[0][0]), "=&v"(wq[0][1]), "=&v"(wq[1][0]), "=&v"(wq[1][1]), "=&v"(ws[0]), "=&v"(ws[1])
        : "v"(aw0), "v"(aw1), "v"(as)
        : "memory");
}

template <int R>
__device__ __forceinline__ void lds_read_window(uint32_t aw0, uint32_t aw1, uint32_t as,
                                                u32x4 (&wq)[R][2], u32x4 (&vq)[2],
                                                uint32_t (&ws)[R], uint32_t &vs) {
    static_assert(R == 1 || R == 2, "one or two row tiles per wave");
    if constexpr (R == 2) {
        asm volatile(
            "ds_read_b128 %0, %9\n\t"
            "ds_read_b128 %1, %10\n\t"
            "ds_read_b128 %2, %9 offset:2048\n\t"
            "ds_read_b128 %3, %10 offset:2048\n\t"
            "ds_read_b128 %4, %9 offset:4096\n\t"
            "ds_read_b128 %5, %10 offset:4096\n\t"
            "ds_read_b32 %6, %11\n\t"
            "ds_read_b32 %7, %11 offset:1024\n\t"
            "ds_read_b32 %8, %11 offset:2048\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(wq[0][0]), "=&v"(wq[0][1]), "=&v"(wq[1][0]), "=&v"(wq[1][1]), "=&v"(vq[0]),
              "=&v"(vq[1]), "=&v"(ws[0]), "=&v"(ws[1]), "=&v"(vs)
            : "v"(aw0), "v"(aw1), "v"(as)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %6\n\t"
            "ds_read_b128 %1, %7\n\t"
            "ds_read_b128 %2, %6 offset:2048\n\t"
            "ds_read_b128 %3, %7 offset:2048\n\t"
            "ds_read_b32 %4, %8\n\t"
            "ds_read_b32 %5, %8 offset:1024\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(wq[0][0]), "=&v"(wq[0][1]), "=&v"(vq[0]), "=&v"(vq[1]), "=&v"(ws[0]), "=&v"(vs)
            : "v"(aw0), "v"(aw1), "v"(as)
            : "memory");
    }
}

// The same products as mma_stream on row-major weights, with every operand
// brought in by 16-byte direct-to-LDS buffer loads of whole 128-byte lines.
// In mma_stream each load instruction covers 16 rows x 64 bytes (the shape
// the matrix-core lanes want), and its scale and vector loads 16 rows x 16 or
// 64 bytes, so the address units handle many partial lines per byte.  Here:
//  * each wave takes a contiguous run of the workgroup's windows;
//  * per window, 8 rows x 128 bytes per instruction: the R*16 weight rows,
//    then the 16 vectors (one window slot of a per-wave LDS ring, NS slots);
//  * per group of 4 windows, the block scales of those rows and vectors, 64
//    bytes per row, into one of two scale slots: 16 rows per 16-byte copy
//    when every scale row and group starts 16-byte aligned (S16), else 4 rows
//    per 4-byte copy (scale rows are only 4-byte aligned in general, and a
//    16-byte copy from a 4-byte aligned address does not return the
//    addressed bytes);
//  * one asm block of LDS reads per window gives every lane the same 32 code
//    bytes and scale words that mma_stream's lane holds, so the decode and
//    the MFMAs are mma_stream's;
//  * with VR, only the weight rows and their scales go through LDS: every
//    lane loads its own 32 vector code bytes and scale word of the window
//    from L2 into registers (one ring of NS register slots), issued with the
//    window just before its copies, so the same waits cover them.  The slot
//    shrinks by the 16 vector rows, and more workgroups fit a compute unit;
//    with many vectors, 16 rows x 32 bytes per lane cost more as register
//    loads than as whole-line copies.
// Staged rows are swizzled (chunk_pos at 16 bytes, scale_pos at 4 bytes) so
// the reads hit distinct banks.  A window's loads always number the same
// (out-of-range ones read nothing but still count), so explicit vmcnt waits
// say exactly when a window has landed; the compiler's own tracking does not
// cover direct-to-LDS loads.  Lane pieces past the wave's K range get zero
// scales; rows and vectors past the block's read zeros or stale LDS, which
// only reach outputs that are never written (an MFMA output row or column
// depends on its own row and vector alone, and e2m1 codes are finite).
template <int R, int NS, int W, bool GROUPED, bool S16, bool VR = false, bool EARLY = false>
__global__ void __launch_bounds__(W * kWave) mma_lds(const MmaArgs a) {
    static_assert(NS == 2 || NS == 4, "window slots must divide a scale group");
    static_assert(!VR || R == 2, "register-fed vectors: two row tiles");
    constexpr int kRows = (R + (VR ? 0 : 1)) * kTile;    // staged rows: weight tiles, then vectors
    constexpr int kVecLoads = VR ? 3 : 0;                // per window: 2 code loads, 1 scale load
    constexpr int kWinSlot = kRows * (kWinElems / 2);    // 128 bytes per row and window
    constexpr int kScaleSlot = kRows * kGroupWins * 16;  // 64 bytes per row and group
    constexpr int kWinLoads = kRows / 8;                 // 1 KiB copies per window
    // scale copies per group: 16 rows x 64 bytes each when every scale row
    // and group start is 16-byte aligned (S16), else 4 rows x 64 bytes
    constexpr int kScaleLoads = S16 ? kRows / 16 : kRows / 4;
    constexpr int kWaveBytes = NS * kWinSlot + 2 * kScaleSlot;
    static_assert(NS * (kWinLoads + kVecLoads) + kScaleLoads <= 63, "loads in flight must fit the 6-bit vmcnt");
    __shared__ __attribute__((aligned(16))) uint8_t ring[W * kWaveBytes];
    __shared__ f32x4 red[(W > 1 ? W - 1 : 1) * R * kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int li = lane & (kTile - 1);
    const int kq = lane >> 4;

    const uint32_t gi = blockIdx.x;
    const uint32_t rbs = static_cast<uint32_t>(a.row_blocks), gs = static_cast<uint32_t>(a.groups);
    const uint32_t q = gi / rbs;
    const int64_t rb = gi - q * rbs;
    const int64_t grp = q % gs;
    const int64_t split = q / gs;

    int64_t v0, v1;
    vector_range<GROUPED>(a, grp, &v0, &v1);
    if (v1 <= v0) return;   // workgroup-uniform: an expert without tokens

    // K positions fit 32 bits (k <= 2^26).  The wave's windows: a contiguous
    // run [wbeg, wend) of the workgroup's, elements [kwb, kwe).
    const int64_t k = a.k;
    const uint32_t half = static_cast<uint32_t>(k / 2);
    const uint32_t sixteenth = static_cast<uint32_t>(k / 16);
    const int kb0 = static_cast<int>(split * a.kchunk);
    const int kend = static_cast<int>((k - kb0 < a.kchunk) ? k : kb0 + a.kchunk);
    const int nwin = (kend - kb0 + kWinElems - 1) / kWinElems;
    const int wbeg = wave * nwin / W, wend = (wave + 1) * nwin / W;
    const int niter = wend - wbeg;
    const int kwb = kb0 + wbeg * kWinElems;
    const int kwe = (kb0 + wend * kWinElems < kend) ? kb0 + wend * kWinElems : kend;

    const int64_t row0 = rb * a.rows_per_block;
    const int nrows = static_cast<int>((a.rows - row0 < a.rows_per_block) ? a.rows - row0 : a.rows_per_block);
    const __amdgpu_buffer_rsrc_t wdesc =
        buffer_of(a.W + (grp * a.rows + row0) * (k / 2), nrows * static_cast<int>(half));
    const __amdgpu_buffer_rsrc_t swdesc =
        buffer_of(a.sW + (grp * a.rows + row0) * (k / 16), nrows * static_cast<int>(sixteenth));
    const float al = group_alpha(a, grp, GROUPED);
    uint8_t *wring = ring + wave * kWaveBytes;      // NS window slots
    uint8_t *sring = wring + NS * kWinSlot;         // 2 scale slots

    // Copy lanes, per instruction: window copy n covers staged rows 8n ..
    // 8n+7 (lane l: row 8n + l/8, chunk at position l & 7); a 4-byte scale
    // copy s covers rows 4s .. 4s+3 (lane l: row 4s + l/16, word at position
    // l & 15), a 16-byte one rows 16s .. 16s+15 (lane l: row 16s + l/4, the
    // 4 words at positions 4 (l & 3) .. +3, one window's: scale_pos keeps a
    // window's 4 words together).
    // wbase/sbase: byte offsets without the window's or group's (rows past
    // the block out of range); wlo/slo: the element offset of the chunk in
    // its window, or of the word's window in its group.  Vector rows past the
    // pass read zeros through their descriptor.
    uint32_t wbase[kWinLoads], sbase[kScaleLoads];
    int wlo[kWinLoads], slo[kScaleLoads];
#pragma unroll
    for (int n = 0; n < kWinLoads; ++n) {
        const int rho = 8 * n + (lane >> 3);
        int c = 0;
        for (int t = 0; t < 8; ++t) if (chunk_pos(rho, t) == (lane & 7)) c = t;
        const bool vec = n >= 2 * R;
        const int row = vec ? rho - R * kTile : rho;
        wbase[n] = (vec || row < nrows) ? static_cast<uint32_t>(row) * half + 16u * c : kOutOfRange;
        wlo[n] = 32 * c;
    }
#pragma unroll
    for (int sI = 0; sI < kScaleLoads; ++sI) {
        const int rho = S16 ? 16 * sI + (lane >> 2) : 4 * sI + (lane >> 4);
        // the position map is its own inverse
        const int w = S16 ? scale_pos(rho, 4 * (lane & 3)) : scale_pos(rho, lane & 15);
        const bool vec = rho >= R * kTile;
        const int row = vec ? rho - R * kTile : rho;
        sbase[sI] = (vec || row < nrows) ? static_cast<uint32_t>(row) * sixteenth + 4u * w : kOutOfRange;
        slo[sI] = kWinElems * (w >> 2);
    }
    // Read lanes: row li of tile 0, chunks 2kq and 2kq + 1; the scale word of
    // row li for piece kq of window u of a group.
    const uint32_t rw0 = 128u * li + 16u * chunk_pos(li, 2 * kq);
    const uint32_t rw1 = 128u * li + 16u * chunk_pos(li, 2 * kq + 1);
    uint32_t rs[kGroupWins];
#pragma unroll
    for (int u = 0; u < kGroupWins; ++u) rs[u] = 64u * li + 4u * scale_pos(li, 4 * u + kq);
    const int lpiece = kLaneElems * kq;

    for (int64_t vp = v0; vp < v1; vp += kTile) {
        const int64_t nv = (v1 - vp < kTile) ? v1 - vp : kTile;
        const __amdgpu_buffer_rsrc_t vdesc =
            buffer_of(a.V + vp * (k / 2), static_cast<int>(nv * (k / 2)));
        const __amdgpu_buffer_rsrc_t svdesc =
            buffer_of(a.sV + vp * (k / 16), static_cast<int>(nv * (k / 16)));

        // Window j of the wave (and, when j starts a group, the group's
        // scales).  Offsets carry the out-of-range bit or-ed in: every
        // in-range offset is below 2^31, and adding a window offset to
        // kOutOfRange stays above it.
        u32x4 vreg[NS][2];
        uint32_t vsreg[NS];
        auto issue = [&](auto starts_group, int j, auto slotc) {
            constexpr int slot = decltype(slotc)::value;
            const int kw = kwb + j * kWinElems;   // past kwe for spare windows
            if constexpr (VR) {
                // this lane's 32 code bytes of vector li (bytes 32 kq .. +31 of
                // the window) and its scale word, from L2 into registers
                const uint32_t vo = static_cast<uint32_t>(li) * half + static_cast<uint32_t>(kw) / 2 +
                                    32u * kq;
                vreg[slot][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vdesc, vo, 0, 0));
                vreg[slot][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vdesc, vo + 16, 0, 0));
                vsreg[slot] = __builtin_amdgcn_raw_buffer_load_b32(
                    svdesc, static_cast<uint32_t>(li) * sixteenth + static_cast<uint32_t>(kw) / 16 + 4u * kq, 0, 0);
            }
            if constexpr (decltype(starts_group)::value) {
                const int sl = kwe - kw;          // elements of the group in range
                uint8_t *dst = sring + ((j / kGroupWins) & 1) * kScaleSlot;
#pragma unroll
                for (int sI = 0; sI < kScaleLoads; ++sI) {
                    const uint32_t o = (sbase[sI] + static_cast<uint32_t>(kw) / 16) |
                                       (slo[sI] < sl ? 0u : kOutOfRange);
                    const bool vrows = (S16 ? 16 : 4) * sI >= R * kTile;
                    if constexpr (S16)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrows ? svdesc : swdesc,
                                                                 (lds_void_t *)(dst + 1024 * sI), 16, o,
                                                                 0, 0, 0);
                    else
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrows ? svdesc : swdesc,
                                                                 (lds_void_t *)(dst + 256 * sI), 4, o,
                                                                 0, 0, 0);
                }
            }
            const int lim = kwe - kw;             // elements of this window in range
            uint8_t *dst = wring + slot * kWinSlot;
#pragma unroll
            for (int n = 0; n < kWinLoads; ++n) {
                const uint32_t o = (wbase[n] + static_cast<uint32_t>(kw) / 2) |
                                   (wlo[n] < lim ? 0u : kOutOfRange);
                if (n < 2 * R)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(wdesc, (lds_void_t *)(dst + 1024 * n), 16,
                                                             o, 0, 0, kNonTemporal);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(vdesc, (lds_void_t *)(dst + 1024 * n), 16,
                                                             o, 0, 0, 0);
            }
        };
        f32x4 acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        // Window j's operands, out of its slot (and register slot) into wq,
        // vq, ws, vs: the slot can be refilled once this returns.
        auto fetch = [&](int j, auto slotc, int u, u32x4 (&wq)[R][2], u32x4 (&vq)[2], uint32_t (&ws)[R],
                         uint32_t &vs) {
            constexpr int slot = decltype(slotc)::value;
            const uint8_t *win = wring + slot * kWinSlot;
            const uint8_t *sc = sring + ((j / kGroupWins) & 1) * kScaleSlot;
            if constexpr (VR) {
                lds_read_weights<R>(lds_address(win + rw0), lds_address(win + rw1), lds_address(sc + rs[u]),
                                    wq, ws);
                vq[0] = vreg[slot][0];
                vq[1] = vreg[slot][1];
                vs = vsreg[slot];
            } else {
                lds_read_window<R>(lds_address(win + rw0), lds_address(win + rw1), lds_address(sc + rs[u]),
                                   wq, vq, ws, vs);
            }
            // a lane piece past the wave's K range: zero scales (its codes are
            // zeros or stale)
            const uint32_t keep = lpiece < kwe - (kwb + j * kWinElems) ? ~0u : 0u;
            vs &= keep;
#pragma unroll
            for (int r = 0; r < R; ++r) ws[r] &= keep;
        };
        // The window's decode and products.
        auto compute = [&](const u32x4 (&wq)[R][2], const u32x4 (&vq)[2], const uint32_t (&ws)[R],
                           uint32_t vs) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f16x8 vo[4];
                decode32(vq[h], vs >> (16 * h), vo);
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    f16x8 wo[4];
                    decode32(wq[r][h], ws[r] >> (16 * h), wo);
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        if (GROUPED)
                            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vo[s4], wo[s4], acc[r], 0,
                                                                            0, 0);
                        else
                            acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wo[s4], vo[s4], acc[r], 0,
                                                                            0, 0);
                    }
                }
            }
        };

        // One step at position u of group g: take window j out of its slot,
        // decode and multiply it, refill the slot with window j + NS (spare
        // windows past the run read nothing), wait until window j + 1 has
        // landed.  EARLY refills the slot as soon as the window's operands
        // are in registers, so the refill flies while they are decoded and
        // multiplied.  With two windows in flight and four waves that pays
        // (on a 7168 x 16384 weight: 4 vectors in registers 15.5 -> 14.6 us,
        // 16 vectors all in LDS 16.8 -> 15.5); with four windows in flight,
        // eight waves, or several workgroups per compute unit it was slower.
        auto step = [&](int g, auto pos) {
            constexpr int u = decltype(pos)::value;
            const int j = g * kGroupWins + u;
            constexpr auto slot = std::integral_constant<int, u % NS>{};
            constexpr auto starts = std::integral_constant<bool, (u + NS) % kGroupWins == 0>{};
            u32x4 wq[R][2], vq[2];
            uint32_t ws[R], vs;
            if (j < niter) {   // wave-uniform
                fetch(j, slot, u, wq, vq, ws, vs);
                if constexpr (!EARLY) compute(wq, vq, ws, vs);
            }
            phase_fence();
            issue(starts, j + NS, slot);
            phase_fence();
            if constexpr (EARLY) {
                if (j < niter) compute(wq, vq, ws, vs);
                phase_fence();
            }
            wait_vmcnt<loads_after_next<NS, kWinLoads + kVecLoads, kScaleLoads>(u)>();
            phase_fence();
        };
        if (niter > 0) {   // wave-uniform
            phase_fence();
            issue(std::true_type{}, 0, std::integral_constant<int, 0>{});
            phase_fence();
            if constexpr (NS == 4) {
                issue(std::false_type{}, 1, std::integral_constant<int, 1>{});
                phase_fence();
                issue(std::false_type{}, 2, std::integral_constant<int, 2>{});
                phase_fence();
                issue(std::false_type{}, 3, std::integral_constant<int, 3>{});
            } else {
                issue(std::false_type{}, 1, std::integral_constant<int, 1>{});
            }
            phase_fence();
            wait_vmcnt<(NS - 1) * (kWinLoads + kVecLoads)>();   // window 0 landed
            phase_fence();
            for (int g = 0; g * kGroupWins < niter; ++g) {
                step(g, std::integral_constant<int, 0>{});
                step(g, std::integral_constant<int, 1>{});
                step(g, std::integral_constant<int, 2>{});
                step(g, std::integral_constant<int, 3>{});
            }
            wait_vmcnt<0>();
            phase_fence();
        }

        if (W > 1) {
            if (wave > 0) {
#pragma unroll
                for (int r = 0; r < R; ++r) red[((wave - 1) * R + r) * kWave + lane] = acc[r];
            }
            __syncthreads();
        }
        if (wave == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                f32x4 s = acc[r];
                for (int w = 1; w < W; ++w) s += red[((w - 1) * R + r) * kWave + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (GROUPED) {
                        const int64_t t = vp + kq * 4 + e;
                        const int rr = r * kTile + li;
                        if (t < v1 && rr < nrows)
                            a.c[t * a.rows + row0 + rr] = round_out(al, s[e], a.out_bf16);
                    } else {
                        const int rr = r * kTile + kq * 4 + e;
                        const int64_t col = vp - v0 + li;
                        if (rr < nrows && col < a.nvec) {
                            const int64_t o = (grp * a.rows + row0 + rr) * a.nvec + col;
                            if (a.part != nullptr)
                                a.part[split * a.groups * a.rows * a.nvec + o] = s[e];
                            else
                                a.c[o] = round_out(al, s[e], a.out_bf16);
                        }
                    }
                }
            }
        }
        if (W > 1 && vp + kTile < v1) __syncthreads();   // before the next pass reuses `red`
    }
}

// ---------------------------------------------------------------- VALU row tiles
// For few vectors per weight matrix (small-N GEMM with n <= 4, experts with a
// handful of tokens) the products fit the VALU, and the weights are better
// read row-contiguously than in the 16-rows x 64-bytes pattern the matrix
// cores want.  A workgroup owns a tile of TR weight rows of one group; its W
// waves take K slices of 2048 elements (1 KiB of every row) in turn.  The
// group's vectors are taken in passes of up to T: for one slice a wave loads
// the pass's vectors (16 bytes and a scale pair per lane each, cached: every
// workgroup of the group reads them) and then one 16-byte non-temporal load
// per lane for each of the TR rows, back to back; decodes each vector once to
// fp16 (e2m1 * e4m3, exact), each row's codes once, and takes the T dot
// products of the row with v_dot2_f32_f16, scaling each 16-element block sum
// by its weight scale in fp32.  Vectors past the pass's count read zeros
// and are skipped (wave-uniform).  Per pass, the TR x T per-lane sums are
// halved across the 32-lane halves and the 16-lane rows of the wave, summed
// inside each 16-lane row by DPP, and the waves' sums meet in LDS in wave
// order.  More than T vectors mean another pass over the tile's rows.
template <int TR, int T, int W, bool GROUPED>
__global__ void __launch_bounds__(W * kWave) vec_tile(const MmaArgs a) {
    constexpr int NV = TR * T;   // sums per pass
    static_assert(NV >= 4 && (NV & (NV - 1)) == 0, "TR * T: a power of two, at least 4");
    constexpr int H = NV / 2, Q = NV / 4;
    __shared__ float red[W * NV];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

    // the plan keeps the workgroup count below 2^31: 32-bit division
    const uint32_t gi = blockIdx.x;
    const uint32_t rbs = static_cast<uint32_t>(a.row_blocks);
    const uint32_t grp32 = gi / rbs;
    const int64_t rb = gi - grp32 * rbs;
    const int64_t grp = grp32;

    int64_t v0, v1;
    vector_range<GROUPED>(a, grp, &v0, &v1);
    if (v1 <= v0) return;   // workgroup-uniform: an expert without tokens

    const int64_t k = a.k;
    const uint32_t half = static_cast<uint32_t>(k / 2);
    const uint32_t sixteenth = static_cast<uint32_t>(k / 16);
    const int nsl = static_cast<int>((k + kSliceElems - 1) / kSliceElems);
    const int64_t row0 = rb * a.rows_per_block;
    const int nrows = static_cast<int>((a.rows - row0 < a.rows_per_block) ? a.rows - row0
                                                                           : a.rows_per_block);
    const __amdgpu_buffer_rsrc_t wdesc =
        buffer_of(a.W + (grp * a.rows + row0) * (k / 2), nrows * static_cast<int>(half));
    const __amdgpu_buffer_rsrc_t swdesc =
        buffer_of(a.sW + (grp * a.rows + row0) * (k / 16), nrows * static_cast<int>(sixteenth));
    const float al = group_alpha(a, grp, GROUPED);

    for (int64_t vp = v0; vp < v1; vp += T) {
        const int nv = static_cast<int>((v1 - vp < T) ? v1 - vp : T);
        const __amdgpu_buffer_rsrc_t vdesc =
            buffer_of(a.V + vp * (k / 2), nv * static_cast<int>(half));
        const __amdgpu_buffer_rsrc_t svdesc =
            buffer_of(a.sV + vp * (k / 16), nv * static_cast<int>(sixteenth));

        float acc[TR][T];
#pragma unroll
        for (int r = 0; r < TR; ++r)
#pragma unroll
            for (int j = 0; j < T; ++j) acc[r][j] = 0.0f;

        for (int sl = wave; sl < nsl; sl += W) {
            const int64_t e0 = static_cast<int64_t>(sl) * kSliceElems + 32 * lane;
            const uint32_t lo = e0 < k ? static_cast<uint32_t>(e0 / 2) : kOutOfRange;
            const uint32_t lso = e0 < k ? static_cast<uint32_t>(e0 / 16) : kOutOfRange;

            phase_fence();
            u32x4 xv[T];
            uint32_t xs[T];
#pragma unroll
            for (int j = 0; j < T; ++j) {
                xv[j] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(vdesc, lo + j * half, 0, 0));
                xs[j] = __builtin_amdgcn_raw_buffer_load_b16(svdesc, lso + j * sixteenth, 0, 0);
            }
            u32x4 av[TR];
            uint32_t sv[TR];
#pragma unroll
            for (int r = 0; r < TR; ++r) {
                av[r] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(wdesc, lo + r * half, 0, kNonTemporal));
                sv[r] = __builtin_amdgcn_raw_buffer_load_b16(swdesc, lso + r * sixteenth, 0,
                                                             kNonTemporal);
                phase_fence();   // row by row, in the order the rows are consumed
            }

            u32x4 xq[T][4];   // x~ pairs: xq[j][i / 4][i % 4] holds elements 2i, 2i + 1
#pragma unroll
            for (int j = 0; j < T; ++j) {
                f16x8 o[4];
                decode32(xv[j], xs[j], o);
#pragma unroll
                for (int q = 0; q < 4; ++q) xq[j][q] = __builtin_bit_cast(u32x4, o[q]);
            }
#pragma unroll
            for (int r = 0; r < TR; ++r) {
                const uint32_t aw[4] = {av[r].x, av[r].y, av[r].z, av[r].w};
                f16x2 ad[16];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    ad[4 * q + 0] = e2m1x2_f16<0>(aw[q]);
                    ad[4 * q + 1] = e2m1x2_f16<1>(aw[q]);
                    ad[4 * q + 2] = e2m1x2_f16<2>(aw[q]);
                    ad[4 * q + 3] = e2m1x2_f16<3>(aw[q]);
                }
                const f32x2 sa = e4m3x2_f32(sv[r]);
#pragma unroll
                for (int j = 0; j < T; ++j) {
                    if (j < nv) {   // wave-uniform
                        float b0 = 0.0f, b1 = 0.0f;
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            b0 = __builtin_amdgcn_fdot2(ad[i], halves(xq[j][i / 4][i % 4]), b0, false);
#pragma unroll
                        for (int i = 8; i < 16; ++i)
                            b1 = __builtin_amdgcn_fdot2(ad[i], halves(xq[j][i / 4][i % 4]), b1, false);
                        acc[r][j] = __builtin_fmaf(b0, sa.x, acc[r][j]);
                        acc[r][j] = __builtin_fmaf(b1, sa.y, acc[r][j]);
                    }
                }
            }
        }

        // Sum i = r * T + j.  Halve across the 32-lane halves (the low half
        // keeps sums 0 .. H - 1), then across 16-lane rows (even rows keep
        // 0 .. Q - 1 of their half's), then inside each 16-lane row.
        float h2[H];
#pragma unroll
        for (int i = 0; i < H; ++i) {
            const auto t = __builtin_amdgcn_permlane32_swap(
                __builtin_bit_cast(unsigned, acc[i / T][i % T]),
                __builtin_bit_cast(unsigned, acc[(i + H) / T][(i + H) % T]), false, false);
            h2[i] = __builtin_bit_cast(float, static_cast<unsigned>(t[0])) +
                    __builtin_bit_cast(float, static_cast<unsigned>(t[1]));
        }
        float h4[Q];
#pragma unroll
        for (int i = 0; i < Q; ++i) {
            const auto t = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, h2[i]),
                                                            __builtin_bit_cast(unsigned, h2[i + Q]),
                                                            false, false);
            h4[i] = __builtin_bit_cast(float, static_cast<unsigned>(t[0])) +
                    __builtin_bit_cast(float, static_cast<unsigned>(t[1]));
        }
#pragma unroll
        for (int i = 0; i < Q; ++i) {
            float v = h4[i];
            v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
            v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
            v += dpp<0x141>(v);   // row_half_mirror
            v += dpp<0x140>(v);   // row_mirror
            h4[i] = v;
        }
        // Lane jj < Q of 16-lane row q holds sum jj + Q (q & 1) + H (q >> 1).
        const int jj = lane & 15, q = lane >> 4;
        if (jj < Q) {
            float v = h4[0];
#pragma unroll
            for (int i = 1; i < Q; ++i)
                if (jj == i) v = h4[i];
            red[wave * NV + jj + Q * (q & 1) + H * (q >> 1)] = v;
        }
        __syncthreads();
        if (wave == 0 && lane < NV) {
            const int r = lane / T, j = lane % T;
            float v = red[lane];
#pragma unroll
            for (int w = 1; w < W; ++w) v += red[w * NV + lane];
            if (r < nrows && j < nv) {
                if (GROUPED)
                    a.c[(vp + j) * a.rows + row0 + r] = round_out(al, v, a.out_bf16);
                else
                    a.c[(grp * a.rows + row0 + r) * a.nvec + (vp - v0 + j)] =
                        round_out(al, v, a.out_bf16);
            }
        }
        if (vp + T < v1) __syncthreads();   // before the next pass reuses `red`
    }
}

// ---------------------------------------------------------------- weight packing
// W [groups][rows][k/2] and sW [groups][rows][k/16] -> the packed layout:
// for tile t (rows 16t .. 16t+15 of a group) and window w (elements 256w ..
// 256w+255), chunk h (0, 1) of lane l = i + 16q holds bytes 128w + 32q + 16h
// .. +15 of row 16t + i, at ((t * windows + w) * 2 + h) * 1024 + 16 l; its
// scale word holds scale bytes 16w + 4q .. +3 of the same row, at
// (t * windows + w) * 256 + 4 l.  Rows past `rows` and elements past k are
// zero.  One thread per 16-byte chunk of codes (and per 4-byte scale word).
__global__ void __launch_bounds__(kPackThreads)
mma_pack_weight(const uint8_t *__restrict__ W, const uint8_t *__restrict__ sW,
                uint8_t *__restrict__ Wp, uint8_t *__restrict__ sWp, int64_t groups,
                int64_t rows, int64_t k) {
    const int64_t wins = (k + kWinElems - 1) / kWinElems;
    const int64_t tiles = (rows + kTile - 1) / kTile;
    const int64_t chunks = groups * tiles * wins * (kPackedWinBytes / 16);
    const int64_t c = static_cast<int64_t>(blockIdx.x) * kPackThreads + threadIdx.x;
    if (c >= chunks) return;
    const int lane = static_cast<int>(c % kWave);
    const int h = static_cast<int>((c / kWave) % 2);
    const int64_t tw = c / (2 * kWave);                // (group, tile, window)
    const int64_t w = tw % wins;
    const int64_t gt = tw / wins;                      // group * tiles + tile
    const int64_t g = gt / tiles, t = gt % tiles;
    const int64_t row = t * kTile + (lane & (kTile - 1));
    const int q = lane >> 4;
    const int64_t byte = w * (kWinElems / 2) + 32 * q + 16 * h;   // within the row's k/2 codes
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < rows && byte < k / 2)
        v = *reinterpret_cast<const u32x4 *>(W + (g * rows + row) * (k / 2) + byte);
    *reinterpret_cast<u32x4 *>(Wp + c * 16) = v;
    if (h == 0) {
        const int64_t sbyte = w * (kWinElems / 16) + 4 * q;
        uint32_t sv = 0u;
        if (row < rows && sbyte < k / 16)
            sv = *reinterpret_cast<const uint32_t *>(sW + (g * rows + row) * (k / 16) + sbyte);
        *reinterpret_cast<uint32_t *>(sWp + tw * kPackedWinScaleBytes + 4 * lane) = sv;
    }
}

// ---------------------------------------------------------------- generic kernel
// Any k % 16 == 0 and any byte alignment.  One wave per (group, weight row);
// lanes take 16-element blocks; bytes are loaded singly; vectors one by one.
__device__ __forceinline__ uint32_t load_u32_bytes(const uint8_t *p) {
    return static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[1]) << 8) |
           (static_cast<uint32_t>(p[2]) << 16) | (static_cast<uint32_t>(p[3]) << 24);
}

__device__ __forceinline__ float dot8_codes(uint32_t a, uint32_t v, float acc) {
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<0>(a), e2m1x2_f16<0>(v), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<1>(a), e2m1x2_f16<1>(v), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<2>(a), e2m1x2_f16<2>(v), acc, false);
    acc = __builtin_amdgcn_fdot2(e2m1x2_f16<3>(a), e2m1x2_f16<3>(v), acc, false);
    return acc;
}

template <bool GROUPED>
__global__ void __launch_bounds__(kGenericWaves * kWave) mma_generic(const MmaArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint32_t rbs = static_cast<uint32_t>(a.row_blocks);
    const int64_t rb = blockIdx.x % rbs;
    const int64_t grp = blockIdx.x / rbs;
    const int64_t row = rb * kGenericWaves + wave;
    if (row >= a.rows) return;
    int64_t v0, v1;
    vector_range<GROUPED>(a, grp, &v0, &v1);
    const int64_t k = a.k;
    const uint8_t *wrow = a.W + (grp * a.rows + row) * (k / 2);
    const uint8_t *swrow = a.sW + (grp * a.rows + row) * (k / 16);
    const float al = group_alpha(a, grp, GROUPED);
    for (int64_t v = v0; v < v1; ++v) {
        const uint8_t *vrow = a.V + v * (k / 2);
        const uint8_t *svrow = a.sV + v * (k / 16);
        float acc = 0.0f;
        for (int64_t blk = lane; blk < k / 16; blk += kWave) {
            float bs = dot8_codes(load_u32_bytes(wrow + blk * 8), load_u32_bytes(vrow + blk * 8), 0.0f);
            bs = dot8_codes(load_u32_bytes(wrow + blk * 8 + 4), load_u32_bytes(vrow + blk * 8 + 4), bs);
            // sW * sV is exact in fp32 (4 + 4 significant bits)
            const float sc = e4m3x2_f32(swrow[blk]).x * e4m3x2_f32(svrow[blk]).x;
            acc = __builtin_fmaf(bs, sc, acc);
        }
        const float s = wave_sum(acc);
        if (lane == 0) {
            if (GROUPED) {
                a.c[v * a.rows + row] = round_out(al, s, a.out_bf16);
            } else {
                a.c[(grp * a.rows + row) * a.nvec + (v - v0)] = round_out(al, s, a.out_bf16);
            }
        }
    }
}

// ---------------------------------------------------------------- split-K second pass
// c[i] = out(alpha[i / per_group] * (((0 + p[0][i]) + p[1][i]) + ...)).
__global__ void __launch_bounds__(kReduceThreads)
mma_splitk_reduce(const float *__restrict__ part, const float *__restrict__ alpha,
                  uint16_t *__restrict__ c, int64_t total, int64_t per_group, int64_t ksplit,
                  int32_t out_bf16) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kReduceThreads + threadIdx.x;
    if (i >= total) return;
    float s = 0.0f;
    for (int64_t j = 0; j < ksplit; ++j) s += part[j * total + i];
    const float al = alpha ? alpha[i / per_group] : 1.0f;
    c[i] = round_out(al, s, out_bf16);
}

}  // namespace

#endif  // NVFP4_MMA_KERNELS_H
