/*
 * nvfp4_mma.h - C ABI of two MI355X (gfx950) NVFP4 block-scaled products of a
 * weight matrix with several vectors: the small-N GEMM and the grouped (MoE)
 * GEMV.  Both use the scaled dot product of nvfp4_gemv.h (16 consecutive K
 * elements share one E4M3 scale, E2M1 codes packed two per byte with element
 * 2i in bits 3:0, sign in bit 3 of a code), accumulate in fp32 and round the
 * product with the global scale to fp16 or bf16 (round to nearest even).
 *
 * Small-N GEMM.  The blog post "nvFP4 Batch GEMV算子系列(下)" (section
 * "pytorch实现NVFP4 batch gemv") computes its batched GEMV as a scaled matrix
 * product whose N dimension is padded for the library call; here N = n
 * vectors are used as they are:
 *
 *   S[b,r,j] = sum_kk e2m1(A[b,r,kk]) e4m3(sfA[b,r,kk/16]) e2m1(B[b,j,kk]) e4m3(sfB[b,j,kk/16])
 *   c[b,r,j] = out( f32( alpha[b] * S[b,r,j] ) )
 *
 * for b < l, r < m, j < n, with
 *   A_packed uint8 [l][m][k/2], sfA uint8 [l][m][k/16],
 *   B_packed uint8 [l][n][k/2], sfB uint8 [l][n][k/16],
 *   alpha    float [l] or NULL (1), c uint16 [l][m][n] (fp16 or bf16 bits).
 *
 * Grouped GEMV.  The CuTeDSL bridge page (sections "Tensor Layout
 * Conversion" and "Kernel Launch") runs a 2D x 3D grouped GEMM: token rows
 * sorted by expert, one weight matrix per expert, cumulative token offsets per
 * expert and one fp32 global scale per expert for each operand.  Token t with
 * offsets[e-1] <= t < offsets[e] (offsets[-1] = 0) belongs to expert e and
 *
 *   S[t,r]  = sum_kk e2m1(X[t,kk]) e4m3(sfX[t,kk/16]) e2m1(W[e,r,kk]) e4m3(sfW[e,r,kk/16])
 *   c[t,r]  = out( f32( f32(gs_x[e] * gs_w[e]) * S[t,r] ) )
 *
 * for r < n, with
 *   X_packed uint8 [tokens][k/2], sfX uint8 [tokens][k/16],
 *   W_packed uint8 [experts][n][k/2], sfW uint8 [experts][n][k/16],
 *   offsets  int32 [experts] cumulative token counts (non-decreasing, at most
 *            `tokens`), gs_x, gs_w float [experts] or NULL (1),
 *   c        uint16 [tokens][n] (fp16 or bf16 bits).
 * Rows of c whose token belongs to no expert (t >= offsets[experts-1]) are
 * left untouched.  The offsets live on the device and are never read by the
 * host; the kernels clamp them to [0, tokens], so any values are memory-safe,
 * but token ranges that overlap (decreasing offsets) give unspecified values
 * in the overlapping rows.
 *
 * out_type: NVFP4_OUT_F16 (the blog post's output type) or NVFP4_OUT_BF16
 * (the bridge page's).  Accumulation order inside the fp32 sums is not fixed;
 * with the integer-coded inputs every partial sum is exact, so results are
 * bit-identical to the exact values rounded as above.
 *
 * All data pointers are DEVICE pointers owned by the caller; the library never
 * keeps them after the enqueued work.  `stream` is a hipStream_t (NULL = the
 * default stream).  Calls only enqueue work: no device synchronisation, no
 * host read of device memory.  Shape rules: every dimension >= 1 (tokens may
 * be 0 for the grouped call), k >= 16, k % 16 == 0, byte sizes within int64,
 * and the output count below 2^31.  The fast kernels need k % 64 == 0,
 * k <= 2^26, 16-byte aligned packed operands and 4-byte aligned scales; other
 * valid calls take a slower generic kernel with the same results.  Every
 * argument is checked before any HIP call; invalid calls return a negative status of
 * nvfp4_gemv.h and enqueue nothing.  No C++ exception crosses this interface.
 */
#ifndef NVFP4_MMA_H
#define NVFP4_MMA_H

#include <stddef.h>
#include <stdint.h>

#include "nvfp4_gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_OUT_F16 0
#define NVFP4_OUT_BF16 1

/* Launch-plan control of the small-N and grouped kernels (tests and sweeps). */
typedef struct nvfp4_mma_tuning_t {
    int32_t path;           /* NVFP4_GEMV_PATH_* of nvfp4_gemv.h                        */
    int32_t variant;        /* fast-kernel variant, 0 = default, 1..nvfp4_mma_num_variants() */
    int32_t ksplit;         /* K split across workgroups, 0 = default, >= 1 explicit;
                               the grouped GEMV takes 0 or 1 only                     */
    int32_t rows_per_block; /* weight rows per workgroup, 0 = default, 1 .. 16 x the
                               variant's row tiles per wave (VALU row tiles: 1 .. the
                               tile's rows)                                            */
} nvfp4_mma_tuning_t;

/*
 * The small-N GEMM above.  When the plan splits K across workgroups the fp32
 * partial sums go to the library-owned per-(device, stream) workspace of
 * nvfp4_gemv_launch (grown on first need without synchronising, kept until
 * the process ends; a call that must grow it while `stream` is being captured
 * returns WORKSPACE: see nvfp4_workspace_reserve).
 * Returns NVFP4_GEMV_OK or a negative status (BAD_ARGUMENT for an unknown
 * out_type).
 */
int nvfp4_gemm_smalln_launch(const uint8_t *A_packed, const uint8_t *sfA,
                             const uint8_t *B_packed, const uint8_t *sfB,
                             const float *alpha, uint16_t *c,
                             int64_t l, int64_t m, int64_t n, int64_t k,
                             int32_t out_type, void *stream);

#define NVFP4_MMA_FORM_MATRIX_CORES 0
#define NVFP4_MMA_FORM_VALU_TILES 1
#define NVFP4_MMA_FORM_LDS_STAGED 2
#define NVFP4_MMA_FORM_LDS_VECTOR_REGS 3

/*
 * Number of fast small-N / grouped kernel variants, and the shape of variant
 * v (1-based).  Its form (nvfp4_mma_variant_form) says how the three numbers
 * read:
 *  - NVFP4_MMA_FORM_MATRIX_CORES: MFMA row tiles of 16 weight rows per wave,
 *    K windows of 256 elements (128 bytes of every row) kept in flight per
 *    wave, waves per workgroup (each wave takes every waves-th window of the
 *    workgroup's K range);
 *  - NVFP4_MMA_FORM_VALU_TILES: weight rows per workgroup tile, vectors per
 *    pass over the tile, waves per workgroup (each wave takes every waves-th
 *    K slice of 2048 elements, 1 KiB of every row per load).  The products
 *    run on the VALU; more vectors than one pass holds mean another pass over
 *    the tile's rows.  These variants never split K: an explicit ksplit above
 *    1 or rows_per_block above the tile's rows is BAD_TUNING;
 *  - NVFP4_MMA_FORM_LDS_STAGED: the matrix-core products with every operand
 *    (weight and vector codes per window, block scales per 4 windows) copied
 *    into LDS by whole-line direct-to-LDS loads and read back in the
 *    matrix-core lane order; the numbers are row tiles per wave, windows in
 *    flight and waves (each wave takes a contiguous run of the workgroup's
 *    windows, so on inexact data the fp32 sums may round differently from a
 *    MATRIX_CORES variant).  Row-major weights only: with packed weights
 *    these variants are BAD_TUNING;
 *  - NVFP4_MMA_FORM_LDS_VECTOR_REGS: as LDS_STAGED for the weight codes and
 *    scales, while every lane loads its own vector codes and scale word from
 *    L2 straight into registers (less LDS per workgroup, more workgroups per
 *    compute unit; it pays while there are few vectors).  Row-major weights
 *    only.
 * Each returns a status (BAD_TUNING for v outside 1 .. num_variants,
 * NULL_POINTER for a NULL output).
 */
int nvfp4_mma_num_variants(void);
int nvfp4_mma_variant_info(int v, int32_t *row_tiles_per_wave, int32_t *windows_in_flight,
                           int32_t *waves_per_group);
int nvfp4_mma_variant_form(int v, int32_t *form);

/*
 * The small-N plan the library would use (path, variant, K split, rows per
 * workgroup; the last three 0 for the generic kernel) and the workspace it
 * needs, as nvfp4_gemv_plan does for the GEMV; `in` may be NULL.  `aligned`
 * says whether the pointers meet the fast kernels' alignment rules.  Returns
 * a status (BAD_SHAPE as the launch would, BAD_TUNING, NULL_POINTER).
 */
int nvfp4_gemm_smalln_plan(int64_t l, int64_t m, int64_t n, int64_t k, int aligned,
                           const nvfp4_mma_tuning_t *in, nvfp4_mma_tuning_t *out,
                           size_t *workspace_bytes);

/*
 * The small-N GEMM with an explicit plan (`tuning` may be NULL) and a
 * caller-owned workspace of at least the bytes nvfp4_gemm_smalln_plan reports
 * (4-byte aligned; may be NULL when that is 0).  Allocates nothing.
 */
int nvfp4_gemm_smalln_launch_tuned(const uint8_t *A_packed, const uint8_t *sfA,
                                   const uint8_t *B_packed, const uint8_t *sfB,
                                   const float *alpha, uint16_t *c,
                                   int64_t l, int64_t m, int64_t n, int64_t k,
                                   int32_t out_type, const nvfp4_mma_tuning_t *tuning,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * The grouped plan the library would use (path, variant, K split (always 1),
 * rows per workgroup; the last three 0 for the generic kernel) for `experts`
 * weight matrices of n x k and `tokens` routed tokens (the launch's count:
 * the default variant depends on the tokens per expert), as
 * nvfp4_gemm_smalln_plan does for the small-N GEMM; `in` may be NULL.  `packed` != 0 asks for the plan of the packed-weight
 * launch (then `aligned` is ignored: packed operands are aligned by
 * definition), else `aligned` says whether the pointers meet the fast
 * kernels' alignment rules.  Returns a status (BAD_SHAPE as the matching
 * launch would, BAD_TUNING, NULL_POINTER for a NULL out).
 */
int nvfp4_grouped_gemv_plan(int64_t experts, int64_t n, int64_t k, int64_t tokens, int aligned,
                            int packed, const nvfp4_mma_tuning_t *in, nvfp4_mma_tuning_t *out);

/*
 * The grouped (MoE) GEMV above.  Never splits K and needs no workspace.
 * Returns NVFP4_GEMV_OK or a negative status.
 */
int nvfp4_grouped_gemv_launch(const uint8_t *X_packed, const uint8_t *sfX,
                              const uint8_t *W_packed, const uint8_t *sfW,
                              const int32_t *offsets, const float *gs_x, const float *gs_w,
                              uint16_t *c, int64_t tokens, int64_t experts, int64_t n, int64_t k,
                              int32_t out_type, void *stream);

/*
 * The grouped GEMV with an explicit kernel choice (`tuning` may be NULL;
 * its ksplit must be 0 or 1).
 */
int nvfp4_grouped_gemv_launch_tuned(const uint8_t *X_packed, const uint8_t *sfX,
                                    const uint8_t *W_packed, const uint8_t *sfW,
                                    const int32_t *offsets, const float *gs_x,
                                    const float *gs_w, uint16_t *c, int64_t tokens,
                                    int64_t experts, int64_t n, int64_t k, int32_t out_type,
                                    const nvfp4_mma_tuning_t *tuning, void *stream);

/*
 * Packed weights.  The matrix cores take a weight tile as 16 rows x 32 K
 * elements spread over the 16-lane groups of a wave, so read from the
 * row-major layout each load instruction covers 16 rows x 64 bytes.  Weights
 * are static in inference, so they can be re-laid out once, offline, in the
 * order the kernel's lanes read them; every load instruction then reads 1 KiB
 * of contiguous memory.  This is the same idea as the pages' 128 x 4 scale
 * swizzle for the library GEMM ("nvFP4 Batch GEMV算子系列(下)", section
 * "关键的to_blocked函数理解"), applied to the codes and scales of the weight.
 *
 * Layout, for `groups` matrices of rows x k (codes [groups][rows][k/2],
 * scales [groups][rows][k/16] as above): tile t holds rows 16t .. 16t+15 and
 * window w holds elements 256w .. 256w+255.  With T = ceil(rows/16) tiles
 * and Wn = ceil(k/256) windows per tile, block b = (g T + t) Wn + w is 2048
 * code bytes at 2048 b and 256 scale bytes at 256 b.  In a block, lane
 * l = i + 16 q (i < 16, q < 4) owns
 *   code bytes 16 l and 1024 + 16 l: bytes 128 w + 32 q .. +15 and
 *     128 w + 32 q + 16 .. +15 of row 16t + i's codes;
 *   scale bytes 4 l .. 4 l + 3: bytes 16 w + 4 q .. +3 of row 16t + i's scales.
 * Rows past `rows` and elements past k are zero.
 *
 * nvfp4_mma_packed_sizes: bytes of the packed codes and scales (NVFP4_GEMV_OK,
 * or BAD_SHAPE unless k % 64 == 0, k <= 2^26 and the sizes fit).
 *
 * nvfp4_mma_pack_weight: writes that layout from W / sW to W_packed /
 * sW_packed (device buffers of those sizes; codes 16-byte aligned, scales
 * 4-byte aligned, no overlap with the inputs or each other).  One kernel on
 * `stream`; nothing is allocated.
 *
 * nvfp4_gemm_smalln_launch_packed / nvfp4_grouped_gemv_launch_packed: the
 * small-N GEMM and the grouped GEMV above, with the weights in the packed
 * layout and the vectors (B, X) as before.  Results are bit-identical to the
 * row-major calls with the same plan.  `tuning` may be NULL; it selects a
 * matrix-core variant (a VALU row-tile variant is BAD_TUNING), a K split
 * (small-N only; splits fall on window boundaries) and rows_per_block, which
 * must be a multiple of 16 (0 = the variant's tiles).  The shape and
 * alignment rules are the fast kernels' (k % 64 == 0, k <= 2^26, 16-byte
 * codes, 4-byte scales): there is no generic path for packed weights, so
 * other shapes are BAD_SHAPE and misaligned pointers ALIGNMENT.  The small-N
 * call takes its split-K partials from the library's per-(device, stream)
 * workspace, as nvfp4_gemm_smalln_launch does.
 */
int nvfp4_mma_packed_sizes(int64_t groups, int64_t rows, int64_t k, size_t *codes_bytes,
                           size_t *scales_bytes);
int nvfp4_mma_pack_weight(const uint8_t *W, const uint8_t *sW, int64_t groups, int64_t rows,
                          int64_t k, uint8_t *W_packed, uint8_t *sW_packed, void *stream);
int nvfp4_gemm_smalln_launch_packed(const uint8_t *A_packed, const uint8_t *sfA_packed,
                                    const uint8_t *B_packed, const uint8_t *sfB,
                                    const float *alpha, uint16_t *c, int64_t l, int64_t m,
                                    int64_t n, int64_t k, int32_t out_type,
                                    const nvfp4_mma_tuning_t *tuning, void *stream);
int nvfp4_grouped_gemv_launch_packed(const uint8_t *X_packed, const uint8_t *sfX,
                                     const uint8_t *W_packed, const uint8_t *sfW_packed,
                                     const int32_t *offsets, const float *gs_x, const float *gs_w,
                                     uint16_t *c, int64_t tokens, int64_t experts, int64_t n,
                                     int64_t k, int32_t out_type, const nvfp4_mma_tuning_t *tuning,
                                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_MMA_H */
