/*
 * nvfp4_quantize.h - C ABI of the MI355X (gfx950) BF16 -> NVFP4 activation
 * quantiser, and of the GEMV fed by a bf16 activation.
 *
 * Operation (the graph-safe activation quantiser of the CuTeDSL NVFP4 bridge
 * page, section "Quantization"; its global scale is precomputed by the caller
 * instead of taken from the tensor's amax, so no host synchronisation is
 * needed).  For each row r and each block of 16 consecutive elements, in fp32
 * with IEEE round-to-nearest-even:
 *
 *   xn   = x / g[r]
 *   am   = max(max |xn| over the block, 1e-8)
 *   s    = float8_e4m3fn(am / 6)        round to nearest even; from 464 up the
 *                                       result is the NaN pattern 0x7F
 *   v    = xn / max(value(s), 1e-8)
 *   code = E2M1 magnitude index of |v| under `rule`, plus 8 when v < 0
 *          (-0 and NaN are not < 0); a NaN v gets code 0
 *
 * Rounding rules (E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6):
 *   NVFP4_ROUND_HALF_STEP     the page's activation quantiser: |v| clamped to 6,
 *                             doubled, rounded to an integer (ties to even), then
 *                             the half-step table 0,1,2,3,4,4,5,5,6,6,6,7,7
 *   NVFP4_ROUND_NEAREST_EVEN  nearest magnitude, ties to the even code
 *   NVFP4_ROUND_NEAREST_LOWER the page's weight quantiser: argmin of the fp32
 *                             distances | |v| - magnitude |, first index on ties
 *
 * Layout (row-major, contiguous, device memory owned by the caller):
 *   x_bf16    uint16 [rows][d]     bf16 bit patterns; 16-byte aligned
 *   x_packed  uint8  [rows][d/2]   two codes per byte, element 2i in bits 3:0;
 *                                  8-byte aligned (output)
 *   sf        uint8  [rows][d/16]  E4M3 codes (output)
 *   g         float  [1] or [rows] global scales, 4-byte aligned; positive and
 *                                  finite for meaningful codes (not checked: the
 *                                  host never reads device memory)
 *
 * Shape rules: rows >= 1, d >= 16, d % 16 == 0, rows * d / 16 < 2^31 - 256.
 * Calls only enqueue work on `stream` (a hipStream_t, NULL = default stream):
 * no synchronisation, no host read of device data, no allocation.  All
 * arguments are validated before any HIP call; an invalid call returns a
 * negative status (nvfp4_gemv.h) and enqueues nothing.
 */
#ifndef NVFP4_QUANTIZE_H
#define NVFP4_QUANTIZE_H

#include <stddef.h>
#include <stdint.h>

#include "nvfp4_gemv.h"

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ROUND_HALF_STEP 0
#define NVFP4_ROUND_NEAREST_EVEN 1
#define NVFP4_ROUND_NEAREST_LOWER 2

/*
 * Quantises x_bf16 [rows][d] into x_packed and sf as above.  scale_per_row = 0:
 * global_scale points to one float used for every row; 1: to `rows` floats.
 * Returns NVFP4_GEMV_OK, or NULL_POINTER, BAD_ARGUMENT (rule or flag out of
 * range), BAD_SHAPE, ALIGNMENT, ALIAS (an output overlaps an input or the
 * other output), LAUNCH.
 */
int nvfp4_quantize_activation(const uint16_t *x_bf16, const float *global_scale,
                              int32_t scale_per_row, uint8_t *x_packed, uint8_t *sf,
                              int64_t rows, int64_t d, int32_t rule, void *stream);

/*
 * Offline weight quantiser: the bridge page's weight quantiser (section
 * "Quantization") on the device, for `groups` tensors of [rows][d] each
 * (e.g. the experts of a MoE layer; groups = 1 for one matrix), stored one
 * after the other in w_bf16 [groups][rows][d].  Each tensor's global scale is
 * computed from its own amax:
 *
 *   global_scale[e] = f32( max(max |T_e|, 1e-8) / (6 * 448) )   (NaN propagates)
 *
 * and the tensor is then quantised with it as nvfp4_quantize_activation does,
 * under `rule` (the page's weight quantiser is NVFP4_ROUND_NEAREST_LOWER):
 * w_packed [groups][rows][d/2], sf [groups][rows][d/16].  global_scale
 * [groups] (float, 4-byte aligned, device) is an output: the weights' global
 * scales for the GEMV's alpha.  Three kernels are enqueued on `stream`; their
 * scratch (groups * 256 bytes + 4 bytes per row) is the library-owned
 * per-(device, stream) workspace of nvfp4_gemv_launch, grown on first need
 * without synchronising (see nvfp4_workspace_reserve for graph capture).
 * Shape and alignment rules as for nvfp4_quantize_activation over groups*rows
 * rows.  Returns NVFP4_GEMV_OK, NULL_POINTER, BAD_ARGUMENT, BAD_SHAPE,
 * ALIGNMENT, ALIAS, DEVICE, WORKSPACE or LAUNCH.
 */
int nvfp4_quantize_weight(const uint16_t *w_bf16, int64_t groups, int64_t rows, int64_t d,
                          int32_t rule, uint8_t *w_packed, uint8_t *sf, float *global_scale,
                          void *stream);

/*
 * The batched GEMV of nvfp4_gemv.h with a bf16 activation: quantises x_bf16
 * [l][k] with one global scale per batch (x_scale [l]) into x_packed [l][k/2]
 * and sfx [l][k/16], writes alpha[b] = f32(A_scale[b] * x_scale[b]) (A_scale
 * [l] are the weights' global scales; NULL means 1), then runs
 * nvfp4_gemv_launch on those operands:
 *
 *   c[b,r] = f16( f32( alpha[b] * sum_kk e2m1(A) e4m3(sfA) e2m1(x_q) e4m3(sfx) ) )
 *
 * x_packed, sfx and alpha are caller-owned device outputs (they double as the
 * quantised operands for reuse).  Two kernels are enqueued on `stream` (three
 * when the GEMV splits K); split-K workspace rules as for nvfp4_gemv_launch.
 * Every argument is validated first; if the GEMV launch itself then fails
 * (WORKSPACE, DEVICE, LAUNCH) the quantised outputs may already be written,
 * c is not.  Returns a status.
 */
int nvfp4_gemv_bf16x_launch(const uint8_t *A_packed, const uint8_t *sfA, const float *A_scale,
                            const uint16_t *x_bf16, const float *x_scale, int32_t rule,
                            uint8_t *x_packed, uint8_t *sfx, float *alpha, uint16_t *c,
                            int64_t l, int64_t m, int64_t k, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_QUANTIZE_H */
