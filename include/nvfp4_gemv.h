/*
 * nvfp4_gemv.h - C ABI of the MI355X (gfx950) NVFP4 block-scaled batched GEMV.
 *
 * Operation (the NVFP4 batched GEMV of "nvFP4 Batch GEMV算子系列(下)", section
 * "NVFP4 Batched GEMV 概念阐述": 16 consecutive K elements share one FP8 E4M3
 * scale, element kk belongs to block floor(kk/16); the E2M1 magnitudes and the
 * block size 16 are the constants of the CuTeDSL NVFP4 bridge page):
 *
 *   S[b,r] = sum_kk e2m1(A[b,r,kk]) * e4m3(sfA[b,r,kk/16]) * e2m1(x[b,kk]) * e4m3(sfx[b,kk/16])
 *   c[b,r] = f16_rne( f32_rne( alpha[b] * S[b,r] ) )
 *
 * for b < l, r < m.  Products are accumulated in fp32; c is fully overwritten
 * (no accumulation into the output).  The per-batch fp32 `alpha` carries the
 * tensors' global scales (the page's formula has one fp32 global scale; the
 * bridge page keeps one per expert).
 *
 * Memory layout (all row-major and contiguous, batch outermost; the blog
 * post's (l, mn, k/2) storage before its permute to (mn, k/2, l)):
 *   A_packed  uint8  [l][m][k/2]   two E2M1 codes per byte, element 2i in bits 3:0,
 *                                  element 2i+1 in bits 7:4, bit 3 of a code = sign
 *   sfA       uint8  [l][m][k/16]  E4M3 (float8_e4m3fn) codes
 *   x_packed  uint8  [l][k/2]      packed like A_packed
 *   sfx       uint8  [l][k/16]     E4M3 codes
 *   alpha     float  [l]           may be NULL: alpha = 1 for every batch
 *   c         uint16 [l][m]        fp16 bit patterns (output)
 *
 * All data pointers are DEVICE pointers owned by the caller; the library never
 * frees them and does not keep them after the enqueued work.  `stream` is a
 * hipStream_t (NULL = the default stream).  Every launch call is asynchronous:
 * it only enqueues work on `stream`, never synchronises the device and never
 * reads device memory from the host.
 *
 * Shape rules: l, m >= 1; k >= 16 and k % 16 == 0 (whole scale blocks); the
 * byte sizes must fit in int64, l*m < 2^31 and k < 2^31.  c must be 2-byte
 * aligned and alpha 4-byte aligned.  The fast kernel needs k % 32 == 0,
 * 16-byte aligned A_packed / x_packed and 2-byte aligned sfA / sfx; every other
 * valid call takes a slower generic kernel with the same results.
 *
 * Errors: all arguments are validated before any HIP call; invalid calls
 * return a negative status and enqueue nothing.  No C++ exception crosses this
 * interface.
 */
#ifndef NVFP4_GEMV_H
#define NVFP4_GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define NVFP4_GEMV_OK 0
#define NVFP4_GEMV_ERR_NULL_POINTER (-1) /* a required pointer is NULL            */
#define NVFP4_GEMV_ERR_BAD_SHAPE (-2)    /* l, m, k out of range or k % 16 != 0  */
#define NVFP4_GEMV_ERR_WORKSPACE (-3)    /* workspace missing, too small or      */
                                         /* could not be allocated               */
#define NVFP4_GEMV_ERR_LAUNCH (-4)       /* the HIP runtime rejected a launch    */
#define NVFP4_GEMV_ERR_ALIAS (-5)        /* c overlaps an input                  */
#define NVFP4_GEMV_ERR_ALIGNMENT (-6)    /* c, alpha or workspace misaligned     */
#define NVFP4_GEMV_ERR_DEVICE (-7)       /* no current HIP device                */
#define NVFP4_GEMV_ERR_BAD_TUNING (-8)   /* invalid nvfp4_gemv_tuning_t field    */
#define NVFP4_GEMV_ERR_BAD_ARGUMENT (-9) /* an enumerated argument (rounding     */
                                         /* rule, flag) is out of range          */

/*
 * Returns a static, NUL-terminated description of a status code (never NULL).
 */
const char *nvfp4_gemv_status_string(int status);

/*
 * The batched GEMV above.  Arguments as described in the header comment.
 *
 * When the launch plan splits K across workgroups (few rows, long K) the fp32
 * partial sums go to a workspace that the library owns, one per (device,
 * stream), kept until the process ends.  A call that needs more than the
 * stream's workspace holds grows it with hipMalloc: no synchronisation and no
 * free (the outgrown buffer stays allocated, since work enqueued before may
 * still read it).  Such a growing call cannot run while `stream` is being
 * captured into a graph: it then returns NVFP4_GEMV_ERR_WORKSPACE and enqueues
 * nothing.  Calls that need no more than the workspace holds allocate nothing
 * and are capture-safe; nvfp4_workspace_reserve sizes the workspace before a
 * capture.  Callers that must never allocate use nvfp4_gemv_launch_ws.
 * Concurrent calls on different streams never share a workspace.
 *
 * Returns NVFP4_GEMV_OK or a negative status.
 */
int nvfp4_gemv_launch(const uint8_t *A_packed, const uint8_t *sfA,
                      const uint8_t *x_packed, const uint8_t *sfx,
                      const float *alpha, uint16_t *c,
                      int64_t l, int64_t m, int64_t k, void *stream);

/*
 * Bytes of workspace nvfp4_gemv_launch_ws needs for this shape with the
 * default launch plan, whatever the alignment of the operands (0 when no plan
 * splits K; then the workspace may be NULL).  Returns 0 for invalid shapes as
 * well.
 */
size_t nvfp4_gemv_workspace_size(int64_t l, int64_t m, int64_t k);

/*
 * nvfp4_gemv_launch with a caller-owned device workspace of `workspace_bytes`
 * bytes (4-byte aligned, not aliasing any argument, not used by other work
 * that may run concurrently).  Allocates nothing.  Returns
 * NVFP4_GEMV_ERR_WORKSPACE when the workspace is needed and NULL or smaller
 * than nvfp4_gemv_workspace_size().
 */
int nvfp4_gemv_launch_ws(const uint8_t *A_packed, const uint8_t *sfA,
                         const uint8_t *x_packed, const uint8_t *sfx,
                         const float *alpha, uint16_t *c,
                         int64_t l, int64_t m, int64_t k,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * Grows the library-owned workspace of (current device, `stream`) to at least
 * `bytes` bytes, so that later calls on `stream` needing no more than that
 * allocate nothing (for instance under graph capture).  The workspace serves
 * nvfp4_gemv_launch, nvfp4_gemm_smalln_launch(_packed), nvfp4_quantize_weight
 * and nvfp4_gemv_bf16x_launch on that stream; take `bytes` from
 * nvfp4_gemv_workspace_size or the plan calls.  Not capture-safe itself.
 * Returns NVFP4_GEMV_OK, NVFP4_GEMV_ERR_DEVICE (no current device) or
 * NVFP4_GEMV_ERR_WORKSPACE (allocation failed, or `stream` is capturing).
 */
int nvfp4_workspace_reserve(size_t bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): nvfp4_gemv_launch
 * with the same arguments, results and kernels, except that the split-K
 * partial sums go to a fixed array of NVFP4_GEMV_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds in each GPU's memory from when it is loaded until the
 * process ends.  The call never allocates or frees memory.  A shape whose
 * partial sums need more than the array holds (nvfp4_gemv_workspace_size
 * above NVFP4_GEMV_NOALLOC_SCRATCH_BYTES, which takes hundreds of thousands of
 * rows with K split) returns NVFP4_GEMV_ERR_WORKSPACE and enqueues nothing.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (on different streams, or from different threads without
 * ordering) race on it and give undefined results; calls ordered on one
 * stream are safe.  Nothing in the array needs clearing between calls: each
 * call writes every partial sum before reading it.
 */
#define NVFP4_GEMV_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)

int nvfp4_gemv_launch_noalloc(const uint8_t *A_packed, const uint8_t *sfA,
                              const uint8_t *x_packed, const uint8_t *sfx,
                              const float *alpha, uint16_t *c,
                              int64_t l, int64_t m, int64_t k, void *stream);

/* ---- launch-plan control (tests and tuning sweeps) ---------------------- */

/* Kernel choice. */
#define NVFP4_GEMV_PATH_AUTO 0     /* fast kernel when shape and alignment allow */
#define NVFP4_GEMV_PATH_FAST 1     /* fast kernel; BAD_TUNING if not allowed     */
#define NVFP4_GEMV_PATH_GENERIC 2  /* generic kernel (any alignment, k % 32 == 16) */

typedef struct nvfp4_gemv_tuning_t {
    int32_t path;     /* NVFP4_GEMV_PATH_*                                          */
    int32_t variant;  /* fast-kernel variant, 0 = default, 1..nvfp4_gemv_num_variants();
                         must be 0 with NVFP4_GEMV_PATH_GENERIC                     */
    int32_t ksplit;   /* K split across workgroups, 0 = default, >= 1 explicit      */
    int32_t reserved; /* must be 0                                                  */
} nvfp4_gemv_tuning_t;

/* Number of fast-kernel variants. */
int nvfp4_gemv_num_variants(void);

/*
 * Describes fast-kernel variant v (1-based): rows each wave streams at once,
 * 1 KiB K-iterations kept in flight per row, waves per workgroup, and how x
 * reaches the arithmetic: 0 = decoded to fp16 in LDS once per workgroup,
 * 1 = staged in LDS as packed codes, 2 = not staged (each wave loads x's
 * codes next to its rows of A every iteration), 3 = row tiles: the
 * workgroup's waves share a tile of rows_per_wave rows (16, 8 or 4) and take
 * turns over K slices of 2048 elements, each wave keeping x~ of its slice in
 * registers (these variants take k <= 2^26; BAD_TUNING above).  Returns a
 * status.
 */
int nvfp4_gemv_variant_info(int v, int32_t *rows_per_wave, int32_t *iters_in_flight,
                            int32_t *waves_per_group, int32_t *x_staging);

/*
 * The plan the library would use: fills `out` with the resolved path, variant
 * and K split, and `*workspace_bytes` with the workspace it needs.  `aligned`
 * says whether the pointers meet the fast kernel's alignment rules.  `in` may
 * be NULL (all defaults).  Returns a status.
 */
int nvfp4_gemv_plan(int64_t l, int64_t m, int64_t k, int aligned,
                    const nvfp4_gemv_tuning_t *in, nvfp4_gemv_tuning_t *out,
                    size_t *workspace_bytes);

/*
 * nvfp4_gemv_launch_ws with an explicit plan (`tuning` may be NULL).  The
 * workspace must hold the bytes nvfp4_gemv_plan reports for the same tuning.
 */
int nvfp4_gemv_launch_tuned(const uint8_t *A_packed, const uint8_t *sfA,
                            const uint8_t *x_packed, const uint8_t *sfx,
                            const float *alpha, uint16_t *c,
                            int64_t l, int64_t m, int64_t k,
                            const nvfp4_gemv_tuning_t *tuning,
                            void *workspace, size_t workspace_bytes, void *stream);

/* ---- measurement helper ------------------------------------------------- */

/*
 * Streams `bytes` bytes (a multiple of 16, 16-byte aligned device buffer)
 * through the same non-temporal 16-byte loads the GEMV uses, in the fastest
 * plain read order measured on MI355X (contiguous 16 KiB chunks, one per
 * 4-wave workgroup at a time, every load of a chunk in flight together), and
 * writes one word per workgroup into `sink` (device, at least 4096 uint32).
 * Its run time gives the achievable HBM read bandwidth beside the GEMV's.
 * Returns a status.
 */
int nvfp4_hbm_read_probe(const void *buffer, size_t bytes, uint32_t *sink, void *stream);

/*
 * Streams `rows` rows of packed codes (A, k/2 bytes per row, 16-byte aligned)
 * and their scales (sfA, k/16 bytes per row, 2-byte aligned) once, with the
 * load pattern of the GEMV's kernel for long rows (workgroups of 7 waves over
 * 14 rows, 2 rows per wave, 4 iterations of 1 KiB per row in flight), and does
 * no arithmetic.  Its run time is the read ceiling of that pattern for a
 * weight of this shape.  Workgroup g stores the XOR of all words it read in
 * sink[g]: `sink` (device) holds ceil(rows / 14) uint32.  Shape rules:
 * rows >= 1, k >= 32, k % 32 == 0, k < 2^31.  Returns a status.
 */
int nvfp4_hbm_read_probe_rows(const uint8_t *A, const uint8_t *sfA, int64_t rows, int64_t k,
                              uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_GEMV_H */
