"""NVFP4 block-scaled batched GEMV for MI355X (gfx950), the BF16 -> NVFP4
activation quantiser that feeds it, and the same scaled product against
several vectors: the small-N GEMM and the grouped (MoE) GEMV.

The computation runs in the hand-written HIP kernels of ``libnvfp4_gemv.so``
(``csrc/*.hip``, C ABI in ``include/nvfp4_gemv.h``,
``include/nvfp4_quantize.h`` and ``include/nvfp4_mma.h``).  This package
only marshals arguments to that library; it raises if the library is not
built and never computes anything on the CPU.
"""
from ._binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MmaTuning,
    NVFP4_GEMV_ERR_ALIAS,
    NVFP4_GEMV_ERR_ALIGNMENT,
    NVFP4_GEMV_ERR_BAD_ARGUMENT,
    NVFP4_GEMV_ERR_BAD_SHAPE,
    NVFP4_GEMV_ERR_BAD_TUNING,
    NVFP4_GEMV_ERR_DEVICE,
    NVFP4_GEMV_ERR_LAUNCH,
    NVFP4_GEMV_ERR_NULL_POINTER,
    NVFP4_GEMV_ERR_WORKSPACE,
    NVFP4_GEMV_OK,
    NVFP4_GEMV_PATH_AUTO,
    NVFP4_GEMV_PATH_FAST,
    NVFP4_GEMV_PATH_GENERIC,
    NVFP4_OUT_BF16,
    NVFP4_OUT_F16,
    NVFP4_ROUND_HALF_STEP,
    NVFP4_ROUND_NEAREST_EVEN,
    NVFP4_ROUND_NEAREST_LOWER,
    Nvfp4GemvError,
    Tuning,
    gemv,
    load,
    nvfp4_gemm_smalln_launch,
    nvfp4_gemm_smalln_launch_tuned,
    nvfp4_gemm_smalln_plan,
    nvfp4_gemv_bf16x_launch,
    nvfp4_gemv_launch,
    nvfp4_gemv_launch_ws,
    nvfp4_gemv_launch_tuned,
    nvfp4_gemv_num_variants,
    nvfp4_gemv_plan,
    nvfp4_gemv_status_string,
    nvfp4_gemv_variant_info,
    nvfp4_gemv_workspace_size,
    nvfp4_grouped_gemv_launch,
    nvfp4_grouped_gemv_launch_tuned,
    nvfp4_hbm_read_probe,
    nvfp4_mma_num_variants,
    nvfp4_mma_variant_info,
    nvfp4_quantize_activation,
    nvfp4_quantize_weight,
    quantize_activation,
)
