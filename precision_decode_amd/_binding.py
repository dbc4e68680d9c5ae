"""ctypes binding of ``libnvfp4_gemv.so`` (argument marshalling only).

Each C entry point of ``include/nvfp4_gemv.h``, ``include/nvfp4_quantize.h``
and ``include/nvfp4_mma.h`` has a Python function of the same name.  Pointer arguments accept a torch tensor (its ``data_ptr()``), a raw
integer device address, or None where the C side allows NULL; ``stream``
accepts None (torch's current stream), a ``torch.cuda.Stream`` or a raw
``hipStream_t`` integer.  A negative status raises :class:`Nvfp4GemvError`.
All arithmetic happens in the HIP kernels; nothing here falls back to the CPU.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4_gemv.so")

NVFP4_GEMV_OK = 0
NVFP4_GEMV_ERR_NULL_POINTER = -1
NVFP4_GEMV_ERR_BAD_SHAPE = -2
NVFP4_GEMV_ERR_WORKSPACE = -3
NVFP4_GEMV_ERR_LAUNCH = -4
NVFP4_GEMV_ERR_ALIAS = -5
NVFP4_GEMV_ERR_ALIGNMENT = -6
NVFP4_GEMV_ERR_DEVICE = -7
NVFP4_GEMV_ERR_BAD_TUNING = -8
NVFP4_GEMV_ERR_BAD_ARGUMENT = -9

NVFP4_ROUND_HALF_STEP = 0
NVFP4_ROUND_NEAREST_EVEN = 1
NVFP4_ROUND_NEAREST_LOWER = 2

NVFP4_OUT_F16 = 0
NVFP4_OUT_BF16 = 1

NVFP4_MMA_FORM_MATRIX_CORES = 0
NVFP4_MMA_FORM_VALU_TILES = 1
NVFP4_MMA_FORM_LDS_STAGED = 2
NVFP4_MMA_FORM_LDS_VECTOR_REGS = 3

NVFP4_GEMV_PATH_AUTO = 0
NVFP4_GEMV_PATH_FAST = 1
NVFP4_GEMV_PATH_GENERIC = 2

NVFP4_GEMV_NOALLOC_SCRATCH_BYTES = 4 << 20

# Every symbol the header declares.
EXPORTED = (
    "nvfp4_gemv_status_string",
    "nvfp4_gemv_launch",
    "nvfp4_gemv_workspace_size",
    "nvfp4_gemv_launch_ws",
    "nvfp4_gemv_num_variants",
    "nvfp4_gemv_variant_info",
    "nvfp4_gemv_plan",
    "nvfp4_gemv_launch_tuned",
    "nvfp4_hbm_read_probe",
    "nvfp4_hbm_read_probe_rows",
    "nvfp4_workspace_reserve",
    "nvfp4_gemv_launch_noalloc",
    "nvfp4_quantize_activation",
    "nvfp4_quantize_weight",
    "nvfp4_gemv_bf16x_launch",
    "nvfp4_gemm_smalln_launch",
    "nvfp4_mma_num_variants",
    "nvfp4_mma_variant_info",
    "nvfp4_mma_variant_form",
    "nvfp4_gemm_smalln_plan",
    "nvfp4_grouped_gemv_plan",
    "nvfp4_gemm_smalln_launch_tuned",
    "nvfp4_grouped_gemv_launch",
    "nvfp4_grouped_gemv_launch_tuned",
    "nvfp4_mma_packed_sizes",
    "nvfp4_mma_pack_weight",
    "nvfp4_gemm_smalln_launch_packed",
    "nvfp4_grouped_gemv_launch_packed",
)


class Nvfp4GemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({nvfp4_gemv_status_string(status)})")


class Tuning(ctypes.Structure):
    """Mirror of ``nvfp4_gemv_tuning_t``."""
    _fields_ = [("path", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("ksplit", ctypes.c_int32), ("reserved", ctypes.c_int32)]

    def __repr__(self):
        return f"Tuning(path={self.path}, variant={self.variant}, ksplit={self.ksplit})"


class MmaTuning(ctypes.Structure):
    """Mirror of ``nvfp4_mma_tuning_t``."""
    _fields_ = [("path", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("ksplit", ctypes.c_int32), ("rows_per_block", ctypes.c_int32)]

    def __repr__(self):
        return (f"MmaTuning(path={self.path}, variant={self.variant}, ksplit={self.ksplit}, "
                f"rows_per_block={self.rows_per_block})")


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def load():
    """Load the built library; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m precision_decode_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.nvfp4_gemv_status_string.restype = ctypes.c_char_p
    lib.nvfp4_gemv_status_string.argtypes = [ctypes.c_int]
    gemv_args = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64]
    lib.nvfp4_gemv_launch.restype = ctypes.c_int
    lib.nvfp4_gemv_launch.argtypes = gemv_args + [_P]
    lib.nvfp4_gemv_workspace_size.restype = ctypes.c_size_t
    lib.nvfp4_gemv_workspace_size.argtypes = [_I64, _I64, _I64]
    lib.nvfp4_gemv_launch_ws.restype = ctypes.c_int
    lib.nvfp4_gemv_launch_ws.argtypes = gemv_args + [_P, ctypes.c_size_t, _P]
    lib.nvfp4_gemv_num_variants.restype = ctypes.c_int
    lib.nvfp4_gemv_num_variants.argtypes = []
    lib.nvfp4_gemv_variant_info.restype = ctypes.c_int
    lib.nvfp4_gemv_variant_info.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int32)] * 4
    lib.nvfp4_gemv_plan.restype = ctypes.c_int
    lib.nvfp4_gemv_plan.argtypes = [_I64, _I64, _I64, ctypes.c_int, ctypes.POINTER(Tuning),
                                    ctypes.POINTER(Tuning), ctypes.POINTER(ctypes.c_size_t)]
    lib.nvfp4_gemv_launch_tuned.restype = ctypes.c_int
    lib.nvfp4_gemv_launch_tuned.argtypes = gemv_args + [ctypes.POINTER(Tuning), _P, ctypes.c_size_t, _P]
    lib.nvfp4_gemv_launch_noalloc.restype = ctypes.c_int
    lib.nvfp4_gemv_launch_noalloc.argtypes = gemv_args + [_P]
    lib.nvfp4_workspace_reserve.restype = ctypes.c_int
    lib.nvfp4_workspace_reserve.argtypes = [ctypes.c_size_t, _P]
    lib.nvfp4_hbm_read_probe_rows.restype = ctypes.c_int
    lib.nvfp4_hbm_read_probe_rows.argtypes = [_P, _P, _I64, _I64, _P, _P]
    lib.nvfp4_hbm_read_probe.restype = ctypes.c_int
    lib.nvfp4_hbm_read_probe.argtypes = [_P, ctypes.c_size_t, _P, _P]
    lib.nvfp4_quantize_activation.restype = ctypes.c_int
    lib.nvfp4_quantize_activation.argtypes = [_P, _P, ctypes.c_int32, _P, _P, _I64, _I64,
                                              ctypes.c_int32, _P]
    lib.nvfp4_quantize_weight.restype = ctypes.c_int
    lib.nvfp4_quantize_weight.argtypes = [_P, _I64, _I64, _I64, ctypes.c_int32, _P, _P, _P, _P]
    lib.nvfp4_gemv_bf16x_launch.restype = ctypes.c_int
    lib.nvfp4_gemv_bf16x_launch.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P,
                                            _I64, _I64, _I64, _P]
    smalln_args = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int32]
    lib.nvfp4_gemm_smalln_launch.restype = ctypes.c_int
    lib.nvfp4_gemm_smalln_launch.argtypes = smalln_args + [_P]
    lib.nvfp4_mma_num_variants.restype = ctypes.c_int
    lib.nvfp4_mma_num_variants.argtypes = []
    lib.nvfp4_mma_variant_info.restype = ctypes.c_int
    lib.nvfp4_mma_variant_info.argtypes = [ctypes.c_int] + [ctypes.POINTER(ctypes.c_int32)] * 3
    lib.nvfp4_mma_variant_form.restype = ctypes.c_int
    lib.nvfp4_mma_variant_form.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_int32)]
    lib.nvfp4_grouped_gemv_plan.restype = ctypes.c_int
    lib.nvfp4_grouped_gemv_plan.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int, ctypes.c_int,
                                            ctypes.POINTER(MmaTuning), ctypes.POINTER(MmaTuning)]
    lib.nvfp4_gemm_smalln_plan.restype = ctypes.c_int
    lib.nvfp4_gemm_smalln_plan.argtypes = [_I64, _I64, _I64, _I64, ctypes.c_int,
                                           ctypes.POINTER(MmaTuning), ctypes.POINTER(MmaTuning),
                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.nvfp4_gemm_smalln_launch_tuned.restype = ctypes.c_int
    lib.nvfp4_gemm_smalln_launch_tuned.argtypes = smalln_args + [ctypes.POINTER(MmaTuning), _P,
                                                                 ctypes.c_size_t, _P]
    grouped_args = [_P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_int32]
    lib.nvfp4_grouped_gemv_launch.restype = ctypes.c_int
    lib.nvfp4_grouped_gemv_launch.argtypes = grouped_args + [_P]
    lib.nvfp4_grouped_gemv_launch_tuned.restype = ctypes.c_int
    lib.nvfp4_grouped_gemv_launch_tuned.argtypes = grouped_args + [ctypes.POINTER(MmaTuning), _P]
    lib.nvfp4_mma_packed_sizes.restype = ctypes.c_int
    lib.nvfp4_mma_packed_sizes.argtypes = [_I64, _I64, _I64, ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t)]
    lib.nvfp4_mma_pack_weight.restype = ctypes.c_int
    lib.nvfp4_mma_pack_weight.argtypes = [_P, _P, _I64, _I64, _I64, _P, _P, _P]
    lib.nvfp4_gemm_smalln_launch_packed.restype = ctypes.c_int
    lib.nvfp4_gemm_smalln_launch_packed.argtypes = smalln_args + [ctypes.POINTER(MmaTuning), _P]
    lib.nvfp4_grouped_gemv_launch_packed.restype = ctypes.c_int
    lib.nvfp4_grouped_gemv_launch_packed.argtypes = grouped_args + [ctypes.POINTER(MmaTuning), _P]
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not getattr(t, "is_cuda", False):
        raise ValueError("device pointer expected: pass a CUDA/HIP tensor or an integer address")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != NVFP4_GEMV_OK:
        raise Nvfp4GemvError(status, where)


def nvfp4_gemv_status_string(status: int) -> str:
    return load().nvfp4_gemv_status_string(int(status)).decode()


def nvfp4_gemv_launch(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k, stream=None):
    st = load().nvfp4_gemv_launch(_ptr(A_packed), _ptr(sfA), _ptr(x_packed), _ptr(sfx),
                                  _ptr(alpha), _ptr(c), l, m, k, _stream(stream))
    _check(st, "nvfp4_gemv_launch")


def nvfp4_gemv_workspace_size(l, m, k) -> int:
    return int(load().nvfp4_gemv_workspace_size(l, m, k))


def nvfp4_gemv_launch_ws(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k, workspace,
                         workspace_bytes, stream=None):
    st = load().nvfp4_gemv_launch_ws(_ptr(A_packed), _ptr(sfA), _ptr(x_packed), _ptr(sfx),
                                     _ptr(alpha), _ptr(c), l, m, k, _ptr(workspace),
                                     int(workspace_bytes), _stream(stream))
    _check(st, "nvfp4_gemv_launch_ws")


def nvfp4_gemv_num_variants() -> int:
    return int(load().nvfp4_gemv_num_variants())


def nvfp4_gemv_variant_info(v: int):
    """(rows per wave, iterations in flight, waves per group, x staging: 0 fp16 in LDS,
    1 packed codes in LDS, 2 none)."""
    r, u, w, px = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load().nvfp4_gemv_variant_info(v, ctypes.byref(r), ctypes.byref(u), ctypes.byref(w),
                                          ctypes.byref(px)), "nvfp4_gemv_variant_info")
    return r.value, u.value, w.value, px.value


def _tuning(t):
    if t is None:
        return None
    if isinstance(t, Tuning):
        return ctypes.byref(t)
    return ctypes.byref(Tuning(int(t.get("path", 0)), int(t.get("variant", 0)),
                               int(t.get("ksplit", 0)), 0))


def _mma_tuning(t):
    if t is None:
        return None
    if isinstance(t, MmaTuning):
        return ctypes.byref(t)
    return ctypes.byref(MmaTuning(int(t.get("path", 0)), int(t.get("variant", 0)),
                                  int(t.get("ksplit", 0)), int(t.get("rows_per_block", 0))))


def nvfp4_gemv_plan(l, m, k, aligned=True, tuning=None):
    """Returns (Tuning actually used, workspace bytes)."""
    out = Tuning()
    ws = ctypes.c_size_t()
    _check(load().nvfp4_gemv_plan(l, m, k, int(bool(aligned)), _tuning(tuning), ctypes.byref(out),
                                  ctypes.byref(ws)), "nvfp4_gemv_plan")
    return out, int(ws.value)


def nvfp4_gemv_launch_tuned(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k, tuning, workspace,
                            workspace_bytes, stream=None):
    st = load().nvfp4_gemv_launch_tuned(_ptr(A_packed), _ptr(sfA), _ptr(x_packed), _ptr(sfx),
                                        _ptr(alpha), _ptr(c), l, m, k, _tuning(tuning),
                                        _ptr(workspace), int(workspace_bytes), _stream(stream))
    _check(st, "nvfp4_gemv_launch_tuned")


def nvfp4_gemv_launch_noalloc(A_packed, sfA, x_packed, sfx, alpha, c, l, m, k, stream=None):
    st = load().nvfp4_gemv_launch_noalloc(_ptr(A_packed), _ptr(sfA), _ptr(x_packed), _ptr(sfx),
                                          _ptr(alpha), _ptr(c), l, m, k, _stream(stream))
    _check(st, "nvfp4_gemv_launch_noalloc")


def nvfp4_workspace_reserve(nbytes, stream=None):
    _check(load().nvfp4_workspace_reserve(int(nbytes), _stream(stream)), "nvfp4_workspace_reserve")


def nvfp4_hbm_read_probe(buffer, nbytes, sink, stream=None):
    _check(load().nvfp4_hbm_read_probe(_ptr(buffer), int(nbytes), _ptr(sink), _stream(stream)),
           "nvfp4_hbm_read_probe")


def nvfp4_hbm_read_probe_rows(A, sfA, rows, k, sink, stream=None):
    _check(load().nvfp4_hbm_read_probe_rows(_ptr(A), _ptr(sfA), rows, k, _ptr(sink),
                                            _stream(stream)), "nvfp4_hbm_read_probe_rows")


def nvfp4_quantize_activation(x_bf16, global_scale, scale_per_row, x_packed, sf, rows, d, rule,
                              stream=None):
    _check(load().nvfp4_quantize_activation(_ptr(x_bf16), _ptr(global_scale), int(scale_per_row),
                                            _ptr(x_packed), _ptr(sf), rows, d, int(rule),
                                            _stream(stream)), "nvfp4_quantize_activation")


def nvfp4_quantize_weight(w_bf16, groups, rows, d, rule, w_packed, sf, global_scale, stream=None):
    _check(load().nvfp4_quantize_weight(_ptr(w_bf16), groups, rows, d, int(rule), _ptr(w_packed),
                                        _ptr(sf), _ptr(global_scale), _stream(stream)),
           "nvfp4_quantize_weight")


def nvfp4_gemv_bf16x_launch(A_packed, sfA, A_scale, x_bf16, x_scale, rule, x_packed, sfx, alpha, c,
                            l, m, k, stream=None):
    _check(load().nvfp4_gemv_bf16x_launch(_ptr(A_packed), _ptr(sfA), _ptr(A_scale), _ptr(x_bf16),
                                          _ptr(x_scale), int(rule), _ptr(x_packed), _ptr(sfx),
                                          _ptr(alpha), _ptr(c), l, m, k, _stream(stream)),
           "nvfp4_gemv_bf16x_launch")


def nvfp4_gemm_smalln_launch(A_packed, sfA, B_packed, sfB, alpha, c, l, m, n, k,
                             out_type=NVFP4_OUT_F16, stream=None):
    _check(load().nvfp4_gemm_smalln_launch(_ptr(A_packed), _ptr(sfA), _ptr(B_packed), _ptr(sfB),
                                           _ptr(alpha), _ptr(c), l, m, n, k, int(out_type),
                                           _stream(stream)), "nvfp4_gemm_smalln_launch")


def nvfp4_mma_num_variants() -> int:
    return int(load().nvfp4_mma_num_variants())


def nvfp4_mma_variant_info(v: int):
    """Matrix-core variants: (row tiles of 16 per wave, windows in flight, waves
    per group); VALU row-tile variants: (rows per tile, vectors per pass, waves
    per group)."""
    r, u, w = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load().nvfp4_mma_variant_info(v, ctypes.byref(r), ctypes.byref(u), ctypes.byref(w)),
           "nvfp4_mma_variant_info")
    return r.value, u.value, w.value


def nvfp4_mma_variant_form(v: int) -> int:
    """NVFP4_MMA_FORM_MATRIX_CORES (0), NVFP4_MMA_FORM_VALU_TILES (1),
    NVFP4_MMA_FORM_LDS_STAGED (2) or NVFP4_MMA_FORM_LDS_VECTOR_REGS (3)."""
    f = ctypes.c_int32()
    _check(load().nvfp4_mma_variant_form(v, ctypes.byref(f)), "nvfp4_mma_variant_form")
    return f.value


def nvfp4_gemm_smalln_plan(l, m, n, k, aligned=True, tuning=None):
    """Returns (MmaTuning actually used, workspace bytes)."""
    out = MmaTuning()
    ws = ctypes.c_size_t()
    _check(load().nvfp4_gemm_smalln_plan(l, m, n, k, int(bool(aligned)), _mma_tuning(tuning),
                                         ctypes.byref(out), ctypes.byref(ws)),
           "nvfp4_gemm_smalln_plan")
    return out, int(ws.value)


def nvfp4_grouped_gemv_plan(experts, n, k, tokens, aligned=True, packed=False, tuning=None):
    """Returns the MmaTuning the grouped GEMV would use for `tokens` routed tokens."""
    out = MmaTuning()
    _check(load().nvfp4_grouped_gemv_plan(experts, n, k, tokens, int(bool(aligned)),
                                          int(bool(packed)), _mma_tuning(tuning), ctypes.byref(out)),
           "nvfp4_grouped_gemv_plan")
    return out


def nvfp4_gemm_smalln_launch_tuned(A_packed, sfA, B_packed, sfB, alpha, c, l, m, n, k, out_type,
                                   tuning, workspace, workspace_bytes, stream=None):
    _check(load().nvfp4_gemm_smalln_launch_tuned(_ptr(A_packed), _ptr(sfA), _ptr(B_packed),
                                                 _ptr(sfB), _ptr(alpha), _ptr(c), l, m, n, k,
                                                 int(out_type), _mma_tuning(tuning), _ptr(workspace),
                                                 int(workspace_bytes), _stream(stream)),
           "nvfp4_gemm_smalln_launch_tuned")


def nvfp4_grouped_gemv_launch(X_packed, sfX, W_packed, sfW, offsets, gs_x, gs_w, c, tokens, experts,
                              n, k, out_type=NVFP4_OUT_BF16, stream=None):
    _check(load().nvfp4_grouped_gemv_launch(_ptr(X_packed), _ptr(sfX), _ptr(W_packed), _ptr(sfW),
                                            _ptr(offsets), _ptr(gs_x), _ptr(gs_w), _ptr(c), tokens,
                                            experts, n, k, int(out_type), _stream(stream)),
           "nvfp4_grouped_gemv_launch")


def nvfp4_grouped_gemv_launch_tuned(X_packed, sfX, W_packed, sfW, offsets, gs_x, gs_w, c, tokens,
                                    experts, n, k, out_type, tuning, stream=None):
    _check(load().nvfp4_grouped_gemv_launch_tuned(_ptr(X_packed), _ptr(sfX), _ptr(W_packed),
                                                  _ptr(sfW), _ptr(offsets), _ptr(gs_x), _ptr(gs_w),
                                                  _ptr(c), tokens, experts, n, k, int(out_type),
                                                  _mma_tuning(tuning), _stream(stream)),
           "nvfp4_grouped_gemv_launch_tuned")


def nvfp4_mma_packed_sizes(groups, rows, k):
    """(codes bytes, scales bytes) of packed weights for groups matrices of rows x k."""
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().nvfp4_mma_packed_sizes(groups, rows, k, ctypes.byref(cb), ctypes.byref(sb)),
           "nvfp4_mma_packed_sizes")
    return int(cb.value), int(sb.value)


def nvfp4_mma_pack_weight(W, sW, groups, rows, k, W_packed, sW_packed, stream=None):
    _check(load().nvfp4_mma_pack_weight(_ptr(W), _ptr(sW), groups, rows, k, _ptr(W_packed),
                                        _ptr(sW_packed), _stream(stream)), "nvfp4_mma_pack_weight")


def nvfp4_gemm_smalln_launch_packed(A_packed, sfA_packed, B_packed, sfB, alpha, c, l, m, n, k,
                                    out_type=NVFP4_OUT_F16, tuning=None, stream=None):
    _check(load().nvfp4_gemm_smalln_launch_packed(_ptr(A_packed), _ptr(sfA_packed), _ptr(B_packed),
                                                  _ptr(sfB), _ptr(alpha), _ptr(c), l, m, n, k,
                                                  int(out_type), _mma_tuning(tuning),
                                                  _stream(stream)),
           "nvfp4_gemm_smalln_launch_packed")


def nvfp4_grouped_gemv_launch_packed(X_packed, sfX, W_packed, sfW_packed, offsets, gs_x, gs_w, c,
                                     tokens, experts, n, k, out_type=NVFP4_OUT_BF16, tuning=None,
                                     stream=None):
    _check(load().nvfp4_grouped_gemv_launch_packed(_ptr(X_packed), _ptr(sfX), _ptr(W_packed),
                                                   _ptr(sfW_packed), _ptr(offsets), _ptr(gs_x),
                                                   _ptr(gs_w), _ptr(c), tokens, experts, n, k,
                                                   int(out_type), _mma_tuning(tuning),
                                                   _stream(stream)),
           "nvfp4_grouped_gemv_launch_packed")


def quantize_activation(x, global_scale, rule=NVFP4_ROUND_HALF_STEP, stream=None):
    """Tensor-level call: x (rows, d) bfloat16 (or its uint16/int16 bits),
    global_scale a float32 device tensor of 1 or ``rows`` values.  Returns
    (packed uint8 (rows, d/2), scales uint8 (rows, d/16))."""
    import torch

    if x.dim() != 2 or x.element_size() != 2 or not x.is_contiguous() or not x.is_cuda:
        raise ValueError("x must be a contiguous 2-D 16-bit device tensor (bf16 bits)")
    rows, d = x.shape
    if global_scale.dtype != torch.float32 or not global_scale.is_cuda or \
            global_scale.numel() not in (1, rows):
        raise ValueError("global_scale must be a float32 device tensor of 1 or rows values")
    per_row = 1 if (global_scale.numel() == rows and rows > 1) else 0
    q = torch.empty((rows, d // 2), dtype=torch.uint8, device=x.device)
    sf = torch.empty((rows, d // 16), dtype=torch.uint8, device=x.device)
    nvfp4_quantize_activation(x, global_scale, per_row, q, sf, rows, d, rule, stream)
    return q, sf


def gemv(A_packed, sfA, x_packed, sfx, alpha=None, out=None, stream=None):
    """Tensor-level call: shapes (l,m,k/2), (l,m,k/16), (l,k/2), (l,k/16), (l,).

    Checks dtypes, shapes, contiguity and device, allocates ``out`` (uint16
    fp16 bits, (l, m)) if not given, and calls :func:`nvfp4_gemv_launch`.
    """
    import torch

    if A_packed.dim() != 3:
        raise ValueError("A_packed must be (l, m, k/2)")
    l, m, half = A_packed.shape
    k = 2 * half
    want = {"A_packed": (A_packed, (l, m, half)), "sfA": (sfA, (l, m, k // 16)),
            "x_packed": (x_packed, (l, half)), "sfx": (sfx, (l, k // 16))}
    for name, (t, shape) in want.items():
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous uint8 device tensor of shape {shape}")
    if alpha is not None and (alpha.dtype != torch.float32 or tuple(alpha.shape) != (l,)
                              or not alpha.is_cuda):
        raise ValueError("alpha must be a float32 device tensor of shape (l,)")
    if out is None:
        out = torch.empty((l, m), dtype=torch.uint16, device=A_packed.device)
    elif (out.dtype not in (torch.uint16, torch.float16, torch.int16) or tuple(out.shape) != (l, m)
          or not out.is_contiguous() or not out.is_cuda):
        raise ValueError("out must be a contiguous 16-bit device tensor of shape (l, m)")
    nvfp4_gemv_launch(A_packed, sfA, x_packed, sfx, alpha, out, l, m, k, stream)
    return out


def pack_weight(W, sW, stream=None):
    """Tensor-level call: W (groups, rows, k/2) and sW (groups, rows, k/16)
    uint8 device tensors -> (codes, scales), the packed layout of
    :func:`nvfp4_mma_pack_weight` as flat uint8 device tensors, for
    :func:`nvfp4_gemm_smalln_launch_packed` and
    :func:`nvfp4_grouped_gemv_launch_packed`.  A 2-D W is one group."""
    import torch

    if W.dim() == 2:
        W, sW = W.unsqueeze(0), sW.unsqueeze(0)
    if W.dim() != 3:
        raise ValueError("W must be (groups, rows, k/2) or (rows, k/2)")
    groups, rows, half = W.shape
    k = 2 * half
    for name, t, shape in (("W", W, (groups, rows, half)), ("sW", sW, (groups, rows, k // 16))):
        if t.dtype != torch.uint8 or tuple(t.shape) != shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous uint8 device tensor of shape {shape}")
    cb, sb = nvfp4_mma_packed_sizes(groups, rows, k)
    codes = torch.empty(cb, dtype=torch.uint8, device=W.device)
    scales = torch.empty(sb, dtype=torch.uint8, device=W.device)
    nvfp4_mma_pack_weight(W, sW, groups, rows, k, codes, scales, stream)
    return codes, scales
