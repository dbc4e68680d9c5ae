"""CPU oracle of the NVFP4 block-scaled batched GEMV (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may use this
module; the product path never imports it.

    c[b, r] = f16( f32( alpha[b] * S[b, r] ) )
    S[b, r] = sum_k e2m1(A[b,r,k]) e4m3(sfA[b,r,k//16]) e2m1(x[b,k]) e4m3(sfx[b,k//16])

The sum is the NVFP4 batched GEMV formula of "nvFP4 Batch GEMV算子系列(下)"
(section "NVFP4 Batched GEMV 概念阐述"); it is computed in double, in increasing
k, by ``nvfp4_ref.c``.  The page's formula images did not survive, so the
placement of the global scale is a reading: the fp32 global scales of both
operands are folded into one fp32 ``alpha`` per batch, applied after the sum,
and the product is rounded first to fp32 and then to fp16 (the output type of
the page's ``ref_kernel``).  With integer-coded inputs S is exact in double and
the double product ``alpha * S`` is exact too (24 + 24 significant bits), so
the two roundings are the only ones.

The f64 -> f32 and f32 -> f16 roundings are numpy casts (IEEE
round-to-nearest-even, overflow to infinity).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_e2m1.restype = ctypes.c_double
        lib.oracle_e2m1.argtypes = [ctypes.c_uint]
        lib.oracle_e4m3.restype = ctypes.c_double
        lib.oracle_e4m3.argtypes = [ctypes.c_uint]
        lib.oracle_gemv_sums.restype = None
        lib.oracle_gemv_sums.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [
            ctypes.c_void_p, ctypes.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host cores this process may run on, capped by OMP_NUM_THREADS if set."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return n


def e2m1_table() -> np.ndarray:
    """Values of the 16 E2M1 codes, as float64."""
    lib = _load()
    return np.array([lib.oracle_e2m1(c) for c in range(16)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """Values of the 256 E4M3 (float8_e4m3fn) codes, as float64 (NaN at 0x7F, 0xFF)."""
    lib = _load()
    return np.array([lib.oracle_e4m3(c) for c in range(256)], dtype=np.float64)


def _check(A, sfA, x, sfx, l, m, k):
    if k % 16 != 0 or l < 1 or m < 1 or k < 16:
        raise ValueError(f"bad shape l={l} m={m} k={k}")
    want = {"A": (l, m, k // 2), "sfA": (l, m, k // 16), "x": (l, k // 2), "sfx": (l, k // 16)}
    got = {}
    for name, arr in (("A", A), ("sfA", sfA), ("x", x), ("sfx", sfx)):
        a = np.ascontiguousarray(np.asarray(arr, dtype=np.uint8)).reshape(want[name])
        got[name] = a
    return got


def gemv_sums(A, sfA, x, sfx, l, m, k, nthreads=None) -> np.ndarray:
    """S (l, m) in float64: the scaled dot products before alpha and rounding."""
    ops = _check(A, sfA, x, sfx, l, m, k)
    S = np.empty((l, m), dtype=np.float64)
    lib = _load()
    lib.oracle_gemv_sums(ops["A"].ctypes.data, ops["sfA"].ctypes.data,
                         ops["x"].ctypes.data, ops["sfx"].ctypes.data,
                         l, m, k, S.ctypes.data,
                         int(nthreads or default_threads()))
    return S


def epilogue(S, alpha) -> np.ndarray:
    """fp16 bit patterns (uint16) of f16(f32(alpha[b] * S[b, r]))."""
    S = np.asarray(S, dtype=np.float64)
    al = np.asarray(alpha, dtype=np.float32).astype(np.float64).reshape(-1, 1)
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = (al * S).astype(np.float32)
        return f32.astype(np.float16).view(np.uint16)


def gemv(A, sfA, x, sfx, alpha, l, m, k, nthreads=None) -> np.ndarray:
    """The oracle's output: fp16 bits, shape (l, m).  ``alpha=None`` means 1.0."""
    if alpha is None:
        alpha = np.ones(l, dtype=np.float32)
    S = gemv_sums(A, sfA, x, sfx, l, m, k, nthreads)
    return epilogue(S, alpha)


def gemv_rows(A, sfA, x, sfx, alpha, l, m, k, batch_rows, nthreads=None) -> np.ndarray:
    """Oracle outputs for selected (batch, row) pairs only, one at a time.

    ``batch_rows`` is an int array of shape (n, 2).  Returns uint16 fp16 bits of
    shape (n,).  Used to check full-size launches on sampled outputs.
    """
    ops = _check(A, sfA, x, sfx, l, m, k)
    if alpha is None:
        alpha = np.ones(l, dtype=np.float32)
    alpha = np.asarray(alpha, dtype=np.float32)
    br = np.asarray(batch_rows, dtype=np.int64).reshape(-1, 2)
    out = np.empty(len(br), dtype=np.uint16)
    for i, (b, r) in enumerate(br):
        s = gemv_sums(ops["A"][b, r], ops["sfA"][b, r], ops["x"][b], ops["sfx"][b],
                      1, 1, k, nthreads=1)
        out[i] = epilogue(s, alpha[b:b + 1])[0, 0]
    return out
