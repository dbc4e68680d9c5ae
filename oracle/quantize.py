"""BF16 -> NVFP4 quantiser of the CPU oracle (test infrastructure only).

It turns the Gaussian workload's bf16 values into the bytes both sides of the
parity check consume.  The steps follow ``quantize_to_nvfp4`` on the CuTeDSL
bridge page (section "Quantization"), in fp32 as the page computes them:

1. amax = max(max |T|, 1e-8) over the whole tensor T;
2. global scale g = amax / (6 * 448): the largest E2M1 value times the largest
   finite E4M3 value, so the scaled tensor fits the two formats together;
3. Tn = T / g;
4. per block of 16 consecutive elements along the last axis:
   bamax = max(max |block|, 1e-8) and block scale s = e4m3(bamax / 6), the cast
   being torch's float -> float8_e4m3fn (round to nearest even), as on the page;
5. v = block / max(float(s), 1e-8), magnitude clamped to 6;
6. E2M1 code = index of the nearest magnitude in {0, .5, 1, 1.5, 2, 3, 4, 6},
   plus 8 when v < 0;
7. pack two codes per byte, the even element in the low nibble.

Reading taken in step 6: the page offers two rules that disagree (a half-step
look-up table, and an argmin over distances in its weight quantiser).  This
oracle takes the nearest magnitude, and on an exact tie the even code (IEEE
round-to-nearest-even on the E2M1 grid).  The rule only decides which bytes are
generated: the GEMV never quantises, so parity does not depend on it.

Parity unpinned: the pages print no quantised values, so the tie rule and the
exact bytes are pinned only by the properties the tests check (round trip of
grid values, nearest-value property, error bound, scale range).
"""
from __future__ import annotations

import numpy as np

from .reference import e2m1_table, e4m3_table

_E2M1_GRID = None
_E4M3 = None


def _tables():
    global _E2M1_GRID, _E4M3
    if _E2M1_GRID is None:
        _E2M1_GRID = e2m1_table()[:8].copy()          # magnitudes of codes 0..7
        _E4M3 = e4m3_table()
    return _E2M1_GRID, _E4M3


def e2m1_nearest_index(mag) -> np.ndarray:
    """Index 0..7 of the E2M1 magnitude nearest to each ``mag`` (0 <= mag <= 6).

    The nearest grid value is found by counting the midpoints between
    neighbouring grid values that lie below ``mag`` (compared in float64, exact
    for fp32 inputs); a value exactly on a midpoint is a tie, and takes the even
    one of its two neighbours.
    """
    grid, _ = _tables()
    mid = (grid[:-1] + grid[1:]) / 2.0
    m64 = np.asarray(mag).astype(np.float64)
    idx = np.searchsorted(mid, m64, side="left")          # ties land on the lower neighbour
    tie = (idx < len(mid)) & (mid[np.minimum(idx, len(mid) - 1)] == m64)
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)
    return idx.astype(np.uint8)


def e4m3_encode(values) -> np.ndarray:
    """float32 -> float8_e4m3fn codes with torch's cast (round to nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(np.asarray(values, dtype=np.float32)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def quantize_nvfp4(t):
    """Quantise one tensor ``t`` (float32, last axis a multiple of 16).

    Returns (packed uint8 (..., K/2), block-scale codes uint8 (..., K/16),
    global scale float32).
    """
    t = np.asarray(t, dtype=np.float32)
    K = t.shape[-1]
    if K % 16 != 0:
        raise ValueError("last axis must be a multiple of 16")
    _, e4m3 = _tables()
    amax = np.float32(max(np.float32(np.abs(t).max()), np.float32(1e-8)))
    g = np.float32(amax / np.float32(6.0 * 448.0))
    tn = t / g
    blocks = tn.reshape(*t.shape[:-1], K // 16, 16)
    bamax = np.maximum(np.abs(blocks).max(axis=-1), np.float32(1e-8))
    scale_codes = e4m3_encode(bamax / np.float32(6.0))
    scale_vals = e4m3[scale_codes].astype(np.float32)
    v = blocks / np.maximum(scale_vals, np.float32(1e-8))[..., None]
    mag = np.minimum(np.abs(v), np.float32(6.0))
    idx = e2m1_nearest_index(mag)
    codes = np.where(v < 0, idx + 8, idx).astype(np.uint8).reshape(t.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale_codes, g


def gaussian_operands(raw, l, m, k):
    """NVFP4 operands of the Gaussian workload from its bf16 draws.

    ``raw`` holds float32 arrays A (l, m, k) and x (l, k).  Each batch's A[b]
    and x[b] are quantised as separate tensors, each with its own global scale;
    alpha[b] = f32(gA[b] * gx[b]) carries both into the GEMV.
    """
    A = np.empty((l, m, k // 2), dtype=np.uint8)
    sfA = np.empty((l, m, k // 16), dtype=np.uint8)
    x = np.empty((l, k // 2), dtype=np.uint8)
    sfx = np.empty((l, k // 16), dtype=np.uint8)
    alpha = np.empty(l, dtype=np.float32)
    for b in range(l):
        A[b], sfA[b], ga = quantize_nvfp4(raw["A"][b])
        x[b], sfx[b], gx = quantize_nvfp4(raw["x"][b])
        alpha[b] = np.float32(ga * gx)
    return {"A": A, "sfA": sfA, "x": x, "sfx": sfx, "alpha": alpha}


def dequantize(packed, scale_codes, g) -> np.ndarray:
    """float64 values represented by quantised bytes (for round-trip tests)."""
    e2m1 = e2m1_table()
    _, e4m3 = _tables()
    packed = np.asarray(packed, dtype=np.uint8)
    codes = np.stack([packed & 15, packed >> 4], axis=-1).reshape(*packed.shape[:-1], -1)
    vals = e2m1[codes]
    K = vals.shape[-1]
    sv = e4m3[np.asarray(scale_codes)]
    return (vals.reshape(*vals.shape[:-1], K // 16, 16) * sv[..., None]).reshape(vals.shape) * float(g)
