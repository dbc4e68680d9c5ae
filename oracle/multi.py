"""CPU oracle for several NVFP4 vectors against block-scaled weights (test
infrastructure only: only tests, the smoke check and the benchmark's
CPU-baseline leg use it).

Both operations are the batched GEMV's scaled dot product applied to more
than one vector per weight matrix; every sum is the plain C fp64 sum of
``reference.gemv_sums`` (increasing k), so nothing here re-implements the
decode or the sum.

* small-N GEMM (the blog post's ``ref_kernel`` computes a scaled matrix
  product with N padded for the library call, "nvFP4 Batch GEMV算子系列(下)",
  section "pytorch实现NVFP4 batch gemv"; here N = n is used as is):

      C[b, r, j] = out( f32( alpha[b] * S ) ),
      S = sum_k e2m1(A[b,r,k]) e4m3(sfA[b,r,k//16]) e2m1(B[b,j,k]) e4m3(sfB[b,j,k//16])

  with A (l, m, k/2), B (l, n, k/2), C (l, m, n);

* grouped (MoE) GEMV (the CuTeDSL bridge page's 2Dx3D grouped GEMM, section
  "Kernel Launch", with one output column per token):  token rows
  offs[e-1] <= t < offs[e] (offs[-1] = 0, offsets cumulative as the page's
  ``compute_expert_offsets`` builds them) belong to expert e and

      C[t, r] = out( f32( f32(gs_x[e] * gs_w[e]) * S ) ),
      S = sum_k e2m1(X[t,k]) e4m3(sfX[t,k//16]) e2m1(W[e,r,k]) e4m3(sfW[e,r,k//16])

  with X (T, k/2), W (E, n, k/2), C (T, n); a missing scale array means 1;
  rows t >= offs[E-1] are not written.

``out`` is fp16 (the blog post's output type) or bf16 (the bridge page's),
each by IEEE round-to-nearest-even from the fp32 product (torch's casts).
"""
from __future__ import annotations

import numpy as np

from . import reference as ref


def round_f32_to(f32, out: str) -> np.ndarray:
    """uint16 bit patterns of float32 values rounded to fp16 or bf16 (RNE)."""
    import torch

    f32 = np.ascontiguousarray(np.asarray(f32, dtype=np.float32))
    if out == "f16":
        with np.errstate(over="ignore", invalid="ignore"):
            return f32.astype(np.float16).view(np.uint16)
    if out == "bf16":
        t = torch.from_numpy(f32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(out)


def scale_sums(S, alpha, out: str) -> np.ndarray:
    """out(f32(alpha * S)); alpha broadcasts against S."""
    with np.errstate(over="ignore", invalid="ignore"):
        f32 = (np.asarray(alpha, dtype=np.float32).astype(np.float64) *
               np.asarray(S, dtype=np.float64)).astype(np.float32)
    return round_f32_to(f32, out)


def gemm_smalln_sums(A, sfA, B, sfB, l, m, n, k, nthreads=None) -> np.ndarray:
    """S (l, m, n) in float64."""
    B = np.asarray(B, dtype=np.uint8).reshape(l, n, k // 2)
    sfB = np.asarray(sfB, dtype=np.uint8).reshape(l, n, k // 16)
    S = np.empty((l, m, n), dtype=np.float64)
    for j in range(n):
        S[:, :, j] = ref.gemv_sums(A, sfA, np.ascontiguousarray(B[:, j]),
                                   np.ascontiguousarray(sfB[:, j]), l, m, k, nthreads)
    return S


def gemm_smalln(A, sfA, B, sfB, alpha, l, m, n, k, out="f16", nthreads=None) -> np.ndarray:
    """C (l, m, n) as uint16 bit patterns.  ``alpha=None`` means 1."""
    S = gemm_smalln_sums(A, sfA, B, sfB, l, m, n, k, nthreads)
    al = np.ones(l, dtype=np.float32) if alpha is None else np.asarray(alpha, dtype=np.float32)
    return scale_sums(S, al.reshape(l, 1, 1), out)


def expert_ranges(offsets, experts):
    """[(first token, end token)] per expert from cumulative offsets."""
    offs = [int(v) for v in np.asarray(offsets).reshape(experts)]
    out, prev = [], 0
    for e in range(experts):
        out.append((prev, offs[e]))
        prev = offs[e]
    return out


def grouped_gemv(X, sfX, W, sfW, offsets, gs_x, gs_w, tokens, experts, n, k, out="bf16",
                 fill=0xFFFF, nthreads=None) -> np.ndarray:
    """C (tokens, n) as uint16 bit patterns; rows no expert covers hold ``fill``."""
    X = np.asarray(X, dtype=np.uint8).reshape(tokens, k // 2)
    sfX = np.asarray(sfX, dtype=np.uint8).reshape(tokens, k // 16)
    W = np.asarray(W, dtype=np.uint8).reshape(experts, n, k // 2)
    sfW = np.asarray(sfW, dtype=np.uint8).reshape(experts, n, k // 16)
    C = np.full((tokens, n), fill, dtype=np.uint16)
    for e, (t0, t1) in enumerate(expert_ranges(offsets, experts)):
        if t1 <= t0:
            continue
        gx = np.float32(1.0) if gs_x is None else np.float32(gs_x[e])
        gw = np.float32(1.0) if gs_w is None else np.float32(gs_w[e])
        alpha = np.float32(gx * gw)
        for t in range(t0, t1):
            S = ref.gemv_sums(W[e:e + 1], sfW[e:e + 1], X[t:t + 1], sfX[t:t + 1], 1, n, k, nthreads)
            C[t] = scale_sums(S[0], alpha, out)
    return C
