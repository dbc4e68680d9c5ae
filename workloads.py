"""Seeded synthetic inputs for the NVFP4 block-scaled batched GEMV.

This module only draws random numbers and lays them out in the storage order
the GEMV reads.  It contains none of the operation's arithmetic (no E2M1 or
E4M3 decode, no products, no sums, no quantisation), so both the CPU oracle and
the GPU path can take their inputs from it without sharing any of the method.

Storage order (row-major, contiguous, batch outermost), following the tensors
built in "nvFP4 Batch GEMV算子系列(下)", section 准备数据, before their
permute to (m, k/2, l):

    A     uint8 (l, m, k/2)   two E2M1 codes per byte, element 2i in bits 3:0
    sfA   uint8 (l, m, k/16)  one E4M3 code per 16 consecutive k
    x     uint8 (l, k/2)      packed like A
    sfx   uint8 (l, k/16)     like sfA
    alpha float32 (l,)        per-batch global scale

Two generators:

* integer-coded: every byte of A and x uniform in 0..255 (i.e. both nibbles
  uniform over all 16 E2M1 codes), block scales drawn uniformly from the
  integers {0, 1, 2} and stored as their E4M3 codes, as the blog post's data
  preparation does with ``randint(0, 3)`` cast to ``float8_e4m3fn``;
* Gaussian: A and x drawn N(0, 1) in float32 and rounded to bfloat16, the
  input of the BF16 -> NVFP4 quantiser on the CuTeDSL bridge page (section
  "Quantization"). Turning them into NVFP4 bytes is the quantiser's job, not
  this module's.

Draw order is fixed: A, sfA, x, sfx, alpha for integer-coded inputs; per batch
A[l] then x[l] for Gaussian inputs.  numpy's PCG64 (``default_rng``) is the
generator, seed 0 unless stated.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# E4M3 (float8_e4m3fn) codes of the integers 0, 1 and 2: 0x00, 0x38 (exponent
# field 7 = bias, mantissa 0) and 0x40 (exponent field 8).  A not-gpu test
# checks them against torch's own float -> float8_e4m3fn cast.
INT_SCALE_CODES = np.array([0x00, 0x38, 0x40], dtype=np.uint8)


@dataclass(frozen=True)
class Config:
    name: str
    l: int
    m: int
    k: int
    kind: str          # "integer" or "gaussian"
    alpha: str         # "one", "uniform" (U[0.5, 2] per batch) or "quantizer"
    seed: int = 0
    note: str = ""

    @property
    def bytes_moved(self) -> int:
        """Algorithmic HBM bytes of one GEMV: A + sfA + x + sfx + c."""
        l, m, k = self.l, self.m, self.k
        return l * m * k // 2 + l * m * k // 16 + l * k // 2 + l * k // 16 + 2 * l * m


# The five workloads the GEMV is measured and checked on.
CONFIGS = {
    "tiny": Config("tiny", 1, 128, 256, "integer", "one",
                   note="tiny single matrix"),
    "decode": Config("decode", 1, 7168, 16384, "integer", "one",
                     note="single large weight, decode-style"),
    "batched": Config("batched", 8, 4096, 7168, "integer", "uniform",
                      note="8 independent batches, per-batch alpha"),
    "shortk": Config("shortk", 4, 7168, 2048, "integer", "one",
                     note="short K, many rows"),
    "gaussian": Config("gaussian", 16, 2048, 4096, "gaussian", "quantizer",
                       note="bf16 N(0,1) quantised to NVFP4 per batch"),
}


def integer_coded(l: int, m: int, k: int, seed: int = 0, alpha: str = "one"):
    """Integer-coded NVFP4 operands as raw bytes.

    Returns a dict with uint8 arrays A (l,m,k/2), sfA (l,m,k/16), x (l,k/2),
    sfx (l,k/16) and float32 alpha (l,).
    """
    if k % 16 != 0:
        raise ValueError("k must be a multiple of 16")
    rng = np.random.default_rng(seed)
    A = rng.integers(0, 256, size=(l, m, k // 2), dtype=np.uint8)
    sfA = INT_SCALE_CODES[rng.integers(0, 3, size=(l, m, k // 16))]
    x = rng.integers(0, 256, size=(l, k // 2), dtype=np.uint8)
    sfx = INT_SCALE_CODES[rng.integers(0, 3, size=(l, k // 16))]
    if alpha == "one":
        al = np.ones(l, dtype=np.float32)
    elif alpha == "uniform":
        al = rng.uniform(0.5, 2.0, size=l).astype(np.float32)
    else:
        raise ValueError(f"unknown alpha mode {alpha!r}")
    return {"A": A, "sfA": np.ascontiguousarray(sfA), "x": x,
            "sfx": np.ascontiguousarray(sfx), "alpha": al}


def random_bytes(l: int, m: int, k: int, seed: int = 0, scale_codes=None):
    """Arbitrary bytes everywhere (scales drawn from ``scale_codes``, default all
    256 codes).  Used for edge-case tests (NaN, negative and subnormal scales)."""
    rng = np.random.default_rng(seed)
    if scale_codes is None:
        scale_codes = np.arange(256, dtype=np.uint8)
    scale_codes = np.asarray(scale_codes, dtype=np.uint8)
    A = rng.integers(0, 256, size=(l, m, k // 2), dtype=np.uint8)
    sfA = scale_codes[rng.integers(0, len(scale_codes), size=(l, m, k // 16))]
    x = rng.integers(0, 256, size=(l, k // 2), dtype=np.uint8)
    sfx = scale_codes[rng.integers(0, len(scale_codes), size=(l, k // 16))]
    al = rng.uniform(0.5, 2.0, size=l).astype(np.float32)
    return {"A": A, "sfA": np.ascontiguousarray(sfA), "x": x,
            "sfx": np.ascontiguousarray(sfx), "alpha": al}


def gaussian_bf16(l: int, m: int, k: int, seed: int = 0):
    """Gaussian operands before quantisation: float32 arrays holding bf16 values.

    A is (l, m, k) and x is (l, k); both are N(0, 1) draws rounded to bfloat16
    (round-to-nearest-even, by torch's own cast) and widened back to float32.
    """
    import torch

    rng = np.random.default_rng(seed)
    A = np.empty((l, m, k), dtype=np.float32)
    x = np.empty((l, k), dtype=np.float32)
    for b in range(l):
        a32 = rng.standard_normal(size=(m, k), dtype=np.float32)
        x32 = rng.standard_normal(size=(k,), dtype=np.float32)
        A[b] = torch.from_numpy(a32).to(torch.bfloat16).float().numpy()
        x[b] = torch.from_numpy(x32).to(torch.bfloat16).float().numpy()
    return {"A": A, "x": x}


def for_config(cfg: Config):
    """Raw inputs of an integer-coded config (Gaussian configs need the
    quantiser on top of :func:`gaussian_bf16`)."""
    if cfg.kind != "integer":
        raise ValueError(f"{cfg.name} is not integer-coded")
    return integer_coded(cfg.l, cfg.m, cfg.k, cfg.seed, cfg.alpha)


def bf16_bits(values) -> np.ndarray:
    """Bit patterns (uint16) of float32 values that hold bf16 numbers: the upper
    half of each float32 word (a pure re-encoding, no rounding)."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    return (v.view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class ActConfig:
    """A bf16 activation batch for the activation quantiser: ``rows`` vectors
    of length ``d``, N(0, 1) rounded to bf16."""
    name: str
    rows: int
    d: int
    seed: int = 0
    note: str = ""

    @property
    def bytes_moved(self) -> int:
        """Algorithmic HBM bytes of one quantisation: bf16 in, codes and block
        scales out (the per-row global scales are 4 bytes a row)."""
        n = self.rows * self.d
        return 2 * n + n // 2 + n // 16 + 4 * self.rows


ACT_CONFIGS = {
    "decode_x": ActConfig("decode_x", 1, 16384,
                          note="the decode workload's activation vector (k = 16384)"),
    "tokens": ActConfig("tokens", 4096, 7168,
                        note="4096 token activations of the batched workload's K (7168)"),
}


def activation_bf16(cfg: ActConfig) -> np.ndarray:
    """float32 (rows, d) holding bf16 values, N(0, 1)."""
    return gaussian_bf16(1, cfg.rows, cfg.d, seed=cfg.seed)["A"][0]


@dataclass(frozen=True)
class SmallNConfig:
    """n integer-coded vectors per batch against one integer-coded weight
    matrix per batch (A (l, m, k/2), B (l, n, k/2))."""
    name: str
    l: int
    m: int
    n: int
    k: int
    seed: int = 0
    note: str = ""

    @property
    def bytes_moved(self) -> int:
        l, m, n, k = self.l, self.m, self.n, self.k
        return l * m * k * 9 // 16 + l * n * k * 9 // 16 + 2 * l * m * n + 4 * l


SMALLN_CONFIGS = {
    "tiny_n3": SmallNConfig("tiny_n3", 2, 80, 3, 256, note="tiny, ragged rows"),
    "decode_n1": SmallNConfig("decode_n1", 1, 7168, 1, 16384,
                              note="the decode weight against 1 vector (the GEMV through the GEMM call)"),
    "decode_n2": SmallNConfig("decode_n2", 1, 7168, 2, 16384,
                              note="the decode weight against 2 vectors (one speculative token)"),
    "decode_n4": SmallNConfig("decode_n4", 1, 7168, 4, 16384,
                              note="the decode weight against 4 vectors (speculative tokens)"),
    "decode_n8": SmallNConfig("decode_n8", 1, 7168, 8, 16384,
                              note="the decode weight against 8 vectors"),
    "decode_n16": SmallNConfig("decode_n16", 1, 7168, 16, 16384,
                               note="the decode weight against 16 vectors (a decode batch)"),
}


def smalln_operands(cfg: SmallNConfig):
    """A, sfA (l, m, .), B, sfB (l, n, .), alpha (l,) U[0.5, 2]."""
    a = integer_coded(cfg.l, cfg.m, cfg.k, seed=cfg.seed, alpha="uniform")
    b = integer_coded(cfg.l, cfg.n, cfg.k, seed=cfg.seed + 1)
    return {"A": a["A"], "sfA": a["sfA"], "B": b["A"], "sfB": b["sfA"], "alpha": a["alpha"]}


@dataclass(frozen=True)
class MoeConfig:
    """Grouped (MoE) GEMV: ``tokens`` token rows already grouped by expert, the
    count of each expert drawn from a seeded multinomial (some experts get
    none), integer-coded activations and expert weights (experts, n, k/2),
    per-expert global scales U[0.5, 2]."""
    name: str
    experts: int
    n: int
    k: int
    tokens: int
    seed: int = 0
    note: str = ""


MOE_CONFIGS = {
    "moe_tiny": MoeConfig("moe_tiny", 6, 96, 256, 20, note="tiny, ragged rows"),
    "moe_decode": MoeConfig("moe_decode", 64, 2048, 7168, 128,
                            note="64 experts of 2048 x 7168, 128 routed token slots"),
}


def moe_operands(cfg: MoeConfig):
    """X, sfX (tokens, .), W, sfW (experts, n, .), offsets int32 (experts,)
    cumulative token counts, gs_x, gs_w (experts,)."""
    rng = np.random.default_rng(cfg.seed + 1000)
    counts = rng.multinomial(cfg.tokens, np.full(cfg.experts, 1.0 / cfg.experts))
    offsets = np.cumsum(counts).astype(np.int32)
    gs_x = rng.uniform(0.5, 2.0, size=cfg.experts).astype(np.float32)
    gs_w = rng.uniform(0.5, 2.0, size=cfg.experts).astype(np.float32)
    w = integer_coded(cfg.experts, cfg.n, cfg.k, seed=cfg.seed)
    x = integer_coded(1, cfg.tokens, cfg.k, seed=cfg.seed + 1)
    return {"X": x["A"][0], "sfX": x["sfA"][0], "W": w["A"], "sfW": w["sfA"], "offsets": offsets,
            "gs_x": gs_x, "gs_w": gs_w}


def moe_bytes_moved(cfg: MoeConfig, offsets) -> int:
    """Algorithmic bytes of one grouped call: the weights of experts with at
    least one token, the token activations, the outputs (bf16)."""
    counts = np.diff(np.concatenate([[0], np.asarray(offsets, dtype=np.int64)]))
    active = int((counts > 0).sum())
    return active * cfg.n * cfg.k * 9 // 16 + cfg.tokens * cfg.k * 9 // 16 + 2 * cfg.tokens * cfg.n
