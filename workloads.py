"""Seeded synthetic inputs and workload shapes.

This module is shared by the tests, the benchmark and the oracle checks.  It
holds random-number generation and shapes only -- none of the quantization or
GEMM arithmetic -- so that the HIP path and the oracle never share code.

Every generator uses numpy's PCG64 seeded with SeedSequence([seed, workload_id,
tensor_id]), seed 0 by default.

Workloads (the pages run whole Qwen3.5/3.6 models, whose weights are not
available; these synthetic tensors of the stated shapes stand in for them):

  small   Q8_0 x Q8_0 GEMM M=16, K=256, N=512; W ~ N(0, 0.02), A ~ N(0, 1)
  decode  GEMV M in {1, 4, 16}, K=4096, N=12288; W ~ N(0, 0.02), A ~ N(0, 1)
  prefill GEMM M=2048, K=5120, N=17408; W ~ N(0, 0.02), A ~ N(0, 1)
  long    GEMM M=18432, K=5120, N=5120; A ~ Student-t(3) with 1% of the K
          columns (51 distinct, seeded) scaled by 20; W ~ N(0, 0.02)
  moe     grouped W4A8: 947 tokens, top-8 of 128 experts (uniformly random
          8-subsets, kept in permutation order), K=2048, N=768 per expert;
          W ~ N(0, 0.02) per expert; A ~ N(0, 1)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

WORKLOAD_IDS = {"small": 0, "decode": 1, "prefill": 2, "long": 3, "moe": 4}

# tensor ids within a workload
T_ACT, T_WEIGHT, T_IDS, T_OUTLIER_COLS, T_W4_CODES, T_W4_SCALES = range(6)


@dataclass(frozen=True)
class GemmShape:
    name: str
    m: int
    k: int
    n: int


SMALL = GemmShape("small", 16, 256, 512)
DECODE = [GemmShape("decode_m%d" % m, m, 4096, 12288) for m in (1, 4, 16)]
PREFILL = GemmShape("prefill", 2048, 5120, 17408)
# a short prompt against the same weights: 136 output tiles, fewer than CUs
PREFILL_SHORT = GemmShape("prefill_short", 128, 5120, 17408)
LONG = GemmShape("long", 18432, 5120, 5120)


@dataclass(frozen=True)
class MoeShape:
    name: str
    tokens: int
    top_k: int
    experts: int
    k: int
    n: int


MOE = MoeShape("moe", 947, 8, 128, 2048, 768)


def rng(workload: str | int, tensor: int, seed: int = 0) -> np.random.Generator:
    wid = WORKLOAD_IDS[workload] if isinstance(workload, str) else int(workload)
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, tensor])))


def normal(workload, tensor, shape, std=1.0, seed=0) -> np.ndarray:
    g = rng(workload, tensor, seed)
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def activations(workload: str, m: int, k: int, seed: int = 0) -> np.ndarray:
    """Activation matrix [m][k] fp32 for a workload."""
    if workload == "long":
        g = rng(workload, T_ACT, seed)
        a = g.standard_t(3, size=(m, k)).astype(np.float32)
        cols = rng(workload, T_OUTLIER_COLS, seed).choice(k, size=k // 100, replace=False)
        a[:, cols] *= np.float32(20.0)
        return a
    return normal(workload, T_ACT, (m, k), 1.0, seed)


def outlier_columns(k: int, seed: int = 0) -> np.ndarray:
    return np.sort(rng("long", T_OUTLIER_COLS, seed).choice(k, size=k // 100, replace=False))


def weights(workload: str, n: int, k: int, seed: int = 0, experts: int | None = None) -> np.ndarray:
    """Weight matrix [n][k] (or [experts][n][k]) fp32 ~ N(0, 0.02)."""
    shape = (n, k) if experts is None else (experts, n, k)
    return normal(workload, T_WEIGHT, shape, 0.02, seed)


def topk_ids(tokens: int, top_k: int, experts: int, seed: int = 0, workload="moe") -> np.ndarray:
    """Uniform random router: each token takes the first top_k entries of a
    seeded permutation of the experts.  int32 [tokens][top_k]."""
    g = rng(workload, T_IDS, seed)
    ids = np.empty((tokens, top_k), np.int32)
    for t in range(tokens):
        ids[t] = g.permutation(experts)[:top_k]
    return ids


def random_w4_codes(experts: int, n: int, k: int, seed: int = 0, workload="moe"):
    """Uniform random packed 4-bit codes (every byte = two codes 0..15)
    [experts][n][k/2] uint8, and random fp16 scales [experts][n][k/32] whose
    values are 2^u with u uniform in [-12, -5] times a uniform mantissa."""
    g = rng(workload, T_W4_CODES, seed)
    packed = g.integers(0, 256, size=(experts, n, k // 2), dtype=np.uint8)
    gs = rng(workload, T_W4_SCALES, seed)
    e = gs.integers(-12, -5, size=(experts, n, k // 32))
    mant = gs.uniform(1.0, 2.0, size=(experts, n, k // 32))
    scales = np.ldexp(mant, e).astype(np.float16).view(np.uint16)
    return packed, scales


def random_int8(workload, tensor, shape, seed=0) -> np.ndarray:
    """Uniform random int8 codes over the full range -128..127."""
    return rng(workload, tensor, seed).integers(-128, 128, size=shape, dtype=np.int8)


def random_scales(workload, tensor, shape, lo=-12, hi=-2, seed=0) -> np.ndarray:
    """Random normal-range fp16 scales (bits)."""
    g = rng(workload, tensor, seed)
    e = g.integers(lo, hi, size=shape)
    mant = g.uniform(1.0, 2.0, size=shape)
    return np.ldexp(mant, e).astype(np.float16).view(np.uint16)
