"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds input generation only: normal draws rounded to bf16, the
outlier mask, the per-expert token counts and the row -> group map of the
contiguous grouped layout.  It contains none of the
method's arithmetic (no quantization, no scales, no GEMM), and it imports
neither the oracle nor the HIP library.

Every tensor has its own numpy PCG64 stream, ``default_rng([seed, tensor_id])``,
so any tensor can be regenerated alone.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# tensor ids for the per-tensor streams
T_A, T_B, T_OUTLIER, T_X = 1, 2, 3, 5


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, std: float = 1.0, seed: int = 0, tensor_id: int = T_A) -> np.ndarray:
    rng = np.random.default_rng([seed, tensor_id])
    v = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return f32_to_bf16_bits(v)


def normal_bf16_outliers(shape, std: float = 1.0, frac: float = 0.01, factor: float = 50.0,
                         seed: int = 0, tensor_id: int = T_A) -> np.ndarray:
    """N(0, std) with an independent Bernoulli(frac) mask of entries multiplied by factor,
    applied before the bf16 rounding."""
    rng = np.random.default_rng([seed, tensor_id])
    v = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    mask = np.random.default_rng([seed, T_OUTLIER]).random(size=shape) < frac
    v = np.where(mask, v * np.float32(factor), v).astype(np.float32)
    return f32_to_bf16_bits(v)


def zipf_counts(E: int = 32, tokens: int = 4096, s: float = 1.1, cap: int = 256, seed: int = 0) -> np.ndarray:
    """Per-expert valid-row counts: Multinomial(tokens, p_e ~ (e+1)^-s), each capped at cap.

    Drawn from ``default_rng(seed)`` directly (seed 0: 2780 valid rows, 3 experts at the cap)."""
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    draw = np.random.default_rng(seed).multinomial(tokens, p)
    return np.minimum(draw, cap).astype(np.int32)


def topk_routing(T: int = 512, topk: int = 8, E: int = 32, s: float = 1.1, seed: int = 0) -> np.ndarray:
    """Expert choices int32 [T, topk]: for every token, topk distinct experts drawn without
    replacement with weights p_e ~ (e+1)^-s (the masked workload's Zipf skew), from
    ``default_rng([seed, 7])``."""
    p = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    p /= p.sum()
    rng = np.random.default_rng([seed, 7])
    return np.stack([rng.choice(E, size=topk, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def contiguous_layout(counts, align: int = 128, tail_blocks: int = 0) -> np.ndarray:
    """Row -> group map of the contiguous grouped layout: group g's rows in a run of
    round_up(counts[g], align) rows (the first counts[g] name g, the rest are padding,
    -1), then tail_blocks runs of padding only."""
    parts = []
    for g, c in enumerate(np.asarray(counts, np.int64)):
        run = -(-int(c) // align) * align
        parts.append(np.concatenate([np.full(int(c), g, np.int32), np.full(run - int(c), -1, np.int32)]))
    parts.append(np.full(tail_blocks * align, -1, np.int32))
    return np.concatenate(parts).astype(np.int32)


@dataclasses.dataclass(frozen=True)
class DenseShape:
    name: str
    M: int
    N: int
    K: int
    outliers: bool = False


# The dense workloads: a small parity case, the decode shape, and the prefill sweep.
DENSE_SMALL = DenseShape("dense_8x512x512", 8, 512, 512)
DENSE_DECODE = DenseShape("dense_decode_64x7168x18432", 64, 7168, 18432, outliers=True)
DENSE_PREFILL = tuple(
    DenseShape("dense_prefill_%dx%dx%d" % (m, n, k), m, n, k)
    for (n, k) in ((4096, 7168), (18432, 7168))
    for m in (1024, 2048, 4096)
)

# Masked MoE workloads: 32 experts, rows padded to 256, Zipf(1.1) counts over 4096 tokens.
MOE_E, MOE_M_MAX, MOE_TOKENS = 32, 256, 4096
MOE_GATE_UP = dict(N=4096, K=7168)
MOE_DOWN = dict(N=7168, K=2048, H=2048)


def dense_inputs(shape: DenseShape, seed: int = 0):
    """(A bf16 [M, K], B bf16 [N, K]); A ~ N(0,1) (with outliers if the shape says so),
    B ~ N(0, 0.02)."""
    if shape.outliers:
        a = normal_bf16_outliers((shape.M, shape.K), seed=seed, tensor_id=T_A)
    else:
        a = normal_bf16((shape.M, shape.K), seed=seed, tensor_id=T_A)
    b = normal_bf16((shape.N, shape.K), std=0.02, seed=seed, tensor_id=T_B)
    return a, b
