"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds input generation only: normal draws rounded to bf16, the
outlier mask, the per-expert token counts and the row -> group map of the
contiguous grouped layout.  It contains none of the
method's arithmetic (no quantization, no scales, no GEMM), and it imports
neither the oracle nor the HIP library.

Every tensor is drawn in fixed chunks of 2^20 elements (row-major order), chunk i
from its own numpy PCG64 stream ``default_rng([seed, tensor_id, i])``: any tensor can
be regenerated alone, and the chunks are drawn on several threads with a result that
does not depend on how many.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 20  # elements per independent stream


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _chunked(n: int, fn) -> None:
    """fn(i, lo, hi) for every chunk [lo, hi) of [0, n), on a thread pool."""
    nch = -(-n // CHUNK)
    if nch <= 1:
        if n:
            fn(0, 0, n)
        return
    with ThreadPoolExecutor(max_workers=min(_threads(), nch)) as ex:
        list(ex.map(lambda i: fn(i, i * CHUNK, min(n, (i + 1) * CHUNK)), range(nch)))

# tensor ids for the per-tensor streams
T_A, T_B, T_OUTLIER, T_X = 1, 2, 3, 5


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even) and return the uint16 bits.

    In uint32: for every finite value, bits + 0x7FFF + lsb stays below 2^32 (the largest
    finite pattern is 0xFF7FFFFF), so nothing wraps; NaNs are set afterwards."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.reshape(-1).view(np.uint32)
    out = np.empty(u.size, np.uint16)

    def part(i, lo, hi):
        x = u[lo:hi]
        r = x >> 16
        r &= 1
        r += x
        r += 0x7FFF
        r >>= 16
        o = out[lo:hi]
        o[:] = r
        nan = np.isnan(a.reshape(-1)[lo:hi])
        if nan.any():
            o[nan] = 0x7FC0

    _chunked(u.size, part)
    return out.reshape(a.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_f32(shape, std: float, seed: int, tensor_id: int, outliers=None) -> np.ndarray:
    """float32 N(0, std) draws; outliers = (frac, factor) multiplies a Bernoulli(frac) set
    of entries (their own streams, tensor id T_OUTLIER) by factor."""
    n = int(np.prod(shape))
    v = np.empty(n, np.float32)

    def part(i, lo, hi):
        x = v[lo:hi]
        np.random.default_rng([seed, tensor_id, i]).standard_normal(size=hi - lo, dtype=np.float32, out=x)
        x *= np.float32(std)
        if outliers is not None:
            frac, factor = outliers
            mask = np.random.default_rng([seed, T_OUTLIER, i]).random(size=hi - lo) < frac
            x[mask] *= np.float32(factor)

    _chunked(n, part)
    return v.reshape(shape)


def normal_bf16(shape, std: float = 1.0, seed: int = 0, tensor_id: int = T_A) -> np.ndarray:
    return f32_to_bf16_bits(_normal_f32(shape, std, seed, tensor_id))


def normal_bf16_outliers(shape, std: float = 1.0, frac: float = 0.01, factor: float = 50.0,
                         seed: int = 0, tensor_id: int = T_A) -> np.ndarray:
    """N(0, std) with an independent Bernoulli(frac) mask of entries multiplied by factor,
    applied before the bf16 rounding."""
    return f32_to_bf16_bits(_normal_f32(shape, std, seed, tensor_id, outliers=(frac, factor)))


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
