"""GPU parity of the pre-shuffled weight layout and of the dense GEMM that reads it.

The shuffle kernel must reproduce the oracle's byte permutation bit for bit.  The
GEMM on shuffled weights is compared element by element with the oracle's double
result on the unshuffled weights (|C_gpu - ref| <= 1e-2 |ref| + 1e-2 rms(ref)), and
with the plain-layout GEMM of the same tile and split: the shuffle only moves each
weight byte to the lane and register the plain kernel loads it into, so the two
results must be bit-identical.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_token_amd as F
import oracle as O
import workloads as W
from gpu_helpers import DEV, gemm_tolerance_check, poisoned_bf16, sync, to_dev, to_host

pytestmark = pytest.mark.gpu

SHUF = F.LAYOUT_DENSE_PRESHUFFLED


def _shuffled(qb: np.ndarray) -> torch.Tensor:
    return F.fp8_weight_preshuffle(to_dev(qb))


@pytest.mark.parametrize("rows,K", [(32, 128), (64, 640), (96, 1152), (4 * 256, 512), (7168, 18432)])
def test_preshuffle_bit_exact(rows, K):
    print("preshuffle %dx%d" % (rows, K), flush=True)
    w = np.random.default_rng(rows + K).integers(0, 256, (rows, K), dtype=np.uint8)
    out = F.fp8_weight_preshuffle(to_dev(w))
    sync()
    assert np.array_equal(to_host(out), O.weight_preshuffle(w))


def test_preshuffle_experts_flattened():
    """[E, N, K] expert weights shuffle as E*N rows: each expert's block equals its own shuffle."""
    w = np.random.default_rng(3).integers(0, 256, (3, 128, 256), dtype=np.uint8)
    out = to_host(F.fp8_weight_preshuffle(to_dev(w)))
    sync()
    for e in range(3):
        assert np.array_equal(out[e], O.weight_preshuffle(w[e]))


SMALL = [(1, 64, 128), (17, 192, 384), (64, 512, 1024), (100, 640, 640), (130, 256, 512), (64, 128, 2560)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_preshuffled_gemm_every_entry(M, N, K):
    print("preshuffled gemm %dx%dx%d" % (M, N, K), flush=True)
    rng_seed = M + N + K
    a = W.normal_bf16((M, K), seed=rng_seed)
    b = W.normal_bf16((N, K), std=1.0, seed=rng_seed, tensor_id=W.T_B)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    ref = O.gemm_nt(qa, sfa, qb, sfb)
    da, dsa, dsb = to_dev(qa), to_dev(sfa), to_dev(sfb)
    db = _shuffled(qb)
    entries = [k for k in range(F.gemm_config_count()) if F.gemm_config_of(k, SHUF, M, N, K) is not None]
    assert entries
    for kernel in entries:
        for splits in (1, 2, 3, 5):
            c = F.fp8_block_gemm_nt_preshuffled(da, dsa, db, dsb, c=poisoned_bf16(M, N), kernel=kernel,
                                                splits=splits)
            sync()
            gemm_tolerance_check(to_host(c), ref, "kernel %d splits %d %dx%dx%d" % (kernel, splits, M, N, K))
    c = F.fp8_block_gemm_nt_preshuffled(da, dsa, db, dsb, c=poisoned_bf16(M, N))
    sync()
    gemm_tolerance_check(to_host(c), ref, "auto")


def test_preshuffled_decode_shape_matches_plain_and_oracle():
    """64 x 7168 x 18432 with 1% x50 outliers: the automatic pre-shuffled call equals the
    plain-layout decode kernel with the same tile and split bit for bit, is
    deterministic, and agrees with the oracle on 16 sampled rows (every column)."""
    s = W.DENSE_DECODE
    a, b = W.dense_inputs(s)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    da, dsa, db, dsb = to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb)
    dbs = F.fp8_weight_preshuffle(db)
    cfg = F.gemm_config(SHUF, s.M, s.N, s.K)
    print("preshuffled decode cfg", cfg, flush=True)
    c1 = to_host(F.fp8_block_gemm_nt_preshuffled(da, dsa, dbs, dsb, c=poisoned_bf16(s.M, s.N)))
    c2 = to_host(F.fp8_block_gemm_nt_preshuffled(da, dsa, dbs, dsb, c=poisoned_bf16(s.M, s.N)))
    sync()
    assert np.array_equal(c1, c2)
    # the plain-layout entry of the same kernel shape and reduction
    plain = [k for k in range(F.gemm_config_count())
             if (F.gemm_config_of(k, False, s.M, s.N, s.K, cfg["splits"]) or {}).get("splits") == cfg["splits"]
             and F.gemm_config_of(k, False, s.M, s.N, s.K, cfg["splits"])["bn"] == cfg["bn"]]
    matched = False
    for k in plain:
        cp = to_host(F.fp8_block_gemm_nt(da, dsa, db, dsb, c=poisoned_bf16(s.M, s.N), kernel=k,
                                         splits=cfg["splits"]))
        sync()
        matched = matched or np.array_equal(cp, c1)
    assert matched, "no plain-layout entry with the same tile and split reproduces the bits"
    rows = np.unique(np.linspace(0, s.M - 1, 16).astype(np.int64))
    ref = O.gemm_nt(qa, sfa, qb, sfb, rows=rows)
    gemm_tolerance_check(c1[rows], ref, s.name)
