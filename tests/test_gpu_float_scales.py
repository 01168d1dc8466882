"""GPU parity of the float-scale (non-UE8M0) format: activation group quant and
weight block quant bit-exact against the oracle (same fp32 IEEE steps), and the
float-scale GEMM within the GEMM tolerance for every float-scale tile entry."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_token_amd as F
import oracle as O
import workloads as W
from gpu_helpers import DEV, gemm_tolerance_check, poisoned_bf16, sync, to_dev, to_host

pytestmark = pytest.mark.gpu

FLOAT = F.LAYOUT_DENSE_FLOAT
SF_CANARY = -12345.5


def _quant(x, ld_sf=None):
    M, K = x.shape
    ld = ld_sf if ld_sf is not None else max(4, -(-M // 4) * 4)
    sf = torch.full((K // 128, ld), SF_CANARY, dtype=torch.float32, device=DEV)
    q, sf = F.fp8_quant_group_float(to_dev(x), sf=sf)
    sync()
    return q.cpu().numpy(), sf.cpu().numpy()


@pytest.mark.parametrize("M,K,ld_sf", [(1, 128, None), (33, 640, 40), (300, 2048, None), (1024, 7168, None)])
def test_float_quant_bit_exact(M, K, ld_sf):
    x = W.normal_bf16_outliers((M, K), seed=M + K)
    q, sf = _quant(x, ld_sf)
    q_ref, sf_ref = O.quant_group_float(x, ld_sf=sf.shape[1])
    assert np.array_equal(q, q_ref)
    assert np.array_equal(sf[:, :M].view(np.uint32), sf_ref[:, :M].view(np.uint32))
    assert np.all(sf[:, M:] == SF_CANARY)


def test_float_quant_zero_tiny_and_boundary_groups():
    M, K = 4, 512
    x = W.normal_bf16((M, K), seed=4)
    x[0, :128] = 0
    x[0, 128:256] = 0x8000                                   # -0 everywhere
    x[1, :128] = W.f32_to_bf16_bits(np.full(128, 1e-30, np.float32))
    x[2, :128] = W.f32_to_bf16_bits(np.linspace(-448, 448, 128).astype(np.float32))
    x[3, 256:384] = W.f32_to_bf16_bits(np.full(128, 3.0e38, np.float32))
    q, sf = _quant(x)
    q_ref, sf_ref = O.quant_group_float(x, ld_sf=sf.shape[1])
    assert np.array_equal(q, q_ref)
    assert np.array_equal(sf[:, :M].view(np.uint32), sf_ref[:, :M].view(np.uint32))


@pytest.mark.parametrize("N,K", [(200, 256), (1000, 1024)])
def test_float_block_quant_bit_exact(N, K):
    w = W.normal_bf16((N, K), std=0.02, seed=N, tensor_id=W.T_B)
    q, sfb = F.fp8_block_quant_128x128_float(to_dev(w))
    sync()
    q_ref, sfb_ref = O.block_quant_128x128_float(w)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sfb.cpu().numpy().view(np.uint32), sfb_ref.view(np.uint32))


def _float_operands(M, N, K, seed):
    qa, sfa = O.quant_group_float(W.normal_bf16_outliers((M, K), seed=seed))
    qb, sfb = O.block_quant_128x128_float(W.normal_bf16((N, K), std=1.0, seed=seed, tensor_id=W.T_B))
    return qa, sfa, qb, sfb


def _gemm(qa, sfa, qb, sfb, kernel=None, splits=None):
    M, N = qa.shape[0], qb.shape[0]
    c = F.fp8_block_gemm_nt_float_scales(to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb), c=poisoned_bf16(M, N),
                                         kernel=kernel, splits=splits)
    sync()
    return to_host(c)


SMALL = [(1, 64, 128), (17, 192, 384), (64, 512, 1024), (130, 256, 512), (257, 384, 1152)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_float_gemm_every_float_kernel(M, N, K):
    qa, sfa, qb, sfb = _float_operands(M, N, K, seed=M + N + K)
    ref = O.gemm_nt_float_scales(qa, sfa, qb, sfb)
    ran = 0
    for kernel in range(F.gemm_config_count()):
        if F.gemm_config_of(kernel, FLOAT, M, N, K) is None:
            continue
        for splits in (1, 3):
            gemm_tolerance_check(_gemm(qa, sfa, qb, sfb, kernel=kernel, splits=splits), ref,
                                 "float kernel %d splits %d %dx%dx%d" % (kernel, splits, M, N, K))
        ran += 1
    assert ran >= 4
    gemm_tolerance_check(_gemm(qa, sfa, qb, sfb), ref, "float auto")


@pytest.mark.parametrize("M,N,K", [(64, 7168, 18432), (4096, 4096, 7168)])
def test_float_chain_on_gpu_sampled_rows(M, N, K):
    """bf16 A and B -> float-scale quant of both on the GPU -> float-scale GEMM; sampled
    rows against the oracle's chain (bit-exact quant checked on the way)."""
    a = W.normal_bf16_outliers((M, K), seed=7)
    b = W.normal_bf16((N, K), std=0.02, seed=7, tensor_id=W.T_B)
    qa, sfa = F.fp8_quant_group_float(to_dev(a))
    qb, sfb = F.fp8_block_quant_128x128_float(to_dev(b))
    print("float chain %dx%dx%d config %s" % (M, N, K, F.gemm_config(FLOAT, M, N, K)), flush=True)
    c = F.fp8_block_gemm_nt_float_scales(qa, sfa, qb, sfb, c=poisoned_bf16(M, N))
    sync()
    c = to_host(c)
    rows = np.unique(np.linspace(0, M - 1, 8).astype(np.int64))
    qa_ref, sfa_ref = O.quant_group_float(a[rows])
    assert np.array_equal(qa.cpu().numpy()[rows], qa_ref)
    qb_ref, sfb_ref = O.block_quant_128x128_float(b)
    assert np.array_equal(sfb.cpu().numpy().view(np.uint32), sfb_ref.view(np.uint32))
    ref = O.gemm_nt_float_scales(qa_ref, sfa_ref, qb_ref, sfb_ref)
    gemm_tolerance_check(c[rows], ref, "float chain %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [(1, 64, 128), (17, 192, 384), (64, 512, 1024), (64, 128, 2560)])
def test_float_gemm_preshuffled_every_entry(M, N, K):
    """Float scales on pre-shuffled weights: every entry reading that combination, several
    splits, within the tolerance of the oracle on the unshuffled weights, and bit-equal to
    the float-scale decode kernel on the plain layout with the same tile and split."""
    qa, sfa, qb, sfb = _float_operands(M, N, K, seed=M + N + K + 1)
    ref = O.gemm_nt_float_scales(qa, sfa, qb, sfb)
    da, dsa, db, dsb = to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb)
    dbs = F.fp8_weight_preshuffle(db)
    entries = [k for k in range(F.gemm_config_count())
               if F.gemm_config_of(k, F.LAYOUT_DENSE_FLOAT_PRESHUFFLED, M, N, K) is not None]
    assert entries
    for kernel in entries:
        for splits in (1, 2, 3):
            cfg = F.gemm_config_of(kernel, F.LAYOUT_DENSE_FLOAT_PRESHUFFLED, M, N, K, splits)
            c = to_host(F.fp8_block_gemm_nt_float_scales(da, dsa, dbs, dsb, c=poisoned_bf16(M, N), kernel=kernel,
                                                         splits=splits, preshuffled=True))
            sync()
            gemm_tolerance_check(c, ref, "float preshuffled kernel %d splits %d %dx%dx%d" % (kernel, splits, M, N, K))
            plain = [k for k in range(F.gemm_config_count())
                     if F.gemm_config_of(k, FLOAT, M, N, K, splits) == {**cfg, "kernel": k}]
            outs = [to_host(F.fp8_block_gemm_nt_float_scales(da, dsa, db, dsb, c=poisoned_bf16(M, N), kernel=k,
                                                             splits=splits)) for k in plain]
            sync()
            assert any(np.array_equal(c, x) for x in outs), "kernel %d splits %d" % (kernel, splits)
    c = to_host(F.fp8_block_gemm_nt_float_scales(da, dsa, dbs, dsb, c=poisoned_bf16(M, N), preshuffled=True))
    sync()
    gemm_tolerance_check(c, ref, "float preshuffled auto")
