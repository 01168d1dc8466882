"""GPU parity of the masked grouped GEMM (and the SiLU-quant -> down GEMM chain)
against the CPU oracle.  Valid rows must meet the GEMM tolerance; rows at or past
an expert's count must keep the canary the test wrote there."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_token_amd as F
import oracle as O
import workloads as W
from gpu_helpers import DEV, bf16_to_f64, gemm_tolerance_check, poisoned_bf16, sync, to_dev, to_host

pytestmark = pytest.mark.gpu

CANARY = 0x7E7E  # a bf16 pattern the GEMM never produces here (a huge finite value)


def _moe_operands(E, M_max, N, K, seed=0):
    x = W.normal_bf16((E * M_max, K), seed=seed)
    qa, sfa_flat = O.quant_group_pack(x, ld_sf=E * M_max)
    Wd = (K // 128 + 3) // 4
    a = qa.reshape(E, M_max, K)
    sfa = np.ascontiguousarray(sfa_flat.reshape(Wd, E, M_max).transpose(1, 0, 2))
    w = W.normal_bf16((E * N, K), std=0.02, seed=seed, tensor_id=W.T_B)
    qb = np.empty((E, N, K), np.uint8)
    sfb = np.empty((E, (N + 127) // 128, K // 128), np.float32)
    for e in range(E):
        qb[e], sfb[e] = O.block_quant_128x128(np.ascontiguousarray(w[e * N:(e + 1) * N]))
    return a, sfa, qb, sfb


def _run_masked(a, sfa, b, sfb, counts, kernel=None):
    E, M_max, K = a.shape
    N = b.shape[1]
    c = torch.full((E, M_max, N), 0, dtype=torch.int16, device=DEV)
    c.fill_(CANARY)
    c = c.view(torch.bfloat16)
    F.fp8_block_gemm_grouped_masked(to_dev(a), to_dev(sfa), to_dev(b), to_dev(sfb), to_dev(counts), c=c,
                                    kernel=kernel)
    sync()
    return to_host(c)


def _check(c, a, sfa, b, sfb, counts, rows=None, what=""):
    E, M_max, _ = a.shape
    ref = O.gemm_grouped_masked(a, sfa, b, sfb, counts, rows=rows)
    for e in range(E):
        ce = int(min(max(counts[e], 0), M_max))
        sel = np.arange(ce) if rows is None else np.array([r for r in rows if r < ce], np.int64)
        if sel.size:
            gemm_tolerance_check(c[e, sel], ref[e, sel], "%s expert %d" % (what, e))
        assert np.all(c[e, ce:] == CANARY), "%s expert %d: padded rows written" % (what, e)


def test_masked_small_all_kernels_edge_counts():
    E, M_max, N, K = 6, 72, 192, 384
    a, sfa, b, sfb = _moe_operands(E, M_max, N, K, seed=1)
    counts = np.array([0, 1, 72, 100, -2, 33], np.int32)
    for kernel in range(F.gemm_config_count()):
        if F.gemm_config_of(kernel, F.LAYOUT_DENSE_FLOAT, M_max, N, K) is not None:
            continue  # float-scale entry: another scale format
        if (F.gemm_config_of(kernel, F.LAYOUT_DENSE_PRESHUFFLED, M_max, N, K) is not None
                or F.gemm_config_of(kernel, F.LAYOUT_DENSE_PRESHUFFLED, 64, N, K) is not None):
            continue  # dense entry on pre-shuffled weights (the weight-streaming ones take M <= 64 only)
        if F.gemm_config_of(kernel, F.LAYOUT_DENSE_FLOAT_PRESHUFFLED, M_max, N, K) is not None:
            continue  # float scales on pre-shuffled weights
        if (F.gemm_config_of(kernel, F.LAYOUT_MASKED_PRESHUFFLED, M_max, N, K) is not None
                and F.gemm_config_of(kernel, F.LAYOUT_MASKED, M_max, N, K) is None):
            continue  # masked entry on pre-shuffled weights only (test_gpu_preshuffled.py)
        assert F.gemm_config_of(kernel, True, M_max, N, K) is not None, kernel
        c = _run_masked(a, sfa, b, sfb, counts, kernel=kernel)
        _check(c, a, sfa, b, sfb, counts, what="kernel %d" % kernel)


def test_masked_full_counts_equal_dense():
    E, M_max, N, K = 3, 64, 256, 512
    a, sfa, b, sfb = _moe_operands(E, M_max, N, K, seed=2)
    counts = np.full(E, M_max, np.int32)
    c = _run_masked(a, sfa, b, sfb, counts)
    for e in range(E):
        d = F.fp8_block_gemm_nt(to_dev(a[e]), to_dev(sfa[e]), to_dev(b[e]), to_dev(sfb[e]), c=poisoned_bf16(M_max, N))
        sync()
        ref = O.gemm_nt(a[e], sfa[e], b[e], sfb[e])
        gemm_tolerance_check(c[e], ref, "masked e%d" % e)
        gemm_tolerance_check(to_host(d), ref, "dense e%d" % e)


def test_masked_padded_rows_poisoned_do_not_leak():
    E, M_max, N, K = 4, 128, 128, 256
    a, sfa, b, sfb = _moe_operands(E, M_max, N, K, seed=4)
    counts = np.array([5, 70, 128, 0], np.int32)
    clean = _run_masked(a, sfa, b, sfb, counts)
    a2, sfa2 = a.copy(), sfa.copy()
    for e in range(E):
        a2[e, counts[e]:] = 0x7F                 # e4m3 NaN in every padded row
        sfa2[e, :, counts[e]:] = 0xFFFFFFFF      # and NaN-coded scales
    poisoned = _run_masked(a2, sfa2, b, sfb, counts)
    assert np.array_equal(clean, poisoned)
    _check(clean, a, sfa, b, sfb, counts, what="poison")


def test_masked_gate_up_full_shape_every_valid_row():
    """32 experts x 256 padded rows, Zipf(1.1) counts (2780 valid rows), N=4096, K=7168:
    every element of every valid row against the oracle; padded rows keep the canary."""
    E, M_max = W.MOE_E, W.MOE_M_MAX
    N, K = W.MOE_GATE_UP["N"], W.MOE_GATE_UP["K"]
    a, sfa, b, sfb = _moe_operands(E, M_max, N, K, seed=0)
    counts = W.zipf_counts()
    c = _run_masked(a, sfa, b, sfb, counts)
    _check(c, a, sfa, b, sfb, counts, what="gate_up")


def test_silu_quant_then_masked_down_chain():
    """[32, 256, 4096] bf16 -> fused SiLU-mul-quant -> masked down GEMM (N=7168, K=2048),
    all on the GPU with the counts on the device; every element of every valid row
    compared with the oracle's chain."""
    E, M_max, H = W.MOE_E, W.MOE_M_MAX, W.MOE_DOWN["H"]
    N = W.MOE_DOWN["N"]
    x = W.normal_bf16((E, M_max, 2 * H), seed=0, tensor_id=W.T_X)
    counts = W.zipf_counts()
    w = W.normal_bf16((E * N, H), std=0.02, seed=0, tensor_id=W.T_B)
    qb = np.empty((E, N, H), np.uint8)
    sfb = np.empty((E, N // 128, H // 128), np.float32)
    for e in range(E):
        qb[e], sfb[e] = O.block_quant_128x128(np.ascontiguousarray(w[e * N:(e + 1) * N]))
    dcounts = to_dev(counts)
    q, sf = F.silu_mul_quant_group_pack(to_dev(x), dcounts)
    c = torch.empty((E, M_max, N), dtype=torch.int16, device=DEV).fill_(CANARY).view(torch.bfloat16)
    F.fp8_block_gemm_grouped_masked(q, sf, to_dev(qb), to_dev(sfb), dcounts, c=c)
    sync()
    c = to_host(c)
    q_ref, sf_ref = O.silu_mul_quant_group_pack(x, counts)
    ref = O.gemm_grouped_masked(q_ref, sf_ref, qb, sfb, counts)
    for e in range(E):
        ce = int(min(max(counts[e], 0), M_max))
        if ce:  # every element of every valid row
            gemm_tolerance_check(c[e, :ce], ref[e, :ce], "chain expert %d" % e)
        assert np.all(c[e, ce:] == CANARY)
    assert np.isfinite(bf16_to_f64(c[0, :counts[0]])).all()


def test_masked_ragged_round_both_layouts():
    """16 experts x 256 rows x N = 4608: 288 tiles of 256 x 256 (a last round of 32),
    counts from empty through partial 32-row groups to clamped.  Valid rows meet the
    oracle's tolerance, rows past each count keep the canary, and pre-shuffled weights
    give the same bits."""
    print("masked E=16 M_max=256 N=4608 K=256", flush=True)
    E, M_max, N, K = 16, 256, 4608, 256
    a, sfa, b, sfb = _moe_operands(E, M_max, N, K, seed=6)
    counts = np.array([256, 0, 129, 128, 1, 255, 300, -1, 64, 200, 256, 17, 130, 2, 256, 90], np.int32)
    c = _run_masked(a, sfa, b, sfb, counts)
    _check(c, a, sfa, b, sfb, counts, what="ragged round")
    cs = torch.empty((E, M_max, N), dtype=torch.int16, device=DEV).fill_(CANARY).view(torch.bfloat16)
    F.fp8_block_gemm_grouped_masked(to_dev(a), to_dev(sfa), F.fp8_weight_preshuffle(to_dev(b)), to_dev(sfb),
                                    to_dev(counts), c=cs, preshuffled=True)
    sync()
    assert np.array_equal(to_host(cs), c)
