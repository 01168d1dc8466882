"""GPU parity of the per-token quant into the masked expert layout of routed tokens
(slot assignment, counts, e4m3 rows and packed scale words) against the CPU oracle:
bit-exact on every written row, rows at or past an expert's count untouched."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_token_amd as F
import oracle as O
import workloads as W
from gpu_helpers import DEV, gemm_tolerance_check, sync, to_dev, to_host

pytestmark = pytest.mark.gpu

QCANARY = 0x5A          # e4m3 byte the test writes before the call
SCANARY = 0x13579BDF    # scale word likewise


def _run(x, ids, E, M_max):
    T, K = x.shape
    Wd = (K // 128 + 3) // 4
    q = torch.full((E, M_max, K), QCANARY, dtype=torch.uint8, device=DEV)
    sf = torch.full((E, Wd, M_max), SCANARY, dtype=torch.int32, device=DEV)
    mm = torch.full((E,), -7, dtype=torch.int32, device=DEV)
    slot = torch.full((T, ids.shape[1]), -9, dtype=torch.int32, device=DEV)
    F.fp8_quant_group_pack_to_experts(to_dev(x), to_dev(ids), E, M_max, q=q, sf=sf, masked_m=mm, slot_of=slot)
    sync()
    return q.cpu().numpy(), sf.cpu().numpy().view(np.uint32), mm.cpu().numpy(), slot.cpu().numpy()


def _check(x, ids, E, M_max, what):
    q, sf, mm, slot = _run(x, ids, E, M_max)
    q_ref, sf_ref, mm_ref, slot_ref = O.quant_group_pack_to_experts(x, ids, E, M_max)
    assert np.array_equal(slot, slot_ref), what
    assert np.array_equal(mm, mm_ref), what
    for e in range(E):
        c = int(mm_ref[e])
        assert np.array_equal(q[e, :c], q_ref[e, :c]), "%s expert %d rows" % (what, e)
        assert np.array_equal(sf[e, :, :c], sf_ref[e, :, :c]), "%s expert %d scales" % (what, e)
        assert np.all(q[e, c:] == QCANARY) and np.all(sf[e, :, c:] == SCANARY), "%s expert %d padding" % (what, e)
    return q, sf, mm, slot


def test_dispatch_small_edge_cases():
    """41 tokens x 3 choices, ids -1 and past E, one token routed thrice to one expert,
    capacity 9 (overflow dropped), K = 640 (a partial scale word)."""
    rng = np.random.default_rng(1)
    T, topk, E, M_max, K = 41, 3, 5, 9, 640
    ids = rng.integers(-1, E + 2, (T, topk)).astype(np.int32)
    ids[0] = [2, 2, 2]
    x = W.normal_bf16((T, K), seed=1, tensor_id=W.T_X)
    _check(x, ids, E, M_max, "small")


def test_dispatch_many_experts_and_chunks():
    """1000 experts, 300 tokens x 8 choices (2400 pairs: three 1024-pair chunks), capacity 2."""
    rng = np.random.default_rng(2)
    T, topk, E, M_max, K = 300, 8, 1000, 2, 256
    ids = rng.integers(0, 40, (T, topk)).astype(np.int32) * 25  # 40 distinct experts, heavy repeats
    x = W.normal_bf16((T, K), seed=2, tensor_id=W.T_X)
    _check(x, ids, E, M_max, "many experts")


def test_dispatch_wide_rows():
    """K = 9216: 18 packed words per row (the grid strides over more units than it has
    wavefronts' worth of one word each)."""
    rng = np.random.default_rng(3)
    T, topk, E, M_max, K = 20, 4, 6, 15, 9216
    ids = rng.integers(0, E, (T, topk)).astype(np.int32)
    x = W.normal_bf16((T, K), seed=3, tensor_id=W.T_X)
    _check(x, ids, E, M_max, "wide rows")


def test_dispatch_nine_chunks_with_overflow():
    """1100 tokens x 8 choices (8800 pairs: nine 1024-pair rank chunks, the last partial),
    Zipf-skewed ids, capacity overflow on the hot experts."""
    rng = np.random.default_rng(4)
    T, topk, E, M_max, K = 1100, 8, 64, 200, 256
    ids = (rng.zipf(1.3, (T, topk)) % E).astype(np.int32)
    x = W.normal_bf16((T, K), seed=4, tensor_id=W.T_X)
    _check(x, ids, E, M_max, "two-pass")


def test_dispatch_workload_bit_exact_and_deterministic():
    """512 tokens x top-8 of 32 experts with Zipf(1.1) weights, capacity 256, K = 7168."""
    E, M_max, K = W.MOE_E, W.MOE_M_MAX, W.MOE_GATE_UP["K"]
    ids = W.topk_routing()
    x = W.normal_bf16((ids.shape[0], K), seed=0, tensor_id=W.T_X)
    q1, sf1, mm1, slot1 = _check(x, ids, E, M_max, "workload")
    q2, sf2, mm2, slot2 = _run(x, ids, E, M_max)
    assert np.array_equal(slot1, slot2) and np.array_equal(mm1, mm2)
    assert np.array_equal(q1, q2) and np.array_equal(sf1, sf2)


def test_dispatch_empty_and_limits():
    E, M_max, K = 3, 4, 128
    x = torch.zeros((0, K), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((0, 2), dtype=torch.int32, device=DEV)
    q, sf, mm, slot = F.fp8_quant_group_pack_to_experts(x, ids, E, M_max)
    sync()
    assert mm.cpu().tolist() == [0, 0, 0]
    with pytest.raises(F.Fp8bsError):
        F.fp8_quant_group_pack_to_experts(torch.zeros((2, K), dtype=torch.bfloat16, device=DEV),
                                          torch.zeros((2, 1), dtype=torch.int32, device=DEV), 1025, 4)


def test_dispatch_then_masked_gate_up_chain():
    """Routed tokens -> quant into the expert layout -> masked gate_up GEMM with the
    counts the dispatch produced on the device; every valid row against the oracle chain."""
    E, M_max, N, K = W.MOE_E, W.MOE_M_MAX, W.MOE_GATE_UP["N"], W.MOE_GATE_UP["K"]
    ids = W.topk_routing(T=256)
    x = W.normal_bf16((ids.shape[0], K), seed=3, tensor_id=W.T_X)
    w = W.normal_bf16((E * N, K), std=0.02, seed=3, tensor_id=W.T_B)
    qb = np.empty((E, N, K), np.uint8)
    sfb = np.empty((E, N // 128, K // 128), np.float32)
    for e in range(E):
        qb[e], sfb[e] = O.block_quant_128x128(np.ascontiguousarray(w[e * N:(e + 1) * N]))
    q, sf, mm, _ = F.fp8_quant_group_pack_to_experts(to_dev(x), to_dev(ids), E, M_max)
    c = F.fp8_block_gemm_grouped_masked(q, sf, to_dev(qb), to_dev(sfb), mm)
    sync()
    c = to_host(c)
    q_ref, sf_ref, mm_ref, _ = O.quant_group_pack_to_experts(x, ids, E, M_max)
    assert np.array_equal(mm.cpu().numpy(), mm_ref)
    ref = O.gemm_grouped_masked(q_ref, sf_ref, qb, sfb, mm_ref)
    for e in range(E):
        ce = int(min(mm_ref[e], M_max))
        if ce:
            gemm_tolerance_check(c[e, :ce], ref[e, :ce], "chain expert %d (every valid row)" % e)
