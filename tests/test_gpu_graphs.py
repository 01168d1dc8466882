"""HIP graph capture of the hot path: steps captured once and replayed several times,
with eager calls of other shapes (sharing the stream's workspace and split-K arrival
counters) between the replays; every replay must reproduce the eager result bit for
bit (all kernels here are deterministic)."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_token_amd as F
import workloads as W
from gpu_helpers import DEV, sync, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


@pytest.mark.parametrize("preshuffled", [False, True], ids=["plain", "preshuffled"])
def test_graph_replays_of_the_decode_step_match_eager(preshuffled):
    M, N, K = 64, 7168, 18432
    s = torch.cuda.Stream()
    gemm = F.fp8_block_gemm_nt_preshuffled if preshuffled else F.fp8_block_gemm_nt
    x = to_dev(W.normal_bf16_outliers((M, K), seed=3))
    with torch.cuda.stream(s):
        qb, sfb = F.fp8_block_quant_128x128(to_dev(W.normal_bf16((N, K), std=0.02, seed=3, tensor_id=W.T_B)))
        if preshuffled:
            qb = F.fp8_weight_preshuffle(qb)
        q = torch.empty((M, K), dtype=torch.uint8, device=DEV)
        sf = torch.empty(((K // 128 + 3) // 4, M), dtype=torch.int32, device=DEV)
        c = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        # other shapes on the same stream: they share its workspace and counters
        oa, osa = F.fp8_quant_group_pack(to_dev(W.normal_bf16((16, 4096), seed=4)))
        ob, osb = F.fp8_block_quant_128x128(to_dev(W.normal_bf16((1024, 4096), std=0.02, seed=4, tensor_id=W.T_B)))

        def step():
            F.fp8_quant_group_pack(x, q=q, sf=sf)
            gemm(q, sf, qb, sfb, c=c)

        step()  # eager, also creates the stream's workspace before capture
    s.synchronize()
    assert F.gemm_config(F.LAYOUT_DENSE_PRESHUFFLED if preshuffled else F.LAYOUT_DENSE, M, N, K)["splits"] > 1
    eager = _bits(c).copy()
    other_eager = _bits(F.fp8_block_gemm_nt(oa, osa, ob, osb))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(5):
        with torch.cuda.stream(s):
            c.zero_()
            g.replay()
        s.synchronize()
        assert np.array_equal(_bits(c), eager), "replay %d" % rep
        with torch.cuda.stream(s):
            o = F.fp8_block_gemm_nt(oa, osa, ob, osb)
        s.synchronize()
        assert np.array_equal(_bits(o), other_eager), "eager call after replay %d" % rep


def test_graph_replays_of_dispatch_and_masked_moe_match_eager():
    E, M_max, N, K = W.MOE_E, W.MOE_M_MAX, 1024, 2048
    H = 1024
    s = torch.cuda.Stream()
    ids = to_dev(W.topk_routing(T=128))
    x = to_dev(W.normal_bf16((128, K), seed=5, tensor_id=W.T_X))
    y = to_dev(W.normal_bf16((E, M_max, 2 * H), seed=6, tensor_id=W.T_X))
    with torch.cuda.stream(s):
        wq, wsf = [], []
        for e in range(E):
            a, b = F.fp8_block_quant_128x128(to_dev(W.normal_bf16((N, K), std=0.02, seed=100 + e, tensor_id=W.T_B)))
            wq.append(a)
            wsf.append(b)
        qb, sfb = torch.stack(wq), torch.stack(wsf)
        d1, d2 = [], []
        for e in range(E):
            a, b = F.fp8_block_quant_128x128(to_dev(W.normal_bf16((N, H), std=0.02, seed=200 + e, tensor_id=W.T_B)))
            d1.append(a)
            d2.append(b)
        qd, sfd = torch.stack(d1), torch.stack(d2)
        q, sf, mm, slot = F.fp8_quant_group_pack_to_experts(x, ids, E, M_max)
        c = torch.empty((E, M_max, N), dtype=torch.bfloat16, device=DEV)
        qy = torch.empty((E, M_max, H), dtype=torch.uint8, device=DEV)
        sfy = torch.empty((E, (H // 128 + 3) // 4, M_max), dtype=torch.int32, device=DEV)
        cd = torch.empty((E, M_max, N), dtype=torch.bfloat16, device=DEV)

        def step():
            F.fp8_quant_group_pack_to_experts(x, ids, E, M_max, q=q, sf=sf, masked_m=mm, slot_of=slot)
            F.fp8_block_gemm_grouped_masked(q, sf, qb, sfb, mm, c=c)
            F.silu_mul_quant_group_pack(y, mm, q=qy, sf=sfy)
            F.fp8_block_gemm_grouped_masked(qy, sfy, qd, sfd, mm, c=cd)

        step()
    s.synchronize()
    counts = mm.cpu().numpy()
    ref = [_bits(t).copy() for t in (c, cd, slot, mm)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for rep in range(4):
        with torch.cuda.stream(s):
            for t in (c, cd, slot, mm):
                t.zero_()
            g.replay()
        s.synchronize()
        got = [_bits(t) for t in (c, cd, slot, mm)]
        assert np.array_equal(got[2], ref[2]) and np.array_equal(got[3], ref[3]), "replay %d slots/counts" % rep
        for e in range(E):
            r = int(counts[e])
            assert np.array_equal(got[0][e, :r], ref[0][e, :r]), "replay %d gate_up expert %d" % (rep, e)
            assert np.array_equal(got[1][e, :r], ref[1][e, :r]), "replay %d down expert %d" % (rep, e)
        with torch.cuda.stream(s):  # eager work between replays
            F.fp8_quant_group_pack_to_experts(x[:64], ids[:64], E, M_max)
        s.synchronize()


def test_graph_survives_workspace_growth():
    """A graph captured while the stream's workspace is small keeps working after a
    larger call on the same stream has replaced the workspace (the old one is kept)."""
    s = torch.cuda.Stream()
    small = (64, 1024, 4096)
    large = (64, 7168, 18432)
    ops = {}
    for (M, N, K) in (small, large):
        a, sa = F.fp8_quant_group_pack(to_dev(W.normal_bf16((M, K), seed=M + N)))
        b, sb = F.fp8_block_quant_128x128(to_dev(W.normal_bf16((N, K), std=0.02, seed=N, tensor_id=W.T_B)))
        ops[(M, N, K)] = (a, sa, b, sb, torch.empty((M, N), dtype=torch.bfloat16, device=DEV))
    sync()
    a, sa, b, sb, c = ops[small]
    with torch.cuda.stream(s):
        F.fp8_block_gemm_nt(a, sa, b, sb, c=c)  # creates the stream's (small) workspace
    s.synchronize()
    want = _bits(c).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        F.fp8_block_gemm_nt(a, sa, b, sb, c=c)
    la, lsa, lb, lsb, lc = ops[large]
    with torch.cuda.stream(s):
        F.fp8_block_gemm_nt(la, lsa, lb, lsb, c=lc)  # needs a larger workspace: replaced
    s.synchronize()
    large_want = _bits(lc).copy()
    for rep in range(3):
        with torch.cuda.stream(s):
            c.zero_()
            g.replay()  # in stream order with the large calls on the same stream
            F.fp8_block_gemm_nt(la, lsa, lb, lsb, c=lc)
        s.synchronize()
        assert np.array_equal(_bits(c), want), "replay %d" % rep
        assert np.array_equal(_bits(lc), large_want), "large call after replay %d" % rep
