"""GPU parity of the contiguous grouped GEMM (rows grouped by expert in 128-row runs,
a per-row group index, -1 for padding) against the CPU oracle.  Valid rows meet the
GEMM tolerance; blocks that start with padding, or whose first row names no group,
must keep the canary the test wrote there."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_token_amd as F
import oracle as O
import workloads as W
from gpu_helpers import DEV, gemm_tolerance_check, sync, to_dev, to_host

pytestmark = pytest.mark.gpu

CANARY = 0x7E7E  # a bf16 pattern the GEMM never produces here (a huge finite value)
CONTIGUOUS = 2   # layout code of the configuration queries


def _operands(m_indices, E, N, K, seed=0):
    """A quantized from N(0,1) rows (padding rows poisoned with e4m3 NaN codes and
    NaN-coded scale words), weights quantized per group from N(0, 0.02)."""
    M = len(m_indices)
    x = W.normal_bf16((M, K), seed=seed)
    ld = max(4, -(-M // 4) * 4)
    qa, sfa = O.quant_group_pack(x, ld_sf=ld)
    pad = ~((m_indices >= 0) & (m_indices < E))
    qa[pad] = 0x7F
    sfa[:, :M][:, pad] = 0xFFFFFFFF
    w = W.normal_bf16((E * N, K), std=0.02, seed=seed, tensor_id=W.T_B)
    qb = np.empty((E, N, K), np.uint8)
    sfb = np.empty((E, (N + 127) // 128, K // 128), np.float32)
    for g in range(E):
        qb[g], sfb[g] = O.block_quant_128x128(np.ascontiguousarray(w[g * N:(g + 1) * N]))
    return qa, sfa, qb, sfb


def _run(qa, sfa, qb, sfb, m_indices, kernel=None):
    M, N = qa.shape[0], qb.shape[1]
    c = torch.empty((M, N), dtype=torch.int16, device=DEV).fill_(CANARY).view(torch.bfloat16)
    F.fp8_block_gemm_grouped_contiguous(to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb), to_dev(m_indices), c=c,
                                        kernel=kernel)
    sync()
    return to_host(c)


def _check(c, qa, sfa, qb, sfb, m_indices, rows=None, what=""):
    E = qb.shape[0]
    ref = O.gemm_grouped_contiguous(qa, sfa, qb, sfb, m_indices, rows=rows)
    valid = (m_indices >= 0) & (m_indices < E)
    sel = np.nonzero(valid)[0] if rows is None else np.array([r for r in rows if valid[r]], np.int64)
    gemm_tolerance_check(c[sel], ref[sel], what)
    # blocks whose first row is padding are skipped whole
    for b0 in range(0, len(m_indices), 128):
        if not valid[b0]:
            assert np.all(c[b0:b0 + 128] == CANARY), "%s: skipped block at row %d written" % (what, b0)


def test_contiguous_small_all_kernels_edge_runs():
    """Runs of 130 (two blocks, the second almost all padding), 0, 1 and 128 rows, a
    block whose rows name a group past E, a trailing padding block; N = 192 (a partial
    128-column block), K = 384 (a partial scale word)."""
    E, N, K = 4, 192, 384
    mi = W.contiguous_layout([130, 0, 1, 128], tail_blocks=1)
    mi = np.concatenate([mi, np.full(128, E + 5, np.int32), np.full(128, -1, np.int32)])
    qa, sfa, qb, sfb = _operands(mi, E, N, K, seed=3)
    ran = 0
    for kernel in range(F.gemm_config_count()):
        if F.gemm_config_of(kernel, CONTIGUOUS, len(mi), N, K) is None:
            continue
        print("contiguous kernel %d" % kernel, flush=True)
        c = _run(qa, sfa, qb, sfb, mi, kernel=kernel)
        _check(c, qa, sfa, qb, sfb, mi, what="kernel %d" % kernel)
        ran += 1
    assert ran >= 3


def test_contiguous_rejects_tiles_taller_than_a_run():
    cfgs = [F.gemm_config_of(k, CONTIGUOUS, 1024, 256, 1024) for k in range(F.gemm_config_count())]
    assert all(c is None or c["bm"] <= 128 for c in cfgs)
    assert F.gemm_config(CONTIGUOUS, 8192, 4096, 7168)["bm"] <= 128


def test_contiguous_gate_up_full_shape_every_valid_row():
    """The masked gate_up workload in the contiguous layout: 32 experts, Zipf(1.1)
    counts (2780 valid rows) in 128-row runs, N = 4096, K = 7168, plus a padding block;
    every element of every valid row against the oracle."""
    E, N, K = W.MOE_E, W.MOE_GATE_UP["N"], W.MOE_GATE_UP["K"]
    counts = W.zipf_counts()
    mi = W.contiguous_layout(counts, tail_blocks=1)
    qa, sfa, qb, sfb = _operands(mi, E, N, K, seed=0)
    print("contiguous gate_up M=%d auto config %s" % (len(mi), F.gemm_config(CONTIGUOUS, len(mi), N, K)), flush=True)
    c = _run(qa, sfa, qb, sfb, mi)
    starts = np.concatenate([[0], np.cumsum(-(-counts // 128) * 128)])
    rows = np.concatenate([np.arange(starts[g], starts[g] + counts[g]) for g in range(E) if counts[g] > 0])
    _check(c, qa, sfa, qb, sfb, mi, rows=rows.astype(np.int64), what="gate_up contiguous")
