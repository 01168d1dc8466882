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


# K from one K-block up; the three-stage ring turns in trips of twelve K-blocks, so K = 2048
# is a trip and a four-block tail, 2560 a trip and an eight-block tail
SMALL = [(1, 64, 128), (17, 192, 384), (64, 512, 1024), (100, 640, 640), (130, 256, 512), (64, 128, 2560),
         (130, 256, 2048)]


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
    deterministic, and agrees with the oracle on every output element."""
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
    ref = O.gemm_nt(qa, sfa, qb, sfb)
    st = gemm_tolerance_check(c1, ref, s.name)
    print("%s: max |err|/bound %.3f" % (s.name, st["max_err_over_bound"]), flush=True)


CANARY = 0x7E7E


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


def _masked(a, sfa, b_dev, sfb, counts, kernel=None, preshuffled=False):
    E, M_max, K = a.shape
    N = b_dev.shape[1]
    c = torch.full((E, M_max, N), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    F.fp8_block_gemm_grouped_masked(to_dev(a), to_dev(sfa), b_dev, to_dev(sfb), to_dev(counts), c=c, kernel=kernel,
                                    preshuffled=preshuffled)
    sync()
    return to_host(c)


def test_preshuffled_masked_every_entry_edge_counts():
    """Every entry reading pre-shuffled weights in the masked form: valid rows within the
    GEMM tolerance of the oracle, rows past the count untouched (canary), and bit-equal to
    the plain-layout entry of the same tile where there is one."""
    E, M_max, N, K = 4, 96, 256, 640
    a, sfa, qb, sfb = _moe_operands(E, M_max, N, K, seed=4)
    counts = np.array([0, 17, 96, 200], np.int32)  # empty, partial, full, clamped
    ref = O.gemm_grouped_masked(a, sfa, qb, sfb, counts)
    db, dbs = to_dev(qb), F.fp8_weight_preshuffle(to_dev(qb))
    entries = [k for k in range(F.gemm_config_count())
               if F.gemm_config_of(k, F.LAYOUT_MASKED_PRESHUFFLED, M_max, N, K) is not None]
    assert entries
    plain_by_tile = {}
    for k in range(F.gemm_config_count()):
        cfg = F.gemm_config_of(k, True, M_max, N, K)
        if cfg is not None:
            plain_by_tile.setdefault((cfg["bm"], cfg["bn"]), []).append(k)
    for kernel in entries:
        print("masked preshuffled kernel %d" % kernel, flush=True)
        c = _masked(a, sfa, dbs, sfb, counts, kernel=kernel, preshuffled=True)
        for e in range(E):
            ce = int(min(max(counts[e], 0), M_max))
            if ce:
                gemm_tolerance_check(c[e, :ce], ref[e, :ce], "kernel %d expert %d" % (kernel, e))
            assert np.all(c[e, ce:] == CANARY), "kernel %d expert %d: padded rows written" % (kernel, e)
        cfg = F.gemm_config_of(kernel, F.LAYOUT_MASKED_PRESHUFFLED, M_max, N, K)
        same = [_masked(a, sfa, db, sfb, counts, kernel=k) for k in plain_by_tile.get((cfg["bm"], cfg["bn"]), [])]
        assert not same or any(np.array_equal(c, x) for x in same), "kernel %d differs from its plain tile" % kernel
    c = _masked(a, sfa, dbs, sfb, counts, preshuffled=True)
    for e in range(1, E):
        ce = int(min(counts[e], M_max))
        gemm_tolerance_check(c[e, :ce], ref[e, :ce], "auto expert %d" % e)


def test_preshuffled_dense_ring_entries_match_plain():
    """Prefill-sized dense calls on pre-shuffled weights (ring tiles) equal the plain-layout
    ring tiles of the same shape bit for bit and meet the oracle's tolerance."""
    M, N, K = 512, 512, 1152
    a = W.normal_bf16((M, K), seed=21)
    b = W.normal_bf16((N, K), std=1.0, seed=21, tensor_id=W.T_B)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    rows = np.arange(0, M, 7)
    ref = O.gemm_nt(qa, sfa, qb, sfb, rows=rows)
    da, dsa, db, dsb = to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb)
    dbs = F.fp8_weight_preshuffle(db)
    ring = [k for k in range(F.gemm_config_count())
            if (F.gemm_config_of(k, SHUF, M, N, K) or {}).get("bm", 0) >= 128]
    assert ring
    for kernel in ring:
        c = to_host(F.fp8_block_gemm_nt_preshuffled(da, dsa, dbs, dsb, c=poisoned_bf16(M, N), kernel=kernel))
        sync()
        gemm_tolerance_check(c[rows], ref, "ring kernel %d" % kernel)
        cfg = F.gemm_config_of(kernel, SHUF, M, N, K)
        plain = [k for k in range(F.gemm_config_count())
                 if F.gemm_config_of(k, False, M, N, K) == {**cfg, "kernel": k}]
        outs = [to_host(F.fp8_block_gemm_nt(da, dsa, db, dsb, c=poisoned_bf16(M, N), kernel=k)) for k in plain]
        sync()
        assert any(np.array_equal(c, x) for x in outs), "ring kernel %d differs from the plain ring tiles" % kernel


def test_preshuffled_masked_gate_up_shape_matches_plain():
    """The masked gate_up workload (32 experts x 256 padded rows, Zipf counts, N 4096, K 7168):
    pre-shuffled equals the plain layout bit for bit on every valid row, and the oracle
    agrees on sampled rows."""
    E, M_max, N, K = W.MOE_E, W.MOE_M_MAX, W.MOE_GATE_UP["N"], W.MOE_GATE_UP["K"]
    counts = W.zipf_counts()
    a, sfa, qb, sfb = _moe_operands(E, M_max, N, K, seed=0)
    db = to_dev(qb)
    dbs = F.fp8_weight_preshuffle(db)
    print("gate_up preshuffled cfg", F.gemm_config(F.LAYOUT_MASKED_PRESHUFFLED, M_max, N, K), flush=True)
    cs = _masked(a, sfa, dbs, sfb, counts, preshuffled=True)
    cp = _masked(a, sfa, db, sfb, counts)
    assert np.array_equal(cs, cp)
    rows = np.array([0, 1, 63, 64, 127, 200, 255])
    ref = O.gemm_grouped_masked(a, sfa, qb, sfb, counts, rows=rows)
    for e in (0, 1, 7, 31):
        sel = np.array([r for r in rows if r < counts[e]], np.int64)
        if sel.size:
            gemm_tolerance_check(cs[e, sel], ref[e, sel], "gate_up expert %d" % e)


def test_preshuffled_prefill_column_tail_matches_plain():
    """2048 x 9216 x 256: 288 tiles of 256 x 256, so the automatic configuration runs the
    first 8192 columns as 256 x 256 ring tiles and the last 1024 as a second launch of
    128 x 128 ring tiles, on either weight layout; the two layouts agree bit for bit and
    sampled rows meet the oracle's tolerance."""
    M, N, K = 2048, 9216, 256
    a = W.normal_bf16((M, K), seed=23)
    b = W.normal_bf16((N, K), std=1.0, seed=23, tensor_id=W.T_B)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    da, dsa, db, dsb = to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb)
    c_shuf = to_host(F.fp8_block_gemm_nt_preshuffled(da, dsa, F.fp8_weight_preshuffle(db), dsb,
                                                     c=poisoned_bf16(M, N)))
    c_plain = to_host(F.fp8_block_gemm_nt(da, dsa, db, dsb, c=poisoned_bf16(M, N)))
    sync()
    rows = np.unique(np.linspace(0, M - 1, 16).astype(np.int64))
    ref = O.gemm_nt(qa, sfa, qb, sfb, rows=rows)
    gemm_tolerance_check(c_shuf[rows], ref, "pre-shuffled, column tail")
    assert np.array_equal(c_shuf, c_plain)


def test_preshuffled_masked_weight_streaming_all_row_groups():
    """The masked weight-streaming entry (every valid row of an expert in one workgroup)
    with M_max = 256 and counts that end inside and on every kind of 16- and 32-row
    boundary, up to all eight 32-row groups and past M_max: every valid row within the
    oracle's tolerance, rows past the count untouched, and bit-equal to the automatic
    plain-layout call."""
    counts = np.array([0, 1, 15, 16, 31, 32, 33, 64, 100, 200, 255, 256, 300], np.int32)
    E, M_max, N, K = len(counts), 256, 384, 1152
    a, sfa, qb, sfb = _moe_operands(E, M_max, N, K, seed=6)
    ref = O.gemm_grouped_masked(a, sfa, qb, sfb, counts)
    db, dbs = to_dev(qb), F.fp8_weight_preshuffle(to_dev(qb))
    streaming = [k for k in range(F.gemm_config_count())
                 if (F.gemm_config_of(k, F.LAYOUT_MASKED_PRESHUFFLED, M_max, N, K) or {}).get("bn") == 128
                 and F.gemm_config_of(k, F.LAYOUT_MASKED, M_max, N, K) is None
                 and F.gemm_config_of(k, F.LAYOUT_DENSE_PRESHUFFLED, 64, N, K) is None]
    assert streaming
    plain = _masked(a, sfa, db, sfb, counts)
    for kernel in streaming:
        print("masked weight streaming kernel %d" % kernel, flush=True)
        c = _masked(a, sfa, dbs, sfb, counts, kernel=kernel, preshuffled=True)
        for e in range(E):
            ce = int(min(max(counts[e], 0), M_max))
            if ce:
                gemm_tolerance_check(c[e, :ce], ref[e, :ce], "kernel %d expert %d" % (kernel, e))
            assert np.all(c[e, ce:] == CANARY), "kernel %d expert %d: padded rows written" % (kernel, e)
        assert np.array_equal(c, plain), "kernel %d differs from the plain-layout call" % kernel
