"""GPU parity of the dense block-scaled GEMM against the CPU oracle.

Operands are quantized by the oracle on the host (never by the GPU), uploaded,
multiplied on the GPU, and compared element by element with the oracle's double
result: |C_gpu - ref| <= 1e-2 |ref| + 1e-2 rms(ref).  Exactly representable
integer problems must match exactly.
"""
import numpy as np
import pytest
import torch

import block_scaled_fp8_token_amd as F
import oracle as O
import workloads as W
from gpu_helpers import DEV, gemm_tolerance_check, poisoned_bf16, sync, to_dev, to_host

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed=0, outliers=False, b_std=0.02, varied_blocks=False):
    if outliers:
        a = W.normal_bf16_outliers((M, K), seed=seed)
    else:
        a = W.normal_bf16((M, K), seed=seed)
    b = W.normal_bf16((N, K), std=b_std, seed=seed, tensor_id=W.T_B)
    if varied_blocks:  # give every 128x128 block its own magnitude so sfb indexing matters
        rng = np.random.default_rng(seed + 17)
        f = W.bf16_bits_to_f32(b)
        mult = 2.0 ** rng.integers(-8, 9, ((N + 127) // 128, K // 128))
        f = f * np.repeat(np.repeat(mult, 128, 0)[:N], 128, 1).astype(np.float32)
        b = W.f32_to_bf16_bits(f.astype(np.float32))
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    return qa, sfa, qb, sfb


def _run(qa, sfa, qb, sfb, kernel=None, splits=None, c=None):
    if c is None:
        c = poisoned_bf16(qa.shape[0], qb.shape[0])
    out = F.fp8_block_gemm_nt(to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb), c=c, kernel=kernel,
                              splits=splits)
    sync()
    return to_host(out)


def _int_codes(vals):
    """e4m3 codes of -1, 0, 1."""
    return np.where(vals > 0, 0x38, np.where(vals < 0, 0xB8, 0x00)).astype(np.uint8)


@pytest.mark.parametrize("kernel", range(F.gemm_config_count()))
@pytest.mark.parametrize("splits", [1, 2])
def test_gemm_integer_identity_exact(kernel, splits):
    rng = np.random.default_rng(kernel * 10 + splits)
    M, N, K = 37, 320, 256
    ai = rng.integers(-1, 2, (M, K))
    bi = rng.integers(-1, 2, (N, K))
    sfb = np.ones((3, 2), np.float32)
    if F.gemm_config_of(kernel, F.LAYOUT_DENSE_FLOAT, M, N, K) is not None:
        # a float-scale entry: unit float scales
        sfa_f = np.ones((K // 128, 40), np.float32)
        c = F.fp8_block_gemm_nt_float_scales(to_dev(_int_codes(ai)), to_dev(sfa_f), to_dev(_int_codes(bi)),
                                             to_dev(sfb), c=poisoned_bf16(M, N), kernel=kernel, splits=splits)
        sync()
        c = to_host(c)
    elif F.gemm_config_of(kernel, F.LAYOUT_DENSE_FLOAT_PRESHUFFLED, M, N, K) is not None:
        # float scales on pre-shuffled weights: unit float scales, shuffled codes
        sfa_f = np.ones((K // 128, 40), np.float32)
        db = F.fp8_weight_preshuffle(to_dev(_int_codes(bi)))
        c = F.fp8_block_gemm_nt_float_scales(to_dev(_int_codes(ai)), to_dev(sfa_f), db, to_dev(sfb),
                                             c=poisoned_bf16(M, N), kernel=kernel, splits=splits, preshuffled=True)
        sync()
        c = to_host(c)
    elif F.gemm_config_of(kernel, F.LAYOUT_DENSE_PRESHUFFLED, M, N, K) is not None:
        # an entry reading pre-shuffled weights: the same integer problem on shuffled codes
        sfa = np.full((1, 40), 127 | (127 << 8), np.uint32)
        db = F.fp8_weight_preshuffle(to_dev(_int_codes(bi)))
        c = F.fp8_block_gemm_nt_preshuffled(to_dev(_int_codes(ai)), to_dev(sfa), db, to_dev(sfb),
                                            c=poisoned_bf16(M, N), kernel=kernel, splits=splits)
        sync()
        c = to_host(c)
    elif (F.gemm_config_of(kernel, F.LAYOUT_MASKED_PRESHUFFLED, M, N, K) is not None
          and F.gemm_config_of(kernel, F.LAYOUT_DENSE, M, N, K) is None):
        # a masked-only entry on pre-shuffled weights: one expert whose count is M
        if splits != 1:
            pytest.skip("masked entries never split K")
        sfa3 = np.full((1, 1, M), 127 | (127 << 8), np.uint32)
        db = F.fp8_weight_preshuffle(to_dev(_int_codes(bi)[None]))
        c = F.fp8_block_gemm_grouped_masked(to_dev(_int_codes(ai)[None]), to_dev(sfa3), db, to_dev(sfb[None]),
                                            to_dev(np.array([M], np.int32)), c=poisoned_bf16(1, M, N),
                                            kernel=kernel, preshuffled=True)
        sync()
        c = to_host(c)[0]
    else:
        sfa = np.full((1, 40), 127 | (127 << 8), np.uint32)
        c = _run(_int_codes(ai), sfa, _int_codes(bi), sfb, kernel=kernel, splits=splits)
    want = (ai @ bi.T).astype(np.float32)
    got = (c.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(got, want)


# K from one K-block up; the three-stage ring turns in trips of twelve K-blocks, so K = 1152
# is one whole trip, 2048 a trip and a four-block tail, 2560 a trip and an eight-block tail
SMALL = [(1, 64, 128), (17, 192, 384), (64, 512, 1024), (100, 640, 640), (130, 256, 512), (257, 384, 1152),
         (130, 256, 2048)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_gemm_parity_every_tile_config(M, N, K):
    print("gemm parity %dx%dx%d" % (M, N, K), flush=True)
    qa, sfa, qb, sfb = _operands(M, N, K, seed=M + N, b_std=1.0, varied_blocks=True)
    ref = O.gemm_nt(qa, sfa, qb, sfb)
    for kernel in range(F.gemm_config_count()):
        if F.gemm_config_of(kernel, False, M, N, K) is None:
            continue  # float-scale entries: covered by the float-scale tests
        for splits in (1, 3):
            c = _run(qa, sfa, qb, sfb, kernel=kernel, splits=splits)
            gemm_tolerance_check(c, ref, "kernel %d splits %d %dx%dx%d" % (kernel, splits, M, N, K))
    c = _run(qa, sfa, qb, sfb)
    gemm_tolerance_check(c, ref, "auto")


def test_gemm_padded_ldc_and_ld_sfa():
    M, N, K = 20, 128, 512
    qa, sfa, qb, sfb = _operands(M, N, K, seed=3)
    ref = O.gemm_nt(qa, sfa, qb, sfb)
    sfa_pad = np.zeros((sfa.shape[0], 40), np.uint32)
    sfa_pad[:, :M] = sfa[:, :M]
    cbuf = torch.full((M, N + 64), -7.0, dtype=torch.bfloat16, device=DEV)
    out = F.fp8_block_gemm_nt(to_dev(qa), to_dev(sfa_pad), to_dev(qb), to_dev(sfb), c=cbuf[:, :N])
    sync()
    full = to_host(cbuf)
    gemm_tolerance_check(full[:, :N], ref, "padded ldc")
    assert np.all(full[:, N:] == 0xC0E0)  # -7.0 canary untouched
    del out


def test_gemm_small_dense_case():
    """8 x 512 x 512, A ~ N(0,1), B ~ N(0, 0.02), seed 0, automatic launch configuration."""
    s = W.DENSE_SMALL
    a, b = W.dense_inputs(s)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    ref = O.gemm_nt(qa, sfa, qb, sfb)
    gemm_tolerance_check(_run(qa, sfa, qb, sfb), ref, s.name)


def test_gemm_decode_full_and_deterministic():
    """64 x 7168 x 18432 with 1% x50 outliers in A: every output element, automatic
    (split-K) configuration; two runs give identical bits."""
    s = W.DENSE_DECODE
    a, b = W.dense_inputs(s)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    ref = O.gemm_nt(qa, sfa, qb, sfb)
    print("decode cfg", F.gemm_config(False, s.M, s.N, s.K), flush=True)
    da, dsa, db, dsb = to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb)
    c1 = F.fp8_block_gemm_nt(da, dsa, db, dsb, c=poisoned_bf16(s.M, s.N))
    c2 = F.fp8_block_gemm_nt(da, dsa, db, dsb, c=poisoned_bf16(s.M, s.N))
    sync()
    c1, c2 = to_host(c1), to_host(c2)
    gemm_tolerance_check(c1, ref, s.name)
    assert np.array_equal(c1, c2)
    ref_bf16 = O.bf16_rne_array(ref)
    assert O.calc_diff(W.bf16_bits_to_f32(c1).astype(np.float64), ref) < 1e-5
    assert np.mean(c1 == ref_bf16) > 0.9


@pytest.mark.parametrize("shape", W.DENSE_PREFILL, ids=lambda s: s.name)
def test_gemm_prefill_every_element(shape):
    """Prefill sweep at full size in the automatic configuration, every output element
    against the oracle (max |err| / bound and calc_diff printed)."""
    M, N, K = shape.M, shape.N, shape.K
    print("prefill", shape.name, F.gemm_config(False, M, N, K), flush=True)
    qa, sfa, qb, sfb = _operands(M, N, K, seed=0)
    c = _run(qa, sfa, qb, sfb)
    ref = O.gemm_nt(qa, sfa, qb, sfb)
    st = gemm_tolerance_check(c, ref, shape.name)
    cd = O.calc_diff(W.bf16_bits_to_f32(c).astype(np.float64), ref)
    print("%s: max |err|/bound %.3f, calc_diff %.3g" % (shape.name, st["max_err_over_bound"], cd), flush=True)
    assert cd < 1e-5


def test_gemm_varied_block_scales_and_outliers():
    M, N, K = 96, 384, 2048
    qa, sfa, qb, sfb = _operands(M, N, K, seed=5, outliers=True, b_std=1.0, varied_blocks=True)
    assert len(np.unique(sfb)) > 5
    ref = O.gemm_nt(qa, sfa, qb, sfb)
    gemm_tolerance_check(_run(qa, sfa, qb, sfb), ref, "varied")


def test_splitk_workspace_reuse_across_shapes():
    """Split-K calls of different shapes on one stream share the library workspace;
    alternating large and small calls must each read back only their own partials."""
    big = _operands(64, 2048, 4096, seed=8)
    small = _operands(96, 384, 2048, seed=9, outliers=True)
    refs = [O.gemm_nt(*big), O.gemm_nt(*small)]
    for rep in range(2):
        for ops, ref, sp in ((big, refs[0], 8), (small, refs[1], 2)):
            c = _run(*ops, kernel=0 if ops is big else 1, splits=sp)
            gemm_tolerance_check(c, ref, "reuse rep %d splits %d" % (rep, sp))
