"""One weight-scale contract for every UE8M0 entry point: each reads only the exponent
field of a weight block scale, i.e. uses 2^floor(log2 |s|), whatever kernel the table
picks (the scaled-MFMA kernels, whose scale operand is an E8M0 byte, and the fallbacks
that multiply on the VALU alike).  The scales here are 1.75 * 2^k, so an entry using
the whole value would be 75% off; every entry must match the oracle on 2^k."""
import numpy as np
import pytest

import block_scaled_fp8_token_amd as F
import oracle as O
import workloads as W
from gpu_helpers import gemm_tolerance_check, poisoned_bf16, sync, to_dev, to_host

pytestmark = pytest.mark.gpu


def _operands(M, N, K, seed):
    a = W.normal_bf16((M, K), seed=seed)
    b = W.normal_bf16((N, K), std=1.0, seed=seed, tensor_id=W.T_B)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    rng = np.random.default_rng(seed)
    pow2 = (sfb * np.ldexp(1.0, rng.integers(-3, 4, sfb.shape))).astype(np.float32)
    return qa, sfa, qb, (pow2 * np.float32(1.75)).astype(np.float32), pow2


@pytest.mark.parametrize("M,N,K", [(64, 384, 1024), (200, 256, 640)])
def test_every_dense_entry_reads_the_exponent_only(M, N, K):
    print("scale contract dense %dx%dx%d" % (M, N, K), flush=True)
    qa, sfa, qb, sfb_odd, sfb_pow2 = _operands(M, N, K, seed=M + K)
    ref = O.gemm_nt(qa, sfa, qb, sfb_pow2)
    da, dsa, db, dsb = to_dev(qa), to_dev(sfa), to_dev(qb), to_dev(sfb_odd)
    dbs = F.fp8_weight_preshuffle(db)
    ran = 0
    for kernel in range(F.gemm_config_count()):
        for splits in (1, 3):
            if F.gemm_config_of(kernel, F.LAYOUT_DENSE, M, N, K, splits) is not None:
                c = F.fp8_block_gemm_nt(da, dsa, db, dsb, c=poisoned_bf16(M, N), kernel=kernel, splits=splits)
            elif F.gemm_config_of(kernel, F.LAYOUT_DENSE_PRESHUFFLED, M, N, K, splits) is not None:
                c = F.fp8_block_gemm_nt_preshuffled(da, dsa, dbs, dsb, c=poisoned_bf16(M, N), kernel=kernel,
                                                    splits=splits)
            else:
                continue
            sync()
            gemm_tolerance_check(to_host(c), ref, "kernel %d splits %d" % (kernel, splits))
            ran += 1
    for fn, w in ((F.fp8_block_gemm_nt, db), (F.fp8_block_gemm_nt_preshuffled, dbs)):
        c = fn(da, dsa, w, dsb, c=poisoned_bf16(M, N))
        sync()
        gemm_tolerance_check(to_host(c), ref, "automatic %s" % fn.__name__)
    assert ran >= 10


def test_every_masked_entry_reads_the_exponent_only():
    E, M_max, N, K = 3, 72, 256, 640
    print("scale contract masked", flush=True)
    a, sfa, b, sfb_odd, sfb_pow2 = [], [], [], [], []
    for e in range(E):
        qa, s_a, qb, s_odd, s_pow2 = _operands(M_max, N, K, seed=31 + e)
        a.append(qa), sfa.append(s_a), b.append(qb), sfb_odd.append(s_odd), sfb_pow2.append(s_pow2)
    counts = np.array([72, 5, 40], np.int32)
    da, dsa = to_dev(np.stack(a)), to_dev(np.stack(sfa))
    db, dsb = to_dev(np.stack(b)), to_dev(np.stack(sfb_odd))
    dbs = F.fp8_weight_preshuffle(db)
    refs = [O.gemm_nt(a[e], sfa[e], b[e], sfb_pow2[e]) for e in range(E)]
    for kernel in [None] + list(range(F.gemm_config_count())):
        for layout, w, pre in ((F.LAYOUT_MASKED, db, False), (F.LAYOUT_MASKED_PRESHUFFLED, dbs, True)):
            if kernel is not None and F.gemm_config_of(kernel, layout, M_max, N, K) is None:
                continue
            c = F.fp8_block_gemm_grouped_masked(da, dsa, w, dsb, to_dev(counts), c=poisoned_bf16(E, M_max, N),
                                                kernel=kernel, preshuffled=pre)
            sync()
            c = to_host(c)
            for e in range(E):
                gemm_tolerance_check(c[e, :counts[e]], refs[e][:counts[e]],
                                     "masked kernel %s%s expert %d" % (kernel, " pre" if pre else "", e))
