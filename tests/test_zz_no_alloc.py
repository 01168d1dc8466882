"""The entry point that allocates nothing (fp8_block_gemm_nt_preshuffled_noalloc): its
split-K scratch is the library's static device buffer, its kernels those of
fp8_block_gemm_nt_preshuffled, so its output must equal that entry's bit for bit.

Two calls in a row (the decode shape, then a smaller problem), then the large one again
(the arrival counters must have been left clear), each checked against the existing
entry point on the same inputs and the small one also against the oracle; then the call
captured in a HIP graph and replayed several times with eager work in between."""
import numpy as np
import pytest
import torch

import block_scaled_fp8_token_amd as F
import oracle as O
import workloads as W
from gpu_helpers import DEV, gemm_tolerance_check, poisoned_bf16, sync, to_dev, to_host

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, seed):
    rng = np.random.default_rng(seed)
    a = W.normal_bf16((M, K), seed=seed)
    qa, sfa = O.quant_group_pack(a)
    # valid e4m3 weight bytes (no NaN codes) and power-of-two block scales
    qb = rng.integers(0, 255, (N, K), dtype=np.uint8)
    qb[(qb & 0x7F) == 0x7F] = 0x7E
    sfb = np.ldexp(1.0, rng.integers(-14, -6, ((N + 127) // 128, K // 128))).astype(np.float32)
    return qa, sfa, qb, sfb


def _run_both(qa, sfa, qb, sfb):
    da, dsa, dsb = to_dev(qa), to_dev(sfa), to_dev(sfb)
    db = F.fp8_weight_preshuffle(to_dev(qb))
    M, N = qa.shape[0], qb.shape[0]
    c_ref = poisoned_bf16(M, N)
    F.fp8_block_gemm_nt_preshuffled(da, dsa, db, dsb, c=c_ref)
    c_na = poisoned_bf16(M, N)
    F.fp8_block_gemm_nt_preshuffled_noalloc(da, dsa, db, dsb, c_na)
    sync()
    return to_host(c_na), to_host(c_ref), (da, dsa, db, dsb)


def test_noalloc_matches_preshuffled_entry_twice_then_smaller():
    for (M, N, K), seed in (((64, 7168, 18432), 1), ((8, 512, 1024), 2), ((64, 7168, 18432), 3)):
        print("noalloc %dx%dx%d" % (M, N, K), flush=True)
        qa, sfa, qb, sfb = _inputs(M, N, K, seed)
        got, want, _ = _run_both(qa, sfa, qb, sfb)
        assert np.array_equal(got, want), (M, N, K)
        if M * N <= 8 * 512:
            gemm_tolerance_check(got, O.gemm_nt(qa, sfa, qb, sfb), "noalloc %dx%dx%d" % (M, N, K))


def test_noalloc_graph_replays():
    print("noalloc graph", flush=True)
    qa, sfa, qb, sfb = _inputs(64, 1024, 4096, 4)
    want, _, (da, dsa, db, dsb) = _run_both(qa, sfa, qb, sfb)
    c = poisoned_bf16(64, 1024)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        F.fp8_block_gemm_nt_preshuffled_noalloc(da, dsa, db, dsb, c, stream=s)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        F.fp8_block_gemm_nt_preshuffled_noalloc(da, dsa, db, dsb, c, stream=s)
    other = poisoned_bf16(8, 512)
    qa2, sfa2, qb2, sfb2 = _inputs(8, 512, 1024, 5)
    d2 = (to_dev(qa2), to_dev(sfa2), F.fp8_weight_preshuffle(to_dev(qb2)), to_dev(sfb2))
    sync()
    for rep in range(4):
        c.copy_(poisoned_bf16(64, 1024))
        sync()
        g.replay()
        sync()
        assert np.array_equal(to_host(c), want), rep
        # eager work on the same buffer between the replays
        F.fp8_block_gemm_nt_preshuffled_noalloc(*d2[:3], d2[3], other)
        sync()
