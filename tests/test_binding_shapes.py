"""The binding rejects tensors whose shapes break the C ABI's layout rules with ValueError,
before any kernel could read or write past them.  The shape checks look at shapes and
strides only, so the CPU tests drive them with host tensors; the GPU tests pass each
undersized device tensor to the wrappers themselves (nothing is launched: the error is
raised first)."""
import pytest
import torch

import block_scaled_fp8_token_amd as F


def _dense(M=64, N=256, K=640, W=None, ld_sfa=None, nb=None, kb=None, c_cols=None, float_scales=False):
    W = W if W is not None else ((K // 128 if float_scales else (K // 128 + 3) // 4))
    a = torch.zeros((M, K), dtype=torch.uint8)
    b = torch.zeros((N, K), dtype=torch.uint8)
    sfa = torch.zeros((W, ld_sfa if ld_sfa is not None else M), dtype=torch.float32 if float_scales else torch.int32)
    sfb = torch.zeros((nb if nb is not None else (N + 127) // 128, kb if kb is not None else K // 128))
    c = torch.zeros((M, c_cols if c_cols is not None else N), dtype=torch.bfloat16)
    return a, sfa, b, sfb, c


def test_dense_shapes_accept_valid_and_padded():
    F.check_dense_shapes(*_dense())
    F.check_dense_shapes(*_dense(ld_sfa=72))          # padded activation-scale columns
    F.check_dense_shapes(*_dense(float_scales=True), float_scales=True)
    a, sfa, b, sfb, c = _dense()
    F.check_dense_shapes(a, sfa, b, sfb, torch.zeros((64, 320), dtype=torch.bfloat16)[:, :256])  # ldc > N


@pytest.mark.parametrize("bad", [dict(W=1), dict(ld_sfa=60), dict(nb=1), dict(kb=4), dict(c_cols=192)])
def test_dense_shapes_reject_undersized(bad):
    with pytest.raises(ValueError):
        F.check_dense_shapes(*_dense(**bad))


def test_dense_float_scale_shapes_reject_packed_height():
    # float scales need one row per K-block (5 here), packed words need 2
    with pytest.raises(ValueError):
        F.check_dense_shapes(*_dense(W=2, float_scales=True), float_scales=True)


def _masked(E=4, M_max=32, N=256, K=640, **over):
    W = (K // 128 + 3) // 4
    t = dict(a=torch.zeros((E, M_max, K), dtype=torch.uint8), sfa=torch.zeros((E, W, M_max), dtype=torch.int32),
             b=torch.zeros((E, N, K), dtype=torch.uint8), sfb=torch.zeros((E, (N + 127) // 128, K // 128)),
             c=torch.zeros((E, M_max, N), dtype=torch.bfloat16), masked_m=torch.zeros((E,), dtype=torch.int32))
    t.update(over)
    return t


def test_masked_shapes():
    F.check_masked_shapes(**_masked())
    for over in (dict(c=torch.zeros((4, 31, 256), dtype=torch.bfloat16)),
                 dict(masked_m=torch.zeros((3,), dtype=torch.int32)),
                 dict(sfa=torch.zeros((4, 1, 32), dtype=torch.int32)),
                 dict(sfa=torch.zeros((4, 2, 31), dtype=torch.int32)),
                 dict(sfb=torch.zeros((4, 2, 4))),
                 dict(sfb=torch.zeros((3, 2, 5))),
                 dict(b=torch.zeros((3, 256, 640), dtype=torch.uint8))):
        with pytest.raises(ValueError):
            F.check_masked_shapes(**_masked(**over))


def test_contiguous_shapes():
    M, N, K, E = 256, 256, 640, 3
    ok = dict(a=torch.zeros((M, K), dtype=torch.uint8), sfa=torch.zeros((2, M), dtype=torch.int32),
              b=torch.zeros((E, N, K), dtype=torch.uint8), sfb=torch.zeros((E, 2, 5)),
              c=torch.zeros((M, N), dtype=torch.bfloat16), m_indices=torch.zeros((M,), dtype=torch.int32))
    F.check_contiguous_shapes(**ok)
    for over in (dict(m_indices=torch.zeros((M - 1,), dtype=torch.int32)),
                 dict(sfa=torch.zeros((2, M - 4), dtype=torch.int32)),
                 dict(sfb=torch.zeros((E - 1, 2, 5))),
                 dict(c=torch.zeros((M, N - 64), dtype=torch.bfloat16))):
        with pytest.raises(ValueError):
            F.check_contiguous_shapes(**dict(ok, **over))


# ---------------------------------------------------------------- wrappers on the GPU

@pytest.mark.gpu
def test_wrappers_reject_undersized_device_tensors():
    dev = "cuda:0"
    M, N, K, E, M_max = 64, 256, 640, 4, 32
    W = (K // 128 + 3) // 4
    u8 = dict(dtype=torch.uint8, device=dev)
    i32 = dict(dtype=torch.int32, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    a, b = torch.zeros((M, K), **u8), torch.zeros((N, K), **u8)
    sfa, sfb = torch.zeros((W, M), **i32), torch.zeros((2, 5), **f32)
    # dense GEMM: undersized activation scales, weight scales, output
    with pytest.raises(ValueError):
        F.fp8_block_gemm_nt(a, torch.zeros((W, M - 4), **i32), b, sfb)
    with pytest.raises(ValueError):
        F.fp8_block_gemm_nt(a, sfa, b, torch.zeros((1, 5), **f32))
    with pytest.raises(ValueError):
        F.fp8_block_gemm_nt_preshuffled(a, torch.zeros((1, M), **i32), b, sfb)
    with pytest.raises(ValueError):
        F.fp8_block_gemm_nt_float_scales(a, torch.zeros((2, M), **f32), b, sfb)  # needs K/128 = 5 rows
    # masked GEMM: output, counts and scales
    am, bm = torch.zeros((E, M_max, K), **u8), torch.zeros((E, N, K), **u8)
    sfam, sfbm = torch.zeros((E, W, M_max), **i32), torch.zeros((E, 2, 5), **f32)
    mm = torch.zeros((E,), **i32)
    with pytest.raises(ValueError):
        F.fp8_block_gemm_grouped_masked(am, sfam, bm, sfbm, mm, c=torch.zeros((E, M_max - 1, N), **bf))
    with pytest.raises(ValueError):
        F.fp8_block_gemm_grouped_masked(am, sfam, bm, sfbm, torch.zeros((E - 1,), **i32))
    with pytest.raises(ValueError):
        F.fp8_block_gemm_grouped_masked(am, torch.zeros((E, W, M_max - 4), **i32), bm, sfbm, mm)
    with pytest.raises(ValueError):
        F.fp8_block_gemm_grouped_masked(am, sfam, bm, torch.zeros((E, 2, 4), **f32), mm)
    # quant into the expert layout: counts with too few entries
    x = torch.zeros((8, K), **bf)
    ids = torch.zeros((8, 2), **i32)
    with pytest.raises(ValueError):
        F.fp8_quant_group_pack_to_experts(x, ids, E, M_max, masked_m=torch.zeros((E - 1,), **i32))
    # per-token quant: scale columns fewer than the rows
    with pytest.raises(ValueError):
        F.fp8_quant_group_pack(torch.zeros((M, K), **bf), sf=torch.zeros((W, M - 4), **i32))
    torch.cuda.synchronize()
