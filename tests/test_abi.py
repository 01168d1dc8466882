"""Host-side tests of the C ABI (no GPU): the library loads, exports every function
the header declares, and rejects bad arguments with the documented status
before touching the device (the validation runs ahead of any HIP call)."""
import ctypes

import pytest

import block_scaled_fp8_token_amd as F

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN = 0, -1, -2, -3

lib = ctypes.CDLL(F.library_path())
lib.fp8bs_status_string.restype = ctypes.c_char_p

# fake but 256-byte aligned addresses: validation never dereferences them
A, B, C, S, T = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def test_header_declares_the_entry_points():
    names = F.declared_functions()
    for n in ("fp8_quant_group_pack", "silu_mul_quant_group_pack", "fp8_block_gemm_nt",
              "fp8_block_gemm_grouped_masked", "fp8_block_quant_128x128", "fp8bs_status_string",
              "fp8_block_gemm_grouped_contiguous", "fp8_quant_group_pack_to_experts", "fp8_quant_group_float",
              "fp8_block_quant_128x128_float", "fp8_block_gemm_nt_float_scales"):
        assert n in names


def test_library_exports_every_declared_symbol():
    for n in F.declared_functions():
        assert hasattr(lib, n), n


def test_status_strings():
    for st in range(-7, 1):
        s = lib.fp8bs_status_string(st).decode()
        assert s and s != "unknown status"
    assert lib.fp8bs_status_string(-99).decode() == "unknown status"


def _gemm(a=A, sfa=S, ld_sfa=64, b=B, sfb=T, c=C, ldc=512, M=64, N=512, K=512):
    f = F._lib.fp8_block_gemm_nt
    return f(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K, None)


def test_gemm_nt_validation():
    assert _gemm(K=100) == ERR_SHAPE
    assert _gemm(K=0) == ERR_SHAPE
    assert _gemm(N=96) == ERR_SHAPE            # N % 64
    assert _gemm(M=-1) == ERR_SHAPE
    assert _gemm(ld_sfa=63) == ERR_SHAPE        # ld_sfa < M
    assert _gemm(ldc=500) == ERR_SHAPE          # ldc < N
    assert _gemm(a=None) == ERR_NULL
    assert _gemm(sfb=None) == ERR_NULL
    assert _gemm(a=A + 8) == ERR_ALIGN
    assert _gemm(c=C + 2) == ERR_ALIGN
    assert _gemm(ldc=516) == ERR_ALIGN          # rows of C not 16-byte aligned
    assert _gemm(sfa=S + 2) == ERR_ALIGN
    assert _gemm(M=0) == OK and _gemm(N=0) == OK  # empty problems are a no-op
    assert _gemm(M=0, a=None) == OK


def _masked(a=A, sfa=S, b=B, sfb=T, c=C, mm=S + 4096, E=4, M_max=64, N=256, K=256):
    return F._lib.fp8_block_gemm_grouped_masked(a, sfa, b, sfb, c, mm, E, M_max, N, K, None)


def test_masked_validation():
    assert _masked(K=200) == ERR_SHAPE
    assert _masked(N=100) == ERR_SHAPE
    assert _masked(E=-2) == ERR_SHAPE
    assert _masked(mm=None) == ERR_NULL
    assert _masked(b=B + 4) == ERR_ALIGN
    assert _masked(mm=S + 4098) == ERR_ALIGN
    assert _masked(E=0) == OK and _masked(M_max=0) == OK


def test_quant_validation():
    f = F._lib.fp8_quant_group_pack
    assert f(A, 512, 8, 500, B, 512, S, 8, None) == ERR_SHAPE          # K % 128
    assert f(A, 256, 8, 512, B, 512, S, 8, None) == ERR_SHAPE          # ldx < K
    assert f(A, 512, 8, 512, B, 512, S, 7, None) == ERR_SHAPE          # ld_sf < M
    assert f(None, 512, 8, 512, B, 512, S, 8, None) == ERR_NULL
    assert f(A + 4, 512, 8, 512, B, 512, S, 8, None) == ERR_ALIGN
    assert f(A, 516, 8, 512, B, 512, S, 8, None) == ERR_ALIGN          # bf16 rows not 16B aligned
    assert f(A, 512, 8, 512, B, 520, S, 8, None) == ERR_ALIGN          # e4m3 rows not 16B aligned
    assert f(A, 512, 0, 512, None, 512, None, 8, None) == OK
    g = F._lib.silu_mul_quant_group_pack
    assert g(A, S, 2, 8, 100, B, T, None) == ERR_SHAPE
    assert g(A, None, 2, 8, 128, B, T, None) == ERR_NULL
    assert g(A, S, 0, 8, 128, None, None, None) == OK
    h = F._lib.fp8_block_quant_128x128
    assert h(A, 128, 100, B, T, None) == ERR_SHAPE
    assert h(A, 128, 128, None, T, None) == ERR_NULL
    assert h(A + 1, 128, 128, B, T, None) == ERR_ALIGN


def test_contiguous_validation():
    f = F._lib.fp8_block_gemm_grouped_contiguous

    def call(a=A, sfa=S, ld_sfa=256, b=B, sfb=T, c=C, ldc=256, mi=S + 8192, E=4, M=256, N=256, K=256):
        return f(a, sfa, ld_sfa, b, sfb, c, ldc, mi, E, M, N, K, None)

    assert call(K=200) == ERR_SHAPE
    assert call(N=96) == ERR_SHAPE
    assert call(E=-1) == ERR_SHAPE
    assert call(ld_sfa=255) == ERR_SHAPE
    assert call(mi=None) == ERR_NULL
    assert call(mi=S + 8194) == ERR_ALIGN
    assert call(E=0) == OK and call(M=0) == OK and call(E=0, mi=None) == OK


def test_quant_to_experts_validation():
    f = F._lib.fp8_quant_group_pack_to_experts

    def call(x=A, ldx=512, T_=8, K=512, ids=S, topk=2, E=4, M_max=16, q=B, sf=T, mm=C, slot=C + 4096):
        return f(x, ldx, T_, K, ids, topk, E, M_max, q, sf, mm, slot, None)

    assert call(K=500) == ERR_SHAPE
    assert call(topk=0) == ERR_SHAPE and call(topk=65) == ERR_SHAPE
    assert call(E=1025) == ERR_SHAPE
    assert call(ldx=256) == ERR_SHAPE
    assert call(ids=None) == ERR_NULL
    assert call(mm=None) == ERR_NULL
    assert call(slot=None) == ERR_NULL
    assert call(q=None) == ERR_NULL
    assert call(x=A + 4) == ERR_ALIGN
    assert call(ids=S + 2) == ERR_ALIGN
    assert call(E=0) == OK


def test_float_scale_validation():
    q = F._lib.fp8_quant_group_float
    assert q(A, 512, 8, 500, B, 512, S, 8, None) == ERR_SHAPE
    assert q(A, 512, 8, 512, B, 512, S, 7, None) == ERR_SHAPE
    assert q(A, 512, 8, 512, B, 512, None, 8, None) == ERR_NULL
    assert q(A, 512, 8, 512, B, 520, S, 8, None) == ERR_ALIGN
    assert q(A, 512, 0, 512, None, 512, None, 8, None) == OK
    h = F._lib.fp8_block_quant_128x128_float
    assert h(A, 128, 100, B, T, None) == ERR_SHAPE
    assert h(A, 128, 128, B, None, None) == ERR_NULL
    g = F._lib.fp8_block_gemm_nt_float_scales
    assert g(A, S, 64, B, T, C, 512, 64, 512, 100, None) == ERR_SHAPE
    assert g(A, S, 63, B, T, C, 512, 64, 512, 512, None) == ERR_SHAPE
    assert g(A, None, 64, B, T, C, 512, 64, 512, 512, None) == ERR_NULL
    assert g(A, S, 64, B, T, C + 2, 512, 64, 512, 512, None) == ERR_ALIGN
    assert g(A, S, 64, B, T, C, 512, 0, 512, 512, None) == OK


def test_preshuffle_validation():
    f = F._lib.fp8_weight_preshuffle
    assert f(A, 48, 512, B, None) == ERR_SHAPE      # rows % 32
    assert f(A, 64, 500, B, None) == ERR_SHAPE      # K % 128
    assert f(A, -32, 512, B, None) == ERR_SHAPE
    assert f(None, 64, 512, B, None) == ERR_NULL
    assert f(A, 64, 512, None, None) == ERR_NULL
    assert f(A + 8, 64, 512, B, None) == ERR_ALIGN
    assert f(A, 0, 512, B, None) == OK and f(None, 0, 512, None, None) == OK
    g = F._lib.fp8_block_gemm_nt_preshuffled
    assert g(A, S, 64, B, T, C, 512, 64, 96, 512, None) == ERR_SHAPE   # N % 64
    assert g(A, S, 64, B, T, C, 512, 64, 512, 500, None) == ERR_SHAPE  # K % 128
    assert g(None, S, 64, B, T, C, 512, 64, 512, 512, None) == ERR_NULL
    assert g(A, S, 64, B + 8, T, C, 512, 64, 512, 512, None) == ERR_ALIGN
    assert g(A, S, 64, B, T, C, 512, 0, 512, 512, None) == OK


def test_preshuffled_masked_k_limit():
    assert F.gemm_config(F.LAYOUT_MASKED_PRESHUFFLED, 256, 4096, 20480)["kernel"] >= 0
    with pytest.raises(F.Fp8bsError):
        F.gemm_config(F.LAYOUT_MASKED_PRESHUFFLED, 256, 4096, 20480 + 128)
    # the plain masked layout falls back to weight streaming there
    assert F.gemm_config(F.LAYOUT_MASKED, 256, 4096, 20480 + 128)["kernel"] >= 0


def test_preshuffled_config_uses_shuffled_entries_only():
    cfg = F.gemm_config(F.LAYOUT_DENSE_PRESHUFFLED, 64, 7168, 18432)
    assert cfg["kernel"] >= 0 and cfg["splits"] >= 1
    for k in range(F.gemm_config_count()):
        plain = F.gemm_config_of(k, F.LAYOUT_DENSE, 64, 7168, 18432, 4)
        shuf = F.gemm_config_of(k, F.LAYOUT_DENSE_PRESHUFFLED, 64, 7168, 18432, 4)
        assert plain is None or shuf is None  # no entry reads both layouts
    assert F.gemm_config_of(cfg["kernel"], F.LAYOUT_DENSE, 64, 7168, 18432, 4) is None
    assert F.gemm_config_of(cfg["kernel"], F.LAYOUT_MASKED, 64, 7168, 18432, 1) is None


def test_config_table_choices():
    n = F.gemm_config_count()
    assert n >= 2
    d = F.gemm_config(False, 64, 7168, 18432)
    assert 0 <= d["kernel"] < n and d["splits"] >= 1
    p = F.gemm_config(False, 4096, 4096, 7168)
    assert p["splits"] == 1 and (p["bm"], p["bn"]) == (256, 256)
    m = F.gemm_config(True, 256, 4096, 7168)
    assert m["splits"] == 1 and (m["bm"], m["bn"]) == (256, 256)
    s = F.gemm_config(False, 2048, 4096, 7168)  # 128 tiles of 256 x 256 would leave half the chip idle
    assert (s["bm"], s["bn"]) == (256, 128)    # 256 tiles of 256 x 128: one whole round
    s = F.gemm_config(False, 1024, 4096, 7168)  # 128 tiles of 256 x 128 would too
    assert (s["bm"], s["bn"]) == (128, 128)     # 256 tiles of 128 x 128: one round
    s = F.gemm_config(False, 1024, 7168, 7168)  # 448 tiles of 128 x 128, 224 of 256 x 128
    assert (s["bm"], s["bn"]) == (256, 128)
    with pytest.raises(F.Fp8bsError):
        F.gemm_config(False, 64, 100, 512)


def test_config_of_table_entries():
    """fp8bs_gemm_config_of: the chosen configuration is one the table accepts; every
    entry takes a small masked problem; entries with K-bounded scale tables refuse a
    masked problem whose K is past them (a masked group never splits K)."""
    n = F.gemm_config_count()
    for masked, (M, N, K) in ((False, (64, 7168, 18432)), (False, (4096, 4096, 7168)), (True, (256, 4096, 7168))):
        c = F.gemm_config(masked, M, N, K)
        e = F.gemm_config_of(c["kernel"], masked, M, N, K, c["splits"])
        assert e is not None and (e["bm"], e["bn"], e["splits"]) == (c["bm"], c["bn"], c["splits"])
    fl = [k for k in range(n) if F.gemm_config_of(k, F.LAYOUT_DENSE_FLOAT, 72, 192, 384) is not None]
    # (the weight-streaming decode entries take M <= 64 only)
    sh = [k for k in range(n) if F.gemm_config_of(k, F.LAYOUT_DENSE_PRESHUFFLED, 72, 192, 384) is not None
          or F.gemm_config_of(k, F.LAYOUT_DENSE_PRESHUFFLED, 64, 192, 384) is not None]
    fsh = [k for k in range(n) if F.gemm_config_of(k, F.LAYOUT_DENSE_FLOAT_PRESHUFFLED, 72, 192, 384) is not None]
    # masked weight streaming: masked calls on pre-shuffled weights only
    msh = [k for k in range(n) if F.gemm_config_of(k, F.LAYOUT_MASKED_PRESHUFFLED, 72, 192, 384) is not None
           and k not in sh and F.gemm_config_of(k, True, 72, 192, 384) is None]
    assert fl and sh and fsh and msh and not set(fl) & set(sh) and not set(fsh) & set(fl + sh)
    assert not set(msh) & set(fl + sh + fsh)
    assert all(F.gemm_config_of(k, False, 72, 192, 384) is None for k in msh)
    assert all(F.gemm_config_of(k, True, 72, 192, 384) is not None for k in range(n) if k not in fl + sh + fsh + msh)
    assert all(F.gemm_config_of(k, True, 72, 192, 384) is None and F.gemm_config_of(k, False, 72, 192, 384) is None
               for k in fsh)
    # the pre-shuffled entries read only that layout (dense calls)
    assert all(F.gemm_config_of(k, False, 72, 192, 384) is None and F.gemm_config_of(k, True, 72, 192, 384) is None
               for k in sh)
    # the float-scale entries read only the float format, the others only the packed one
    assert all(F.gemm_config_of(k, False, 72, 192, 384) is None and F.gemm_config_of(k, True, 72, 192, 384) is None
               for k in fl)
    assert all(F.gemm_config_of(k, F.LAYOUT_DENSE_FLOAT, 72, 192, 384) is None for k in range(n) if k not in fl)
    assert all(F.gemm_config_of(k, F.LAYOUT_DENSE_PRESHUFFLED, 72, 192, 384) is None
               and F.gemm_config_of(k, F.LAYOUT_DENSE_PRESHUFFLED, 64, 192, 384) is None for k in range(n) if k not in sh)
    for M in (8, 64, 4096):
        assert F.gemm_config(F.LAYOUT_DENSE_FLOAT, M, 7168, 7168)["kernel"] in fl
    long_k = [F.gemm_config_of(k, True, 256, 4096, 128 * 1024) for k in range(n)]
    assert any(x is None for x in long_k) and any(x is not None for x in long_k)
    assert all(x is None or x["splits"] == 1 for x in long_k)
    assert F.gemm_config_of(n, False, 64, 128, 128) is None


def test_config_refuses_what_no_entry_takes():
    """A problem no table entry accepts is refused (FP8BS_ERR_SHAPE), never handed to a
    default entry: a masked call with K past every masked kernel's scale tables, and
    every grouped-layout configuration keeps K unsplit."""
    with pytest.raises(F.Fp8bsError) as ei:
        F.gemm_config(True, 256, 4096, 128 * 4096)
    assert ei.value.status == ERR_SHAPE
    for K in (7168, 128 * 1024, 128 * 4096):
        cfg = F.gemm_config(F.LAYOUT_CONTIGUOUS, 256, 4096, K)
        assert cfg["kernel"] >= 0 and cfg["splits"] == 1
        for k in range(F.gemm_config_count()):
            e = F.gemm_config_of(k, F.LAYOUT_CONTIGUOUS, 256, 4096, K)
            assert e is None or e["splits"] == 1, (k, K)
