"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something it does not share code with:
the closed form of the OCP E4M3FN format, torch's own e4m3 cast (a library
routine), hand-derived UE8M0 exponents, exact integer matmuls, a numpy matmul
of the dequantized matrices, scipy's logistic function, and the accuracy figure
printed on the DeepGEMM benchmark post (section 3.3 / 4.4).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W


# ---------------------------------------------------------------- e4m3 format

def test_e4m3_decode_closed_form_points():
    # OCP E4M3FN: bias 7, max normal 448 = 1.75 * 2^8, min normal 2^-6, min subnormal 2^-9
    assert O.e4m3_decode(0x7E) == 448.0
    assert O.e4m3_decode(0x08) == 2.0 ** -6
    assert O.e4m3_decode(0x01) == 2.0 ** -9
    assert O.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert O.e4m3_decode(0x38) == 1.0
    assert O.e4m3_decode(0x40) == 2.0
    assert O.e4m3_decode(0x44) == 3.0
    assert O.e4m3_decode(0xB8) == -1.0
    assert math.isnan(O.e4m3_decode(0x7F)) and math.isnan(O.e4m3_decode(0xFF))
    z = O.e4m3_decode(0x80)
    assert z == 0.0 and math.copysign(1.0, z) == -1.0


def test_e4m3_decode_table_matches_torch():
    tab = O.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    assert np.array_equal(tab[fin], ref[fin])
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must be strictly increasing"
    assert np.array_equal(tab[0x80:0xFF], -tab[:0x7F])


def test_e4m3_encode_roundtrip_all_codes():
    tab = O.e4m3_table()
    for b in range(256):
        if b in (0x7F, 0xFF):
            continue
        assert O.e4m3_encode(tab[b]) == b, hex(b)


def test_e4m3_encode_matches_torch_cast():
    """All bf16 bit patterns, scaled by several powers of two, and random fp32 values:
    wherever torch's RNE cast is defined (|v| < 464) the oracle agrees bit for bit."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    base = bits.view(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        vals = [base * np.float32(2.0 ** s) for s in (0, -3, 5, -20, 9)]
    rng = np.random.default_rng(7)
    vals.append((rng.standard_normal(200000) * 60).astype(np.float32))
    vals.append((rng.random(200000) * 2.0 ** -6).astype(np.float32))
    v = np.concatenate(vals)
    v = v[np.isfinite(v) & (np.abs(v) < 464)]
    want = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3_encode_array(v.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_e4m3_encode_saturates_and_keeps_sign_of_zero():
    assert O.e4m3_encode(448.0) == 0x7E
    assert O.e4m3_encode(470.0) == 0x7E
    assert O.e4m3_encode(1e30) == 0x7E
    assert O.e4m3_encode(-1e30) == 0xFE
    assert O.e4m3_encode(-0.0) == 0x80
    assert O.e4m3_encode(-1e-9) == 0x80
    assert O.e4m3_encode(1e-9) == 0x00
    # ties go to the even mantissa: 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39)
    assert O.e4m3_encode(1.0625) == 0x38
    assert O.e4m3_encode(1.1875) == 0x3A  # halfway between 1.125 (0x39) and 1.25 (0x3A)
    # smallest subnormal tie: 2^-10 is halfway between 0 and 2^-9 -> 0
    assert O.e4m3_encode(2.0 ** -10) == 0x00
    assert O.e4m3_encode(3 * 2.0 ** -10) == 0x02


def test_e4m3_encode_error_bound():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 0.1, 10, 100)])
    v = v[np.abs(v) < 448]
    tab = O.e4m3_table()
    q = O.e4m3_encode_array(v)
    err = np.abs(tab[q] - v)
    # half an ulp: ulp = 2^(floor(log2|v|) - 3) in the normal range, 2^-9 below 2^-6
    a = np.abs(v)
    ulp = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3))
    assert np.all(err <= ulp / 2)


# ---------------------------------------------------------------- UE8M0 scale

@pytest.mark.parametrize("amax,byte", [(448.0, 127), (449.0, 128), (224.0, 126), (224.5, 127),
                                       (1.0, 119), (0.0, 85), (1e-30, 85), (896.0, 128),
                                       (448.0 * 2 ** 20, 147), (3.3895313892515355e38, 247)])
def test_ue8m0_hand_cases(amax, byte):
    # the scale is amax/448 rounded UP to a power of two; the byte is e + 127; amax floored at 1e-10
    assert O.ue8m0_exponent(amax) + 127 == byte


def test_ue8m0_bracket_invariant():
    rng = np.random.default_rng(3)
    vals = np.concatenate([np.exp(rng.uniform(-30, 80, 5000)), 448.0 * 2.0 ** rng.integers(-40, 100, 500)])
    for a in vals:
        e = O.ue8m0_exponent(float(a))
        fa = max(Fraction(float(a)), Fraction(1e-10))  # amax is floored at 1e-10
        assert Fraction(448) * Fraction(2) ** e >= fa
        assert Fraction(448) * Fraction(2) ** (e - 1) < fa


# ---------------------------------------------------------------- quant + pack

def test_quant_roundtrip_bound_and_group_max():
    x = W.normal_bf16((6, 1024), seed=5)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    q, sf = O.quant_group_pack(x)
    tab = O.e4m3_table()
    for r in range(6):
        for g in range(8):
            e = int((sf[g // 4, r] >> (8 * (g % 4))) & 0xFF) - 127
            seg = xf[r, 128 * g:128 * g + 128]
            deq = tab[q[r, 128 * g:128 * g + 128]] * 2.0 ** e
            scaled = np.abs(seg) * 2.0 ** -e
            ulp = np.where(scaled < 2.0 ** -6, 2.0 ** -9,
                           2.0 ** (np.floor(np.log2(np.maximum(scaled, 2.0 ** -6))) - 3))
            assert np.all(np.abs(deq - seg) <= ulp / 2 * 2.0 ** e)
            m = np.max(np.abs(tab[q[r, 128 * g:128 * g + 128]]))
            assert 224 <= m <= 448


def test_pack_layout_closed_form():
    """Row r, group g gets amax = 448 * 2^(r + 2g - 6) exactly, so its byte is 121 + r + 2g;
    K = 640 gives 5 groups (word 1 only has byte 0), M = 5 with ld_sf = 8."""
    M, K = 5, 640
    x = np.zeros((M, K), np.float32)
    rng = np.random.default_rng(1)
    for r in range(M):
        for g in range(5):
            amax = 448.0 * 2.0 ** (r + 2 * g - 6)
            seg = rng.uniform(-amax, amax, 128).astype(np.float32)
            seg[int(rng.integers(128))] = -amax
            x[r, 128 * g:128 * g + 128] = seg
    xb = W.f32_to_bf16_bits(x)
    q, sf = O.quant_group_pack(xb, ld_sf=8)
    assert sf.shape == (2, 8)
    for r in range(M):
        b = [121 + r + 2 * g for g in range(5)]
        assert sf[0, r] == b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24)
        assert sf[1, r] == b[4]
        # the element that equals -amax encodes to -448 (0xFE)
        for g in range(5):
            assert 0xFE in q[r, 128 * g:128 * g + 128]


def test_zero_group_and_negative_zero():
    x = np.zeros((1, 128), np.uint16)
    x[0, 5] = 0x8000  # -0.0
    q, sf = O.quant_group_pack(x)
    assert sf[0, 0] == 85
    assert q[0, 5] == 0x80 and np.count_nonzero(q) == 1


# ---------------------------------------------------------------- weight block quant

def test_block_quant_weight_blocks():
    N, K = 200, 384  # partial last row block
    w = W.normal_bf16((N, K), std=0.02, seed=9, tensor_id=W.T_B)
    wf = W.bf16_bits_to_f32(w).astype(np.float64)
    # plant one large value in block (1, 2) to make the block exponents differ
    wf_big = wf.copy()
    wf_big[150, 300] = 3.0
    w2 = W.f32_to_bf16_bits(wf_big.astype(np.float32))
    q, sfb = O.block_quant_128x128(w2)
    assert sfb.shape == (2, 3)
    tab = O.e4m3_table()
    wf2 = W.bf16_bits_to_f32(w2).astype(np.float64)
    for nb in range(2):
        for kb in range(3):
            blk = wf2[128 * nb:min(N, 128 * nb + 128), 128 * kb:128 * kb + 128]
            s = float(sfb[nb, kb])
            assert s == 2.0 ** round(math.log2(s))
            amax = np.max(np.abs(blk))
            assert 448 * s >= amax > 224 * s
            deq = tab[q[128 * nb:min(N, 128 * nb + 128), 128 * kb:128 * kb + 128]] * s
            assert np.max(np.abs(deq - blk)) <= s * 16  # half ulp at the top binade (32/2)
    assert sfb[1, 2] == 2.0 ** -7  # 3.0 / 448 -> 2^-7.2 -> rounded up to 2^-7
    assert sfb[0, 0] == 2.0 ** -12  # N(0, 0.02) blocks: amax ~ 0.09 -> 2^-12.2 -> 2^-12


# ---------------------------------------------------------------- GEMM

def _int_e4m3_codes(vals):
    """e4m3 codes of small integers via the format's closed form (not the oracle encoder)."""
    out = np.zeros(vals.shape, np.uint8)
    for idx, v in np.ndenumerate(vals):
        v = int(v)
        if v == 0:
            out[idx] = 0
            continue
        s = 0x80 if v < 0 else 0
        a = abs(v)
        E = a.bit_length() - 1           # a = 2^E * (1 + m/8)
        m = (a - (1 << E)) * 8 // (1 << E)
        assert (1 << E) + m * (1 << E) // 8 == a
        out[idx] = s | ((E + 7) << 3) | m
    return out


def test_gemm_integer_identity():
    rng = np.random.default_rng(2)
    M, N, K = 7, 130, 384
    # integers in [-16, 16] that are exact in e4m3 (all are)
    ai = rng.integers(-16, 17, (M, K))
    bi = rng.integers(-16, 17, (N, K))
    qa, qb = _int_e4m3_codes(ai), _int_e4m3_codes(bi)
    sfa = np.full((1, 8), 127 | (127 << 8) | (127 << 16), np.uint32)  # 3 groups, scale 1
    sfb = np.ones((2, 3), np.float32)
    c = O.gemm_nt(qa, sfa, qb, sfb)
    assert np.array_equal(c, (ai @ bi.T).astype(np.float64))


def test_gemm_equals_dequantized_matmul_with_varied_scales():
    """Block-scaled GEMM == plain matmul of the dequantized operands (torch decodes e4m3)."""
    rng = np.random.default_rng(4)
    for (M, N, K) in [(1, 1, 128), (3, 129, 256), (129, 3, 640), (5, 300, 640)]:
        G = K // 128
        Wd = (G + 3) // 4
        qa = rng.integers(0, 256, (M, K), dtype=np.uint8)
        qb = rng.integers(0, 256, (N, K), dtype=np.uint8)
        qa[(qa & 0x7F) == 0x7F] = 0x3C  # no NaN codes
        qb[(qb & 0x7F) == 0x7F] = 0x41
        ea = rng.integers(-20, 21, (M, G))
        sfa = np.zeros((Wd, M + 3), np.uint32)
        for m in range(M):
            for g in range(G):
                sfa[g // 4, m] |= np.uint32((ea[m, g] + 127) << (8 * (g % 4)))
        eb = rng.integers(-20, 21, ((N + 127) // 128, G))
        sfb = (2.0 ** eb).astype(np.float32)
        c = O.gemm_nt(qa, sfa, qb, sfb)
        dec = lambda q: torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        A = dec(qa) * np.repeat(2.0 ** ea, 128, axis=1)
        B = dec(qb) * np.repeat(np.repeat(2.0 ** eb, 128, axis=0)[:N], 128, axis=1)
        ref = A @ B.T
        bound = (np.abs(A) @ np.abs(B).T) * 2.0 ** -50
        assert np.all(np.abs(c - ref) <= bound)
        # and one entry exactly, with rational arithmetic
        fa = [Fraction(float(v)) for v in A[M - 1]]
        fb = [Fraction(float(v)) for v in B[N - 1]]
        exact = sum(x * y for x, y in zip(fa, fb))
        assert abs(Fraction(c[M - 1, N - 1]) - exact) <= abs(exact) * Fraction(1, 2 ** 52)


def test_gemm_row_col_selection_matches_full():
    rng = np.random.default_rng(8)
    a = W.normal_bf16((9, 256), seed=1)
    b = W.normal_bf16((140, 256), std=0.02, seed=1, tensor_id=W.T_B)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    full = O.gemm_nt(qa, sfa, qb, sfb)
    rows = np.array([8, 0, 3])
    cols = np.array([139, 0, 128, 127])
    sub = O.gemm_nt(qa, sfa, qb, sfb, rows=rows, cols=cols)
    assert np.array_equal(sub, full[np.ix_(rows, cols)])


def test_calc_diff_closed_forms():
    x = np.random.default_rng(0).standard_normal(1000)
    assert O.calc_diff(x, x) == pytest.approx(0.0, abs=1e-15)
    assert O.calc_diff(x, -x) == pytest.approx(2.0)
    assert O.calc_diff(x, 2 * x) == pytest.approx(0.2)


def _golden_calc_diff():
    import os
    p = os.path.join(os.path.dirname(__file__), "golden", "deepgemm_h100_summary.txt")
    for line in open(p):
        if line.startswith("deepgemm"):
            return float(line.split()[4])
    raise AssertionError("fixture missing")


def test_whole_scheme_accuracy_matches_published_calc_diff():
    """A, B ~ randn in bf16, B in 128x128 blocks and A in 1x128 groups with UE8M0 scales:
    calc_diff of the quantized GEMM against the unquantized product is ~0.000684 on the post."""
    want = _golden_calc_diff()
    m, n, k = 128, 512, 7168
    a = W.normal_bf16((m, k), seed=42, tensor_id=W.T_A)
    b = W.normal_bf16((n, k), seed=42, tensor_id=W.T_B)
    qa, sfa = O.quant_group_pack(a)
    qb, sfb = O.block_quant_128x128(b)
    c = O.gemm_nt(qa, sfa, qb, sfb)
    ref = W.bf16_bits_to_f32(a).astype(np.float64) @ W.bf16_bits_to_f32(b).astype(np.float64).T
    d = O.calc_diff(c, ref)
    assert 0.9 * want <= d <= 1.1 * want, d


# ---------------------------------------------------------------- masked grouped GEMM

def _moe_inputs(E, M_max, N, K, seed=0):
    x = W.normal_bf16((E * M_max, K), seed=seed)
    qa, sfa_flat = O.quant_group_pack(x, ld_sf=E * M_max)
    Wd = (K // 128 + 3) // 4
    a = qa.reshape(E, M_max, K)
    # [W][E*M_max] -> [E][W][M_max]
    sfa = np.ascontiguousarray(sfa_flat.reshape(Wd, E, M_max).transpose(1, 0, 2))
    bs, sfbs = [], []
    for e in range(E):
        w = W.normal_bf16((N, K), std=0.02, seed=seed + 100 + e, tensor_id=W.T_B)
        qb, sfb = O.block_quant_128x128(w)
        bs.append(qb)
        sfbs.append(sfb)
    return a, sfa, np.stack(bs), np.stack(sfbs)


def test_masked_full_counts_equal_dense_per_expert():
    E, M_max, N, K = 3, 8, 136, 256
    a, sfa, b, sfb = _moe_inputs(E, M_max, N, K)
    out = O.gemm_grouped_masked(a, sfa, b, sfb, np.full(E, M_max, np.int32))
    for e in range(E):
        assert np.array_equal(out[e], O.gemm_nt(a[e], sfa[e], b[e], sfb[e]))


def test_masked_counts_clamped_and_rows_untouched():
    E, M_max, N, K = 4, 8, 128, 128
    a, sfa, b, sfb = _moe_inputs(E, M_max, N, K, seed=3)
    mm = np.array([0, 3, 99, -5], np.int32)
    out = O.gemm_grouped_masked(a, sfa, b, sfb, mm)
    assert np.all(np.isnan(out[0])) and np.all(np.isnan(out[3]))
    assert np.all(np.isnan(out[1, 3:])) and not np.any(np.isnan(out[1, :3]))
    assert not np.any(np.isnan(out[2]))  # 99 clamps to M_max
    assert np.array_equal(out[1, :3], O.gemm_nt(a[1], sfa[1], b[1], sfb[1])[:3])


# ---------------------------------------------------------------- float-scale format

def _torch_e4m3(y32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_float_quant_matches_fp32_formula_and_torch_cast():
    """s = fp32(max(amax, 1e-10) / 448), q = RNE cast of clamp(fp32(x / s)): numpy fp32
    arithmetic and torch's float8_e4m3fn cast, group by group; zero and tiny groups too."""
    M, K = 6, 640
    x = W.normal_bf16((M, K), seed=9)
    x[1, 128:256] = 0                        # a zero group: s = 1e-10 / 448
    x[2, :128] = W.f32_to_bf16_bits(np.full(128, 1e-20, np.float32))  # below the floor
    q, sf = O.quant_group_float(x)
    xf = W.bf16_bits_to_f32(x)
    for r in range(M):
        for g in range(K // 128):
            blk = xf[r, g * 128:(g + 1) * 128]
            amax = np.float32(np.abs(blk).max())
            s = np.float32(max(amax, np.float32(1e-10))) / np.float32(448.0)
            assert sf[g, r] == s, (r, g)
            y = np.clip(blk / s, np.float32(-448), np.float32(448)).astype(np.float32)
            assert np.array_equal(q[r, g * 128:(g + 1) * 128], _torch_e4m3(y)), (r, g)


def test_float_block_quant_matches_fp32_formula():
    N, K = 200, 256
    w = W.normal_bf16((N, K), std=0.02, seed=10, tensor_id=W.T_B)
    q, sfb = O.block_quant_128x128_float(w)
    wf = W.bf16_bits_to_f32(w)
    for nb in range(2):
        for kb in range(2):
            blk = wf[nb * 128:min(N, nb * 128 + 128), kb * 128:(kb + 1) * 128]
            s = np.float32(max(np.float32(np.abs(blk).max()), np.float32(1e-10))) / np.float32(448.0)
            assert sfb[nb, kb] == s
            y = np.clip(blk / s, np.float32(-448), np.float32(448)).astype(np.float32)
            assert np.array_equal(q[nb * 128:min(N, nb * 128 + 128), kb * 128:(kb + 1) * 128], _torch_e4m3(y))


def test_float_gemm_exact_rational_small_case():
    """Integer operands, arbitrary fp32 scales: every output in exact rational arithmetic."""
    rng = np.random.default_rng(12)
    M, N, K = 3, 130, 256
    ai = rng.integers(-16, 17, (M, K))
    bi = rng.integers(-16, 17, (N, K))
    sfa = rng.uniform(0.001, 3.0, (K // 128, 4)).astype(np.float32)
    sfb = rng.uniform(0.001, 3.0, (2, K // 128)).astype(np.float32)
    out = O.gemm_nt_float_scales(_int_e4m3_codes(ai), sfa, _int_e4m3_codes(bi), sfb)
    for m in range(M):
        for n in range(N):
            ref, mag = Fraction(0), Fraction(0)
            for kb in range(K // 128):
                dot = int(ai[m, kb * 128:(kb + 1) * 128] @ bi[n, kb * 128:(kb + 1) * 128])
                term = Fraction(float(sfa[kb, m])) * Fraction(float(sfb[n // 128, kb])) * dot
                ref += term
                mag += abs(term)
            # double rounding of each scaled block sum and of the running sum
            assert abs(Fraction(out[m, n]) - ref) <= mag * Fraction(1, 2 ** 50), (m, n)


def test_float_gemm_with_power_of_two_scales_equals_packed_gemm():
    """Float scales that are powers of two give the packed-UE8M0 GEMM's result exactly."""
    rng = np.random.default_rng(13)
    M, N, K = 5, 256, 640
    G = K // 128
    qa = rng.integers(0, 256, (M, K), dtype=np.uint8)
    qb = rng.integers(0, 256, (N, K), dtype=np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0
    qb[(qb & 0x7F) == 0x7F] = 0
    ea = rng.integers(-10, 11, (M, G))
    words = np.zeros(((G + 3) // 4, 8), np.uint32)
    for m in range(M):
        for g in range(G):
            words[g // 4, m] |= np.uint32((ea[m, g] + 127) << (8 * (g % 4)))
    sfa_f = np.zeros((G, 8), np.float32)
    sfa_f[:, :M] = np.ldexp(1.0, ea.T)
    sfb = np.ldexp(1.0, rng.integers(-10, 11, (2, G))).astype(np.float32)
    assert np.array_equal(O.gemm_nt_float_scales(qa, sfa_f, qb, sfb), O.gemm_nt(qa, words, qb, sfb))


# ---------------------------------------------------------------- quant into the expert layout

def _dispatch_case(seed=0):
    rng = np.random.default_rng(seed)
    T, topk, E, M_max, K = 41, 3, 5, 9, 640
    ids = rng.integers(-1, E + 2, (T, topk)).astype(np.int32)  # -1 and >= E: not routed
    ids[0] = [2, 2, 2]                                         # one token routed thrice to one expert
    x = W.normal_bf16((T, K), seed=seed, tensor_id=W.T_X)
    return x, ids, E, M_max


def test_dispatch_slots_brute_force():
    """Slots and counts against a dictionary walk over the pairs in token-major order."""
    x, ids, E, M_max = _dispatch_case(1)
    _, _, mm, slot = O.quant_group_pack_to_experts(x, ids, E, M_max)
    seen = {}
    for t in range(ids.shape[0]):
        for j in range(ids.shape[1]):
            e = int(ids[t, j])
            if not 0 <= e < E:
                assert slot[t, j] == -1
                continue
            k = seen.get(e, 0)
            seen[e] = k + 1
            assert slot[t, j] == (k if k < M_max else -1), (t, j)
    assert [int(v) for v in mm] == [min(seen.get(e, 0), M_max) for e in range(E)]
    assert any(seen.get(e, 0) > M_max for e in range(E))  # the case exercises the capacity


def test_dispatch_rows_are_the_token_quant():
    """Every written row equals the per-token quant of its token (the pinned a1 oracle);
    rows at or past the count stay zero."""
    x, ids, E, M_max = _dispatch_case(2)
    q, sf, mm, slot = O.quant_group_pack_to_experts(x, ids, E, M_max)
    qt, sft = O.quant_group_pack(x, ld_sf=x.shape[0])
    written = np.zeros((E, M_max), bool)
    for t, j in zip(*np.nonzero(slot >= 0)):
        e, sl = ids[t, j], slot[t, j]
        assert np.array_equal(q[e, sl], qt[t])
        assert np.array_equal(sf[e, :, sl], sft[:, t])
        written[e, sl] = True
    for e in range(E):
        assert written[e, :mm[e]].all() and not written[e, mm[e]:].any()
        assert not q[e, mm[e]:].any()


# ---------------------------------------------------------------- contiguous grouped GEMM

def test_contiguous_integer_brute_force_with_varied_scales():
    """Integer operands (exact in e4m3), power-of-two activation and weight scales that
    differ per row, group, column block and K-block: the exact result is an integer
    matmul per row against that row's group, scaled per K-block (numpy int64 sums)."""
    rng = np.random.default_rng(11)
    E, N, K = 3, 192, 640
    G, NB = K // 128, (N + 127) // 128
    Wd = (G + 3) // 4
    mi = W.contiguous_layout([130, 0, 5], tail_blocks=1)
    mi[-3] = 7  # a row naming no group (past E): padding
    M = len(mi)
    ai = rng.integers(-16, 17, (M, K))
    bi = rng.integers(-16, 17, (E, N, K))
    qa, qb = _int_e4m3_codes(ai), _int_e4m3_codes(bi)
    ea = rng.integers(-3, 4, (M, G))
    sfa = np.zeros((Wd, M), np.uint32)
    for m in range(M):
        for g in range(G):
            sfa[g // 4, m] |= np.uint32((ea[m, g] + 127) << (8 * (g % 4)))
    eb = rng.integers(-3, 4, (E, NB, G))
    sfb = np.ldexp(1.0, eb).astype(np.float32)
    out = O.gemm_grouped_contiguous(qa, sfa, qb, sfb, mi)
    for m in range(M):
        g = mi[m]
        if not (0 <= g < E):
            assert np.all(np.isnan(out[m]))
            continue
        ref = np.zeros(N)
        for kb in range(G):
            dots = bi[g][:, kb * 128:(kb + 1) * 128] @ ai[m, kb * 128:(kb + 1) * 128]
            ref += np.ldexp(1.0, ea[m, kb]) * np.ldexp(1.0, eb[g][np.arange(N) // 128, kb]) * dots
        assert np.array_equal(out[m], ref), m


def test_contiguous_single_group_equals_dense_and_rows_select():
    E, N, K = 1, 128, 256
    a, sfa, b, sfb = _moe_inputs(1, 256, N, K, seed=5)
    mi = np.zeros(256, np.int32)
    out = O.gemm_grouped_contiguous(a[0], sfa[0], b, sfb, mi)
    assert np.array_equal(out, O.gemm_nt(a[0], sfa[0], b[0], sfb[0]))
    part = O.gemm_grouped_contiguous(a[0], sfa[0], b, sfb, mi, rows=[3, 200])
    assert np.array_equal(part[[3, 200]], out[[3, 200]])
    assert np.all(np.isnan(np.delete(part, [3, 200], axis=0)))


# ---------------------------------------------------------------- SiLU-mul-quant

def test_silu_mul_matches_logistic_closed_form():
    from scipy.special import expit
    E, M_max, H = 2, 4, 256
    x = W.normal_bf16((E, M_max, 2 * H), seed=6, tensor_id=W.T_X)
    mm = np.array([3, 1], np.int32)
    q, sf, y = O.silu_mul_quant_group_pack(x, mm, want_y=True)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    g, u = xf[..., :H], xf[..., H:]
    ref = g * expit(g) * u
    for e in range(E):
        c = mm[e]
        assert np.allclose(y[e, :c], ref[e, :c], rtol=1e-14, atol=1e-300)
        assert np.all(np.isnan(y[e, c:]))
        assert np.all(q[e, c:] == 0) and np.all(sf[e, :, c:] == 0)


def test_silu_mul_special_values():
    H = 128
    x = np.zeros((1, 4, 2 * H), np.float32)
    x[0, 1, :H] = 30.0       # silu(30) = 30 (to double precision) -> y = 30 * u
    x[0, 1, H:] = 0.5
    x[0, 2, :H] = 1.0        # u = 0 -> y = 0 -> all-zero group
    x[0, 3, 7] = -2.0
    x[0, 3, H + 7] = 3.0     # single nonzero: silu(-2) * 3 = -0.7153...
    xb = W.f32_to_bf16_bits(x)
    q, sf = O.silu_mul_quant_group_pack(xb, np.array([4], np.int32))
    assert sf[0, 0, 0] == 85 and np.all(q[0, 0] == 0)          # g = u = 0
    assert sf[0, 0, 2] == 85 and np.all((q[0, 2] & 0x7F) == 0)
    # y = 15 everywhere: e = ceil(log2(15/448)) = -4 -> 15 * 16 = 240 exactly (0x77)
    assert sf[0, 0, 1] == 123 and np.all(q[0, 1] == 0x77)
    yv = -2.0 / (1 + math.exp(2.0)) * 3.0
    e = math.ceil(math.log2(abs(yv) / 448))
    assert sf[0, 0, 3] == 127 + e
    want = torch.tensor([yv * 2.0 ** -e], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    assert q[0, 3, 7] == int(want[0]) == 0xFB  # -366.2 -> -352


@pytest.mark.parametrize("H", [640, 2048])
def test_silu_quant_pack_equals_group_quant_of_exact_y(H):
    """Fused == SiLU then the (separately pinned) per-token-group quant, on every valid row.

    Gate values lie in [20, 60], where silu(g) = g / (1 + e^-g) differs from g by a relative
    e^-g < 2.1e-9, far below half an fp32 ulp; up values are +-2^k.  So y = g * u exactly
    (a bf16 value), and the fused oracle's bytes and packed words must equal those of
    quant_group_pack applied to y.  k varies with row and group, so neighbouring groups have
    different exponents: a wrong word index or byte shift in the masked [E][W][M_max] layout
    cannot pass.  H = 640 gives 5 groups (a partial second word), H = 2048 gives 4 words."""
    E, M_max = 3, 8
    counts = np.array([5, 0, 8], np.int32)
    rng = np.random.default_rng(H)
    G = H // 128
    gate = rng.uniform(20.0, 60.0, (E, M_max, H)).astype(np.float32)
    gate = W.bf16_bits_to_f32(W.f32_to_bf16_bits(gate))
    k = np.zeros((E, M_max, G), np.int64)
    for e in range(E):
        for r in range(M_max):
            for g in range(G):
                k[e, r, g] = (7 * r + 3 * g + 5 * e) % 13 - 6
    up = np.repeat(np.ldexp(1.0, k), 128, axis=2) * rng.choice([-1.0, 1.0], (E, M_max, H))
    x = W.f32_to_bf16_bits(np.concatenate([gate, up.astype(np.float32)], axis=2))
    y = (gate.astype(np.float64) * up).astype(np.float32)
    yb = W.f32_to_bf16_bits(y)
    assert np.array_equal(W.bf16_bits_to_f32(yb), y), "y must be exact in bf16"
    q, sf = O.silu_mul_quant_group_pack(x, counts)
    Wd = (G + 3) // 4
    assert q.shape == (E, M_max, H) and sf.shape == (E, Wd, M_max)
    for e in range(E):
        qr, sfr = O.quant_group_pack(yb[e], ld_sf=M_max)
        c = counts[e]
        assert np.array_equal(q[e, :c], qr[:c]), e
        assert np.array_equal(sf[e, :, :c], sfr[:, :c]), e
        # rows at or past the count are not written (the wrapper's zeros remain)
        assert not q[e, c:].any() and not sf[e, :, c:].any()
    # the test has power: exponents differ between neighbouring groups of a row
    bytes_ = [(sf[2, g // 4, 0] >> (8 * (g % 4))) & 0xFF for g in range(G)]
    assert len(set(bytes_)) > 1 and all(85 <= b <= 247 for b in bytes_)


def test_silu_quant_pack_general_values_against_torch_cast():
    """General SiLU inputs (N(0,1) with a different magnitude per group): each valid row's
    bytes equal torch's e4m3 cast of fp32(y) * 2^-e, where y is the oracle's double SiLU
    product (pinned to scipy above) and e is the smallest integer with 448 * 2^e >= max(amax,
    1e-10), found by exact comparison; byte g % 4 of word g / 4 of the row holds e + 127."""
    E, M_max, H = 2, 6, 640
    G = H // 128
    rng = np.random.default_rng(11)
    xs = rng.standard_normal((E, M_max, 2 * H))
    scale = np.ldexp(1.0, rng.integers(-12, 12, (E, M_max, G)))
    xs[..., :H] *= np.repeat(scale, 128, axis=2)
    xs[..., H:] *= np.repeat(scale[..., ::-1], 128, axis=2)
    x = W.f32_to_bf16_bits(xs.astype(np.float32))
    counts = np.array([6, 3], np.int32)
    q, sf, y = O.silu_mul_quant_group_pack(x, counts, want_y=True)
    for e in range(E):
        for r in range(counts[e]):
            for g in range(G):
                y32 = y[e, r, 128 * g:128 * g + 128].astype(np.float32)
                amax = max(float(np.max(np.abs(y32))), 1e-10)
                ex = math.frexp(amax / 448.0)[1]
                while Fraction(448) * Fraction(2) ** (ex - 1) >= Fraction(amax):
                    ex -= 1
                while Fraction(448) * Fraction(2) ** ex < Fraction(amax):
                    ex += 1
                assert (int(sf[e, g // 4, r]) >> (8 * (g % 4))) & 0xFF == ex + 127, (e, r, g)
                want = torch.from_numpy(np.ldexp(y32, -ex).astype(np.float32)).to(torch.float8_e4m3fn)
                assert np.array_equal(q[e, r, 128 * g:128 * g + 128], want.view(torch.uint8).numpy()), (e, r, g)
            # bytes of the missing groups 5..7 of the last word are zero
            assert (int(sf[e, 1, r]) >> 8) == 0


# ---------------------------------------------------------------- bf16 rounding

def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(12)
    v = np.concatenate([rng.standard_normal(3000).astype(np.float32) * 100,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0e38, 1e-40],
                                 np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.bf16_rne_array(v.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(W.f32_to_bf16_bits(v), want)


def test_weight_preshuffle_layout_properties():
    """The pre-shuffled weight layout is a byte permutation whose every 1 KB load (g, kb, q)
    gives lane l sixteen consecutive bytes of row 32g + (l mod 32), and whose two loads
    q = 2h, 2h + 1 give that lane the 32 consecutive K-bytes 128kb + 64h + 32*(l div 32) ..
    + 31: the operand of lane l for the h-th 64-wide MFMA of K-block kb (a 32-row x 64-K
    operand, lane l holding row l mod 32 and the (l div 32)-th 32-byte half of the K range).
    Checked with position-coded inputs (the source row and column of every output byte)."""
    rows, K = 96, 640
    r_idx, c_idx = np.meshgrid(np.arange(rows), np.arange(K), indexing="ij")
    src_row = O.weight_preshuffle(r_idx.astype(np.uint8)).reshape(-1).astype(np.int64)
    src_lo = O.weight_preshuffle((c_idx % 256).astype(np.uint8)).reshape(-1).astype(np.int64)
    src_hi = O.weight_preshuffle((c_idx // 256).astype(np.uint8)).reshape(-1).astype(np.int64)
    src_col = src_lo + 256 * src_hi
    # a bijection: every (row, col) appears exactly once
    flat = np.sort(src_row * K + src_col)
    assert np.array_equal(flat, np.arange(rows * K))
    KB = K // 128
    loads = np.stack([src_row, src_col], 1).reshape(rows // 32, KB, 4, 64, 16, 2)
    for g in range(rows // 32):
        for kb in range(KB):
            for l in range(64):
                for h in range(2):
                    chunk = np.concatenate([loads[g, kb, 2 * h, l], loads[g, kb, 2 * h + 1, l]])
                    assert (chunk[:, 0] == 32 * g + l % 32).all()
                    start = 128 * kb + 64 * h + 32 * (l // 32)
                    assert np.array_equal(chunk[:, 1], np.arange(start, start + 32))
