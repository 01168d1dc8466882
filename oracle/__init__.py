"""CPU oracle for block-scaled FP8 (e4m3) W8A8 GEMM: numpy front-end to oracle.c.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import this package.  The product path
(the HIP library and its Python binding) never imports, links or calls it, and
it imports nothing from the product path.

All arrays are host numpy arrays holding raw bit patterns: bf16 as uint16,
e4m3 as uint8, packed UE8M0 scales as uint32, weight block scales as float32.
Results of the GEMMs are float64 (the exact block-scaled value, rounded once).
The definitions each function follows are cited in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a prebuilt copy to load instead (the sanitizer test builds one with -fsanitize)
_LIB_OVERRIDE = os.environ.get("FP8BS_ORACLE_LIB")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (OpenMP over output rows only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer into `path`
    (load it with FP8BS_ORACLE_LIB=path in a process that preloads libasan)."""
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           _SRC, "-o", path, "-lm"]
    subprocess.run(cmd, check=True)
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int64
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_ue8m0_exponent.argtypes = [ctypes.c_double]
    lib.orc_ue8m0_exponent.restype = ctypes.c_int
    lib.orc_bf16_rne.argtypes = [ctypes.c_double]
    lib.orc_bf16_rne.restype = ctypes.c_uint16
    lib.orc_quant_group_pack.argtypes = [P, I, I, I, P, I, P, I]
    lib.orc_quant_group_pack.restype = None
    lib.orc_silu_mul_quant_group_pack.argtypes = [P, P, I, I, I, P, P, P]
    lib.orc_silu_mul_quant_group_pack.restype = None
    lib.orc_quant_group_pack_to_experts.argtypes = [P, I, I, I, P, I, I, I, P, P, P, P]
    lib.orc_quant_group_pack_to_experts.restype = None
    lib.orc_quant_group_float.argtypes = [P, I, I, I, P, I, P, I]
    lib.orc_quant_group_float.restype = None
    lib.orc_block_quant_128x128_float.argtypes = [P, I, I, P, P]
    lib.orc_block_quant_128x128_float.restype = None
    lib.orc_gemm_nt_float_scales.argtypes = [P, I, P, I, P, I, P, I, I, I, P, I, P, I, P]
    lib.orc_gemm_nt_float_scales.restype = None
    lib.orc_block_quant_128x128.argtypes = [P, I, I, P, P]
    lib.orc_block_quant_128x128.restype = None
    lib.orc_gemm_nt.argtypes = [P, I, P, I, P, I, P, I, I, I, P, I, P, I, P]
    lib.orc_gemm_nt.restype = None
    lib.orc_gemm_grouped_masked.argtypes = [P, P, P, P, P, I, I, I, I, P, I, P]
    lib.orc_gemm_grouped_masked.restype = None
    lib.orc_gemm_grouped_contiguous.argtypes = [P, P, I, P, P, P, I, I, I, I, P, I, P]
    lib.orc_gemm_grouped_contiguous.restype = None
    lib.orc_weight_preshuffle.argtypes = [P, I, I, P]
    lib.orc_weight_preshuffle.restype = None
    lib.orc_calc_diff.argtypes = [P, P, I]
    lib.orc_calc_diff.restype = ctypes.c_double
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_set_num_threads.argtypes = [ctypes.c_int]
    lib.orc_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _req(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s array, got %s" % (np.dtype(dtype), a.dtype))
    return a


# --------------------------------------------------------------------------
# scalar pieces

def e4m3_decode(b: int) -> float:
    return _load().orc_e4m3_decode(int(b) & 0xFF)


def e4m3_encode(v: float) -> int:
    return int(_load().orc_e4m3_encode(float(v)))


def e4m3_table() -> np.ndarray:
    """float64[256]: the decoded value of every e4m3 byte (NaN for 0x7F / 0xFF)."""
    lib = _load()
    return np.array([lib.orc_e4m3_decode(b) for b in range(256)], dtype=np.float64)


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.asarray(v, dtype=np.float64).ravel()
    return np.array([lib.orc_e4m3_encode(float(x)) for x in flat], dtype=np.uint8).reshape(np.shape(v))


def ue8m0_exponent(amax: float) -> int:
    return int(_load().orc_ue8m0_exponent(float(amax)))


def bf16_rne(v: float) -> int:
    return int(_load().orc_bf16_rne(float(v)))


def bf16_rne_array(v: np.ndarray) -> np.ndarray:
    lib = _load()
    flat = np.asarray(v, dtype=np.float64).ravel()
    return np.array([lib.orc_bf16_rne(float(x)) for x in flat], dtype=np.uint16).reshape(np.shape(v))


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops (for timing; the results do not depend on it)."""
    _load().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------
# the hot-path steps

def quant_group_pack(x: np.ndarray, ld_sf: int | None = None):
    """1x128 per-token-group quant + UE8M0 pack of bf16 x [M, K] (uint16 bits).

    Returns (q uint8 [M, K], sf uint32 [W, ld_sf]).  Entries sf[:, M:] are zero
    here and are not part of the result."""
    x = _req(x, np.uint16)
    M, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    W = (K // 128 + 3) // 4
    if ld_sf is None:
        ld_sf = max(4, (M + 3) // 4 * 4)
    q = np.zeros((M, K), np.uint8)
    sf = np.zeros((W, ld_sf), np.uint32)
    _load().orc_quant_group_pack(_ptr(x), K, M, K, _ptr(q), K, _ptr(sf), ld_sf)
    return q, sf


def silu_mul_quant_group_pack(x: np.ndarray, masked_m: np.ndarray, want_y: bool = False):
    """Fused SiLU-mul + quant/pack of bf16 x [E, M_max, 2H] over rows r < masked_m[e].

    Returns (q uint8 [E, M_max, H], sf uint32 [E, W, M_max][, y float64 [E, M_max, H]]).
    Rows at or past the count are left zero (NaN in y) and are not part of the result."""
    x = _req(x, np.uint16)
    mm = _req(masked_m, np.int32)
    E, M_max, H2 = x.shape
    H = H2 // 2
    if H2 % 2 or H % 128:
        raise ValueError("last dim must be 2H with H a multiple of 128")
    W = (H // 128 + 3) // 4
    q = np.zeros((E, M_max, H), np.uint8)
    sf = np.zeros((E, W, M_max), np.uint32)
    y = np.full((E, M_max, H), np.nan) if want_y else None
    _load().orc_silu_mul_quant_group_pack(_ptr(x), _ptr(mm), E, M_max, H, _ptr(q), _ptr(sf), _ptr(y))
    return (q, sf, y) if want_y else (q, sf)


def quant_group_pack_to_experts(x: np.ndarray, topk_ids: np.ndarray, E: int, M_max: int):
    """Per-token group quant of bf16 x [T, K] into the masked expert layout of the
    routed tokens (topk_ids int32 [T, topk]).  Returns (q uint8 [E, M_max, K],
    sf uint32 [E, W, M_max], masked_m int32 [E], slot_of int32 [T, topk]); rows at
    or past masked_m[e] are zero here and are not part of the result."""
    x = _req(x, np.uint16)
    ids = _req(topk_ids, np.int32)
    T, K = x.shape
    topk = ids.shape[1]
    if K % 128 or ids.shape[0] != T:
        raise ValueError("bad shapes")
    W = (K // 128 + 3) // 4
    q = np.zeros((E, M_max, K), np.uint8)
    sf = np.zeros((E, W, M_max), np.uint32)
    mm = np.zeros(E, np.int32)
    slot = np.zeros((T, topk), np.int32)
    _load().orc_quant_group_pack_to_experts(_ptr(x), K, T, K, _ptr(ids), topk, E, M_max, _ptr(q), _ptr(sf),
                                            _ptr(mm), _ptr(slot))
    return q, sf, mm, slot


def block_quant_128x128(w: np.ndarray):
    """128x128 block quant of bf16 w [N, K] -> (q uint8 [N, K], sfb float32 [ceil(N/128), K/128])."""
    w = _req(w, np.uint16)
    N, K = w.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    q = np.zeros((N, K), np.uint8)
    sfb = np.zeros(((N + 127) // 128, K // 128), np.float32)
    _load().orc_block_quant_128x128(_ptr(w), N, K, _ptr(q), _ptr(sfb))
    return q, sfb


def weight_preshuffle(w: np.ndarray) -> np.ndarray:
    """e4m3 weights [rows, K] (uint8, rows % 32 == 0, K % 128 == 0) -> the same bytes in the
    pre-shuffled layout (a flat uint8 array of rows*K bytes, returned as [rows, K])."""
    w = _req(w, np.uint8)
    rows, K = w.shape
    if rows % 32 or K % 128:
        raise ValueError("rows must be a multiple of 32 and K of 128")
    out = np.zeros((rows, K), np.uint8)
    _load().orc_weight_preshuffle(_ptr(w), rows, K, _ptr(out))
    return out


def gemm_nt(qa, sfa, qb, sfb, rows=None, cols=None):
    """Block-scaled C = A . B^T in double for the selected rows/cols (all by default).

    qa uint8 [M, K], sfa uint32 [W, ld_sfa], qb uint8 [N, K], sfb float32 [ceil(N/128), K/128]."""
    qa = _req(qa, np.uint8)
    qb = _req(qb, np.uint8)
    sfa = _req(sfa, np.uint32)
    sfb = _req(sfb, np.float32)
    M, K = qa.shape
    N = qb.shape[0]
    r = None if rows is None else _req(np.asarray(rows, np.int64), np.int64)
    c = None if cols is None else _req(np.asarray(cols, np.int64), np.int64)
    nr = M if r is None else len(r)
    nc = N if c is None else len(c)
    out = np.zeros((nr, nc), np.float64)
    _load().orc_gemm_nt(_ptr(qa), K, _ptr(sfa), sfa.shape[1], _ptr(qb), K, _ptr(sfb), M, N, K,
                        _ptr(r), nr, _ptr(c), nc, _ptr(out))
    return out


def quant_group_float(x: np.ndarray, ld_sf: int | None = None):
    """1x128 per-token group quant with float scales (amax / 448 in fp32) of bf16 x [M, K].
    Returns (q uint8 [M, K], sf float32 [K/128, ld_sf]); sf[:, M:] is zero here."""
    x = _req(x, np.uint16)
    M, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    if ld_sf is None:
        ld_sf = max(4, (M + 3) // 4 * 4)
    q = np.zeros((M, K), np.uint8)
    sf = np.zeros((K // 128, ld_sf), np.float32)
    _load().orc_quant_group_float(_ptr(x), K, M, K, _ptr(q), K, _ptr(sf), ld_sf)
    return q, sf


def block_quant_128x128_float(w: np.ndarray):
    """128x128 block quant with float scales of bf16 w [N, K] -> (q uint8 [N, K],
    sfb float32 [ceil(N/128), K/128])."""
    w = _req(w, np.uint16)
    N, K = w.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    q = np.zeros((N, K), np.uint8)
    sfb = np.zeros(((N + 127) // 128, K // 128), np.float32)
    _load().orc_block_quant_128x128_float(_ptr(w), N, K, _ptr(q), _ptr(sfb))
    return q, sfb


def gemm_nt_float_scales(qa, sfa, qb, sfb, rows=None, cols=None):
    """Float-scale block GEMM C = A . B^T in double.  qa uint8 [M, K], sfa float32 [K/128, ld_sfa],
    qb uint8 [N, K], sfb float32 [ceil(N/128), K/128]."""
    qa = _req(qa, np.uint8)
    qb = _req(qb, np.uint8)
    sfa = _req(sfa, np.float32)
    sfb = _req(sfb, np.float32)
    M, K = qa.shape
    N = qb.shape[0]
    r = None if rows is None else _req(np.asarray(rows, np.int64), np.int64)
    c = None if cols is None else _req(np.asarray(cols, np.int64), np.int64)
    nr = M if r is None else len(r)
    nc = N if c is None else len(c)
    out = np.zeros((nr, nc), np.float64)
    _load().orc_gemm_nt_float_scales(_ptr(qa), K, _ptr(sfa), sfa.shape[1], _ptr(qb), K, _ptr(sfb), M, N, K,
                                     _ptr(r), nr, _ptr(c), nc, _ptr(out))
    return out


def gemm_grouped_masked(a, sfa, b, sfb, masked_m, rows=None):
    """Masked grouped GEMM in double.  a uint8 [E, M_max, K], sfa uint32 [E, W, M_max],
    b uint8 [E, N, K], sfb float32 [E, ceil(N/128), K/128], masked_m int32 [E].
    Returns double [E, M_max, N]; rows not computed are NaN."""
    a = _req(a, np.uint8)
    b = _req(b, np.uint8)
    sfa = _req(sfa, np.uint32)
    sfb = _req(sfb, np.float32)
    mm = _req(masked_m, np.int32)
    E, M_max, K = a.shape
    N = b.shape[1]
    r = None if rows is None else _req(np.asarray(rows, np.int64), np.int64)
    out = np.full((E, M_max, N), np.nan)
    _load().orc_gemm_grouped_masked(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(mm), E, M_max, N, K,
                                    _ptr(r), 0 if r is None else len(r), _ptr(out))
    return out


def gemm_grouped_contiguous(a, sfa, b, sfb, m_indices, rows=None):
    """Contiguous grouped GEMM in double.  a uint8 [M, K], sfa uint32 [W, ld_sfa],
    b uint8 [E, N, K], sfb float32 [E, ceil(N/128), K/128], m_indices int32 [M]
    (group of every row; values outside [0, E) are padding).
    Returns double [M, N]; rows not computed (padding, or not selected) are NaN."""
    a = _req(a, np.uint8)
    b = _req(b, np.uint8)
    sfa = _req(sfa, np.uint32)
    sfb = _req(sfb, np.float32)
    mi = _req(m_indices, np.int32)
    M, K = a.shape
    E, N = b.shape[0], b.shape[1]
    r = None if rows is None else _req(np.asarray(rows, np.int64), np.int64)
    out = np.full((M, N), np.nan)
    _load().orc_gemm_grouped_contiguous(_ptr(a), _ptr(sfa), sfa.shape[1], _ptr(b), _ptr(sfb), _ptr(mi), E, M, N,
                                        K, _ptr(r), 0 if r is None else len(r), _ptr(out))
    return out


def calc_diff(x, y) -> float:
    x = np.ascontiguousarray(x, dtype=np.float64).ravel()
    y = np.ascontiguousarray(y, dtype=np.float64).ravel()
    return float(_load().orc_calc_diff(_ptr(x), _ptr(y), x.size))
