"""Python binding of the MI355X block-scaled FP8 library (libfp8bs.so).

A thin ctypes layer: it checks tensor dtypes, devices and layouts, allocates
outputs with torch when the caller does not pass them, and forwards raw device
pointers and the current HIP stream to the C ABI declared in include/fp8bs.h.
Every step of the computation runs in the library's gfx950 kernels; there is no
fallback path.  If libfp8bs.so is missing the import fails.

Bit-pattern conventions: bf16 tensors are torch.bfloat16 (or int16/uint16
views of them), e4m3 tensors are torch.uint8 (or torch.float8_e4m3fn), packed
scale words are torch.int32 holding uint32 bits, weight block scales are
torch.float32, and masked counts are torch.int32.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

__all__ = [
    "Fp8bsError", "fp8_quant_group_pack", "silu_mul_quant_group_pack", "fp8_block_quant_128x128",
    "fp8_block_gemm_nt", "fp8_block_gemm_grouped_masked", "gemm_config", "gemm_config_count",
    "library_path", "header_path", "declared_functions", "gemm_config_of",
    "fp8_quant_group_pack_to_experts", "fp8_block_gemm_grouped_contiguous",
    "fp8_quant_group_float", "fp8_block_quant_128x128_float", "fp8_block_gemm_nt_float_scales",
    "fp8_weight_preshuffle", "fp8_block_gemm_nt_preshuffled", "fp8_block_gemm_grouped_masked_preshuffled",
    "fp8_block_gemm_nt_preshuffled_noalloc", "check_dense_shapes", "check_masked_shapes", "check_contiguous_shapes",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfp8bs.so")
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "fp8bs.h")

if not os.path.exists(_LIB_PATH):
    raise ImportError("libfp8bs.so is not built; run `python block_scaled_fp8_token_amd/build.py` "
                      "(or __graft_entry__.build())")

_lib = ctypes.CDLL(_LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_I32P = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "fp8_quant_group_pack": [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P],
    "silu_mul_quant_group_pack": [_P, _P, _I64, _I64, _I64, _P, _P, _P],
    "fp8_block_quant_128x128": [_P, _I64, _I64, _P, _P, _P],
    "fp8_quant_group_pack_to_experts": [_P, _I64, _I64, _I64, _P, _I32, _I64, _I64, _P, _P, _P, _P, _P],
    "fp8_quant_group_float": [_P, _I64, _I64, _I64, _P, _I64, _P, _I64, _P],
    "fp8_block_quant_128x128_float": [_P, _I64, _I64, _P, _P, _P],
    "fp8_block_gemm_nt_float_scales": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _P],
    "fp8_block_gemm_nt_float_scales_cfg": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _P],
    "fp8_block_gemm_nt": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _P],
    "fp8_block_gemm_nt_cfg": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _P],
    "fp8_weight_preshuffle": [_P, _I64, _I64, _P, _P],
    "fp8_block_gemm_nt_preshuffled": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _P],
    "fp8_block_gemm_nt_preshuffled_cfg": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _I32, _P],
    "fp8_block_gemm_nt_preshuffled_noalloc": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _P],
    "fp8_block_gemm_grouped_masked_preshuffled": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P],
    "fp8_block_gemm_grouped_masked_preshuffled_cfg": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P],
    "fp8_block_gemm_nt_float_scales_preshuffled": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _P],
    "fp8_block_gemm_nt_float_scales_preshuffled_cfg": [_P, _P, _I64, _P, _P, _P, _I64, _I64, _I64, _I64, _I32,
                                                       _I32, _P],
    "fp8_block_gemm_grouped_masked": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P],
    "fp8_block_gemm_grouped_masked_cfg": [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I32, _P],
    "fp8_block_gemm_grouped_contiguous": [_P, _P, _I64, _P, _P, _P, _I64, _P, _I64, _I64, _I64, _I64, _P],
    "fp8_block_gemm_grouped_contiguous_cfg": [_P, _P, _I64, _P, _P, _P, _I64, _P, _I64, _I64, _I64, _I64, _I32,
                                              _P],
    "fp8bs_gemm_config_count": [],
    "fp8bs_gemm_config": [ctypes.c_int, _I64, _I64, _I64, _I32P, _I32P, _I32P, _I32P],
    "fp8bs_gemm_config_of": [_I32, ctypes.c_int, _I64, _I64, _I64, _I32, _I32P, _I32P, _I32P],
    "fp8bs_status_string": [ctypes.c_int],
    "fp8bs_last_hip_error": [],
}
for _name, _args in _SIGS.items():
    try:
        _fn = getattr(_lib, _name)
    except AttributeError:
        raise ImportError("libfp8bs.so does not export %s: it is older than the sources; rebuild with "
                          "`python block_scaled_fp8_token_amd/build.py`" % _name) from None
    _fn.argtypes = _args
    _fn.restype = ctypes.c_char_p if _name == "fp8bs_status_string" else ctypes.c_int


class Fp8bsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = _lib.fp8bs_status_string(status).decode()
        if status == -5:
            msg += " (hipError %d)" % _lib.fp8bs_last_hip_error()
        super().__init__("%s: %s [status %d]" % (fn, msg, status))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def header_path() -> str:
    return _HEADER


def declared_functions() -> list[str]:
    """Names of the functions include/fp8bs.h declares."""
    text = open(_HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Fp8bsError(fn, status)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_E4M3 = (torch.uint8, torch.float8_e4m3fn, torch.int8)


def _expect(t: torch.Tensor, name: str, dtypes, ndim: int) -> None:
    _dev(t, name)
    if t.dtype not in dtypes:
        raise TypeError("%s: dtype %s not in %s" % (name, t.dtype, dtypes))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got %d" % (name, ndim, t.dim()))
    if t.stride(-1) != 1:
        raise ValueError("%s must have unit stride in its last dim" % name)


def _contig(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


# Shape rules of the C ABI (include/fp8bs.h), checked on shapes and strides only so
# that a wrong tensor raises ValueError before any kernel could read or write past it.

def _words(K: int) -> int:
    return (K // 128 + 3) // 4


def _need_shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be %s, got %s" % (name, list(shape), list(t.shape)))


def _need_cols(t: torch.Tensor, name: str, rows: int, cols: int) -> None:
    """2-D [rows, >= cols] with unit column stride and a row stride of at least cols."""
    if t.dim() != 2 or t.shape[0] != rows or t.shape[1] < cols or t.stride(1) != 1 or t.stride(0) < cols:
        raise ValueError("%s must be [%d, >= %d] with row stride >= %d, got shape %s strides %s"
                         % (name, rows, cols, cols, list(t.shape), list(t.stride())))


def check_dense_shapes(a, sfa, b, sfb, c, float_scales: bool = False) -> None:
    """a [M, K], b [N, K], c [M, >= N] (row stride >= N), sfb [ceil(N/128), K/128], and
    sfa [ceil(K/512), >= M] (packed UE8M0 words) or [K/128, >= M] (float scales)."""
    if a.dim() != 2 or b.dim() != 2 or c.dim() != 2:
        raise ValueError("a, b and c must have 2 dims")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    _need_cols(c, "c", M, N)
    _need_cols(sfa, "sfa", K // 128 if float_scales else _words(K), M)
    _need_shape(sfb, "sfb", ((N + 127) // 128, K // 128))


def check_masked_shapes(a, sfa, b, sfb, c, masked_m) -> None:
    """a [E, M_max, K], sfa [E, ceil(K/512), M_max], b [E, N, K], sfb [E, ceil(N/128), K/128],
    c [E, M_max, N], masked_m [E]."""
    if a.dim() != 3 or b.dim() != 3:
        raise ValueError("a and b must have 3 dims")
    E, M_max, K = a.shape
    N = b.shape[1]
    _need_shape(b, "b", (E, N, K))
    _need_shape(sfa, "sfa", (E, _words(K), M_max))
    _need_shape(sfb, "sfb", (E, (N + 127) // 128, K // 128))
    _need_shape(c, "c", (E, M_max, N))
    _need_shape(masked_m, "masked_m", (E,))


def check_contiguous_shapes(a, sfa, b, sfb, c, m_indices) -> None:
    """a [M, K], sfa [ceil(K/512), >= M], b [E, N, K], sfb [E, ceil(N/128), K/128],
    c [M, >= N], m_indices [M]."""
    if a.dim() != 2 or b.dim() != 3:
        raise ValueError("a must have 2 dims and b 3")
    M, K = a.shape
    E, N = b.shape[0], b.shape[1]
    if b.shape[2] != K:
        raise ValueError("a and b disagree on K")
    _need_cols(sfa, "sfa", _words(K), M)
    _need_shape(sfb, "sfb", (E, (N + 127) // 128, K // 128))
    _need_cols(c, "c", M, N)
    _need_shape(m_indices, "m_indices", (M,))


# ----------------------------------------------------------------------------

def fp8_quant_group_pack(x: torch.Tensor, q: torch.Tensor | None = None, sf: torch.Tensor | None = None,
                         ld_sf: int | None = None, stream=None):
    """1x128 per-token group quant + UE8M0 pack.  x bf16 [M, K] -> (q uint8 [M, K],
    sf int32 [ceil(K/512), ld_sf]); ld_sf defaults to round_up(M, 4)."""
    _expect(x, "x", _BF16, 2)
    M, K = x.shape
    W = (K // 128 + 3) // 4
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if sf is None:
        ld = ld_sf if ld_sf is not None else max(4, (M + 3) // 4 * 4)
        sf = torch.empty((W, ld), dtype=torch.int32, device=x.device)
    _expect(q, "q", _E4M3, 2)
    _expect(sf, "sf", (torch.int32, torch.uint32), 2)
    _need_cols(q, "q", M, K)
    _need_cols(sf, "sf", W, M)
    st = _lib.fp8_quant_group_pack(x.data_ptr(), x.stride(0), M, K, q.data_ptr(), q.stride(0),
                                   sf.data_ptr(), sf.stride(0), _stream(stream))
    _check("fp8_quant_group_pack", st)
    return q, sf


def silu_mul_quant_group_pack(x: torch.Tensor, masked_m: torch.Tensor, q: torch.Tensor | None = None,
                              sf: torch.Tensor | None = None, stream=None):
    """Fused SiLU-mul + quant/pack over a masked batch.  x bf16 [E, M_max, 2H], masked_m int32 [E]
    -> (q uint8 [E, M_max, H], sf int32 [E, ceil(H/512), M_max]); padded rows are not written."""
    _expect(x, "x", _BF16, 3)
    _contig(x, "x")
    E, M_max, H2 = x.shape
    if H2 % 2:
        raise ValueError("last dim of x must be 2H")
    H = H2 // 2
    W = (H // 128 + 3) // 4
    _expect(masked_m, "masked_m", (torch.int32,), 1)
    if masked_m.shape[0] != E:
        raise ValueError("masked_m must have E entries")
    if q is None:
        q = torch.empty((E, M_max, H), dtype=torch.uint8, device=x.device)
    if sf is None:
        sf = torch.empty((E, W, M_max), dtype=torch.int32, device=x.device)
    _expect(q, "q", _E4M3, 3)
    _contig(q, "q")
    _expect(sf, "sf", (torch.int32, torch.uint32), 3)
    _contig(sf, "sf")
    if tuple(q.shape) != (E, M_max, H) or tuple(sf.shape) != (E, W, M_max):
        raise ValueError("output shapes do not match x")
    st = _lib.silu_mul_quant_group_pack(x.data_ptr(), masked_m.data_ptr(), E, M_max, H, q.data_ptr(),
                                        sf.data_ptr(), _stream(stream))
    _check("silu_mul_quant_group_pack", st)
    return q, sf


def fp8_block_quant_128x128(w: torch.Tensor, q: torch.Tensor | None = None, sfb: torch.Tensor | None = None,
                            stream=None):
    """128x128 weight block quant.  w bf16 [N, K] -> (q uint8 [N, K], sfb float32 [ceil(N/128), K/128])."""
    _expect(w, "w", _BF16, 2)
    _contig(w, "w")
    N, K = w.shape
    if q is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    if sfb is None:
        sfb = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=w.device)
    _expect(q, "q", _E4M3, 2)
    _contig(q, "q")
    _expect(sfb, "sfb", (torch.float32,), 2)
    _contig(sfb, "sfb")
    _need_shape(q, "q", (N, K))
    _need_shape(sfb, "sfb", ((N + 127) // 128, K // 128))
    st = _lib.fp8_block_quant_128x128(w.data_ptr(), N, K, q.data_ptr(), sfb.data_ptr(), _stream(stream))
    _check("fp8_block_quant_128x128", st)
    return q, sfb


def fp8_quant_group_pack_to_experts(x: torch.Tensor, topk_ids: torch.Tensor, E: int, M_max: int,
                                    q: torch.Tensor | None = None, sf: torch.Tensor | None = None,
                                    masked_m: torch.Tensor | None = None, slot_of: torch.Tensor | None = None,
                                    stream=None):
    """Per-token group quant into the masked expert layout of the routed tokens.
    x bf16 [T, K], topk_ids int32 [T, topk] -> (q uint8 [E, M_max, K],
    sf int32 [E, ceil(K/512), M_max], masked_m int32 [E], slot_of int32 [T, topk])."""
    _expect(x, "x", _BF16, 2)
    _expect(topk_ids, "topk_ids", (torch.int32,), 2)
    _contig(topk_ids, "topk_ids")
    T, K = x.shape
    topk = topk_ids.shape[1]
    if topk_ids.shape[0] != T:
        raise ValueError("topk_ids must be [T, topk]")
    Wd = (K // 128 + 3) // 4
    dev = x.device
    if q is None:
        q = torch.empty((E, M_max, K), dtype=torch.uint8, device=dev)
    if sf is None:
        sf = torch.empty((E, Wd, M_max), dtype=torch.int32, device=dev)
    if masked_m is None:
        masked_m = torch.empty((E,), dtype=torch.int32, device=dev)
    if slot_of is None:
        slot_of = torch.empty((T, topk), dtype=torch.int32, device=dev)
    _expect(q, "q", _E4M3, 3)
    _contig(q, "q")
    _expect(sf, "sf", (torch.int32, torch.uint32), 3)
    _contig(sf, "sf")
    _expect(masked_m, "masked_m", (torch.int32,), 1)
    _expect(slot_of, "slot_of", (torch.int32,), 2)
    _contig(slot_of, "slot_of")
    if tuple(q.shape) != (E, M_max, K) or tuple(sf.shape) != (E, Wd, M_max) or tuple(slot_of.shape) != (T, topk):
        raise ValueError("output shapes do not match E, M_max, K, T, topk")
    _need_shape(masked_m, "masked_m", (E,))
    st = _lib.fp8_quant_group_pack_to_experts(x.data_ptr(), x.stride(0), T, K, topk_ids.data_ptr(), topk, E, M_max,
                                              q.data_ptr(), sf.data_ptr(), masked_m.data_ptr(), slot_of.data_ptr(),
                                              _stream(stream))
    _check("fp8_quant_group_pack_to_experts", st)
    return q, sf, masked_m, slot_of


def fp8_block_gemm_nt(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                      c: torch.Tensor | None = None, kernel: int | None = None, splits: int | None = None,
                      stream=None) -> torch.Tensor:
    """Dense block-scaled C = A . B^T -> bf16 [M, N].  a uint8 [M, K], sfa int32 [ceil(K/512), ld_sfa],
    b uint8 [N, K], sfb float32 [ceil(N/128), K/128].  kernel/splits force a tile-table entry."""
    _expect(a, "a", _E4M3, 2)
    _contig(a, "a")
    _expect(b, "b", _E4M3, 2)
    _contig(b, "b")
    _expect(sfa, "sfa", (torch.int32, torch.uint32), 2)
    _expect(sfb, "sfb", (torch.float32,), 2)
    _contig(sfb, "sfb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _expect(c, "c", _BF16, 2)
    if tuple(c.shape) != (M, N):
        raise ValueError("c must be [M, N]")
    check_dense_shapes(a, sfa, b, sfb, c)
    s = _stream(stream)
    if kernel is None and splits is None:
        st = _lib.fp8_block_gemm_nt(a.data_ptr(), sfa.data_ptr(), sfa.stride(0), b.data_ptr(), sfb.data_ptr(),
                                    c.data_ptr(), c.stride(0), M, N, K, s)
    else:
        if kernel is None:
            kernel = gemm_config(False, M, N, K)["kernel"]
        st = _lib.fp8_block_gemm_nt_cfg(a.data_ptr(), sfa.data_ptr(), sfa.stride(0), b.data_ptr(),
                                        sfb.data_ptr(), c.data_ptr(), c.stride(0), M, N, K, int(kernel),
                                        int(splits or 1), s)
    _check("fp8_block_gemm_nt", st)
    return c


def fp8_weight_preshuffle(w: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """e4m3 weights [..., rows, K] (rows over all leading dims a multiple of 32) -> the same
    bytes in the pre-shuffled layout of fp8_block_gemm_nt_preshuffled, same shape."""
    _expect(w, "w", _E4M3, w.dim())
    _contig(w, "w")
    if w.dim() < 2:
        raise ValueError("w must be [..., rows, K]")
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    if out is None:
        out = torch.empty_like(w)
    _expect(out, "out", _E4M3, w.dim())
    _contig(out, "out")
    if tuple(out.shape) != tuple(w.shape):
        raise ValueError("out must have the shape of w")
    _check("fp8_weight_preshuffle", _lib.fp8_weight_preshuffle(w.data_ptr(), rows, K, out.data_ptr(), _stream(stream)))
    return out


def fp8_block_gemm_nt_preshuffled(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                  c: torch.Tensor | None = None, kernel: int | None = None,
                                  splits: int | None = None, stream=None) -> torch.Tensor:
    """fp8_block_gemm_nt with b [N, K] in the pre-shuffled layout (fp8_weight_preshuffle)."""
    _expect(a, "a", _E4M3, 2)
    _contig(a, "a")
    _expect(b, "b", _E4M3, 2)
    _contig(b, "b")
    _expect(sfa, "sfa", (torch.int32, torch.uint32), 2)
    _expect(sfb, "sfb", (torch.float32,), 2)
    _contig(sfb, "sfb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _expect(c, "c", _BF16, 2)
    if tuple(c.shape) != (M, N):
        raise ValueError("c must be [M, N]")
    check_dense_shapes(a, sfa, b, sfb, c)
    s = _stream(stream)
    args = (a.data_ptr(), sfa.data_ptr(), sfa.stride(0), b.data_ptr(), sfb.data_ptr(), c.data_ptr(), c.stride(0),
            M, N, K)
    if kernel is None and splits is None:
        st = _lib.fp8_block_gemm_nt_preshuffled(*args, s)
    else:
        if kernel is None:
            kernel = gemm_config(LAYOUT_DENSE_PRESHUFFLED, M, N, K)["kernel"]
        st = _lib.fp8_block_gemm_nt_preshuffled_cfg(*args, int(kernel), int(splits or 1), s)
    _check("fp8_block_gemm_nt_preshuffled", st)
    return c


def fp8_block_gemm_nt_preshuffled_noalloc(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                          c: torch.Tensor, stream=None) -> torch.Tensor:
    """fp8_block_gemm_nt_preshuffled into a caller-allocated c, with the split-K scratch in the
    library's static device buffer: the call allocates nothing (for graph capture and serving
    loops).  Calls that overlap on one GPU share that buffer and race."""
    _expect(a, "a", _E4M3, 2)
    _contig(a, "a")
    _expect(b, "b", _E4M3, 2)
    _contig(b, "b")
    _expect(sfa, "sfa", (torch.int32, torch.uint32), 2)
    _expect(sfb, "sfb", (torch.float32,), 2)
    _contig(sfb, "sfb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    _expect(c, "c", _BF16, 2)
    if tuple(c.shape) != (M, N):
        raise ValueError("c must be [M, N]")
    check_dense_shapes(a, sfa, b, sfb, c)
    st = _lib.fp8_block_gemm_nt_preshuffled_noalloc(a.data_ptr(), sfa.data_ptr(), sfa.stride(0), b.data_ptr(),
                                                    sfb.data_ptr(), c.data_ptr(), c.stride(0), M, N, K,
                                                    _stream(stream))
    _check("fp8_block_gemm_nt_preshuffled_noalloc", st)
    return c


def fp8_block_gemm_grouped_masked(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                  masked_m: torch.Tensor, c: torch.Tensor | None = None,
                                  kernel: int | None = None, stream=None, preshuffled: bool = False) -> torch.Tensor:
    """Masked grouped GEMM -> bf16 [E, M_max, N].  a uint8 [E, M_max, K], sfa int32 [E, ceil(K/512), M_max],
    b uint8 [E, N, K], sfb float32 [E, ceil(N/128), K/128], masked_m int32 [E].  preshuffled: b is in the
    layout of fp8_weight_preshuffle (fp8_block_gemm_grouped_masked_preshuffled)."""
    for t, n in ((a, "a"), (b, "b")):
        _expect(t, n, _E4M3, 3)
        _contig(t, n)
    _expect(sfa, "sfa", (torch.int32, torch.uint32), 3)
    _contig(sfa, "sfa")
    _expect(sfb, "sfb", (torch.float32,), 3)
    _contig(sfb, "sfb")
    _expect(masked_m, "masked_m", (torch.int32,), 1)
    E, M_max, K = a.shape
    N = b.shape[1]
    if b.shape[0] != E or b.shape[2] != K or masked_m.shape[0] != E:
        raise ValueError("inconsistent expert shapes")
    if c is None:
        c = torch.empty((E, M_max, N), dtype=torch.bfloat16, device=a.device)
    _expect(c, "c", _BF16, 3)
    _contig(c, "c")
    check_masked_shapes(a, sfa, b, sfb, c, masked_m)
    s = _stream(stream)
    name = "fp8_block_gemm_grouped_masked" + ("_preshuffled" if preshuffled else "")
    args = (a.data_ptr(), sfa.data_ptr(), b.data_ptr(), sfb.data_ptr(), c.data_ptr(), masked_m.data_ptr(),
            E, M_max, N, K)
    if kernel is None:
        st = getattr(_lib, name)(*args, s)
    else:
        st = getattr(_lib, name + "_cfg")(*args, int(kernel), s)
    _check(name, st)
    return c


def fp8_block_gemm_grouped_masked_preshuffled(a, sfa, b, sfb, masked_m, c=None, kernel=None, stream=None):
    """fp8_block_gemm_grouped_masked with b [E, N, K] in the pre-shuffled layout."""
    return fp8_block_gemm_grouped_masked(a, sfa, b, sfb, masked_m, c=c, kernel=kernel, stream=stream,
                                         preshuffled=True)


def fp8_block_gemm_grouped_contiguous(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                      m_indices: torch.Tensor, c: torch.Tensor | None = None,
                                      kernel: int | None = None, stream=None) -> torch.Tensor:
    """Contiguous grouped GEMM -> bf16 [M, N].  a uint8 [M, K] (rows grouped by expert in runs
    aligned to 128 rows), sfa int32 [ceil(K/512), ld_sfa], b uint8 [E, N, K],
    sfb float32 [E, ceil(N/128), K/128], m_indices int32 [M] (-1: padding row)."""
    _expect(a, "a", _E4M3, 2)
    _contig(a, "a")
    _expect(b, "b", _E4M3, 3)
    _contig(b, "b")
    _expect(sfa, "sfa", (torch.int32, torch.uint32), 2)
    _expect(sfb, "sfb", (torch.float32,), 3)
    _contig(sfb, "sfb")
    _expect(m_indices, "m_indices", (torch.int32,), 1)
    _contig(m_indices, "m_indices")
    M, K = a.shape
    E, N = b.shape[0], b.shape[1]
    if b.shape[2] != K or sfb.shape[0] != E or m_indices.shape[0] != M:
        raise ValueError("inconsistent shapes")
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _expect(c, "c", _BF16, 2)
    if tuple(c.shape) != (M, N):
        raise ValueError("c must be [M, N]")
    check_contiguous_shapes(a, sfa, b, sfb, c, m_indices)
    s = _stream(stream)
    args = (a.data_ptr(), sfa.data_ptr(), sfa.stride(0), b.data_ptr(), sfb.data_ptr(), c.data_ptr(), c.stride(0),
            m_indices.data_ptr(), E, M, N, K)
    if kernel is None:
        st = _lib.fp8_block_gemm_grouped_contiguous(*args, s)
    else:
        st = _lib.fp8_block_gemm_grouped_contiguous_cfg(*args, int(kernel), s)
    _check("fp8_block_gemm_grouped_contiguous", st)
    return c


(LAYOUT_DENSE, LAYOUT_MASKED, LAYOUT_CONTIGUOUS, LAYOUT_DENSE_FLOAT, LAYOUT_DENSE_PRESHUFFLED,
 LAYOUT_MASKED_PRESHUFFLED, LAYOUT_DENSE_FLOAT_PRESHUFFLED) = 0, 1, 2, 3, 4, 5, 6


def fp8_quant_group_float(x: torch.Tensor, q: torch.Tensor | None = None, sf: torch.Tensor | None = None,
                          ld_sf: int | None = None, stream=None):
    """1x128 per-token group quant with float scales (amax / 448, unrounded).
    x bf16 [M, K] -> (q uint8 [M, K], sf float32 [K/128, ld_sf]); ld_sf defaults to round_up(M, 4)."""
    _expect(x, "x", _BF16, 2)
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if sf is None:
        ld = ld_sf if ld_sf is not None else max(4, (M + 3) // 4 * 4)
        sf = torch.empty((K // 128, ld), dtype=torch.float32, device=x.device)
    _expect(q, "q", _E4M3, 2)
    _expect(sf, "sf", (torch.float32,), 2)
    _need_cols(q, "q", M, K)
    _need_cols(sf, "sf", K // 128, M)
    st = _lib.fp8_quant_group_float(x.data_ptr(), x.stride(0), M, K, q.data_ptr(), q.stride(0), sf.data_ptr(),
                                    sf.stride(0), _stream(stream))
    _check("fp8_quant_group_float", st)
    return q, sf


def fp8_block_quant_128x128_float(w: torch.Tensor, stream=None):
    """128x128 weight block quant with float scales: bf16 w [N, K] -> (q uint8 [N, K],
    sfb float32 [ceil(N/128), K/128])."""
    _expect(w, "w", _BF16, 2)
    _contig(w, "w")
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    sfb = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=w.device)
    st = _lib.fp8_block_quant_128x128_float(w.data_ptr(), N, K, q.data_ptr(), sfb.data_ptr(), _stream(stream))
    _check("fp8_block_quant_128x128_float", st)
    return q, sfb


def fp8_block_gemm_nt_float_scales(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                   c: torch.Tensor | None = None, kernel: int | None = None,
                                   splits: int | None = None, stream=None, preshuffled: bool = False) -> torch.Tensor:
    """Dense GEMM with float scales -> bf16 [M, N].  a uint8 [M, K], sfa float32 [K/128, ld_sfa],
    b uint8 [N, K], sfb float32 [ceil(N/128), K/128].  preshuffled: b is in the layout of
    fp8_weight_preshuffle (fp8_block_gemm_nt_float_scales_preshuffled)."""
    _expect(a, "a", _E4M3, 2)
    _contig(a, "a")
    _expect(b, "b", _E4M3, 2)
    _contig(b, "b")
    _expect(sfa, "sfa", (torch.float32,), 2)
    _expect(sfb, "sfb", (torch.float32,), 2)
    _contig(sfb, "sfb")
    M, K = a.shape
    N = b.shape[0]
    if b.shape[1] != K:
        raise ValueError("a and b disagree on K")
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _expect(c, "c", _BF16, 2)
    if tuple(c.shape) != (M, N):
        raise ValueError("c must be [M, N]")
    check_dense_shapes(a, sfa, b, sfb, c, float_scales=True)
    s = _stream(stream)
    args = (a.data_ptr(), sfa.data_ptr(), sfa.stride(0), b.data_ptr(), sfb.data_ptr(), c.data_ptr(), c.stride(0),
            M, N, K)
    name = "fp8_block_gemm_nt_float_scales" + ("_preshuffled" if preshuffled else "")
    if kernel is None and splits is None:
        st = getattr(_lib, name)(*args, s)
    else:
        if kernel is None:
            kernel = gemm_config(LAYOUT_DENSE_FLOAT_PRESHUFFLED if preshuffled else LAYOUT_DENSE_FLOAT, M, N, K)["kernel"]
        st = getattr(_lib, name + "_cfg")(*args, int(kernel), int(splits or 1), s)
    _check(name, st)
    return c


def gemm_config_count() -> int:
    return int(_lib.fp8bs_gemm_config_count())


def gemm_config_of(kernel: int, masked, M: int, N: int, K: int, splits: int = 1):
    """Workgroup tile and split count table entry `kernel` would use for this
    problem, or None if the entry does not accept it.  masked: False/0 dense,
    True/1 masked grouped, 2 contiguous grouped, 3 dense with float scales, 4 dense
    with pre-shuffled weights."""
    bm, bn, sp = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = _lib.fp8bs_gemm_config_of(int(kernel), int(masked), M, N, K, int(splits), ctypes.byref(bm),
                                   ctypes.byref(bn), ctypes.byref(sp))
    if st == -2:
        return None
    _check("fp8bs_gemm_config_of", st)
    return {"kernel": int(kernel), "bm": bm.value, "bn": bn.value, "splits": sp.value}


def gemm_config(masked, M: int, N: int, K: int) -> dict:
    """Automatic choice for a dense (False/0), masked (True/1), contiguous grouped (2),
    dense float-scale (3) or dense pre-shuffled-weight (4) problem."""
    k, bm, bn, sp = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    st = _lib.fp8bs_gemm_config(int(masked), M, N, K, ctypes.byref(k), ctypes.byref(bm),
                                ctypes.byref(bn), ctypes.byref(sp))
    _check("fp8bs_gemm_config", st)
    return {"kernel": k.value, "bm": bm.value, "bn": bn.value, "splits": sp.value}
