"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import numpy as np
import torch

DEV = "cuda:0"


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy bit-pattern array -> device tensor of the matching torch dtype."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(DEV)
    return torch.from_numpy(a).to(DEV)


BF16_NAN = 0x7FC0


def poisoned_bf16(*shape) -> torch.Tensor:
    """A bf16 output buffer filled with NaN, so that any element a kernel fails to
    write fails the tolerance check (the caching allocator would otherwise hand
    back a previous call's correct output)."""
    return torch.full(shape, BF16_NAN, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_tolerance_check(c_bits: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    """|C_gpu - ref| <= 1e-2 |ref| + 1e-2 rms(ref), element by element."""
    c = bf16_to_f64(c_bits)
    assert c.shape == ref.shape
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bound = 1e-2 * np.abs(ref) + 1e-2 * rms
    err = np.abs(c - ref)
    bad = ~(err <= bound)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d/%d outside tolerance; first %s: gpu %s ref %s" % (
            what, int(bad.sum()), bad.size, idx.tolist(), [c[tuple(i)] for i in idx], [ref[tuple(i)] for i in idx]))
    return {"max_err_over_bound": float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0,
            "rms": rms}


def sync():
    torch.cuda.synchronize()
