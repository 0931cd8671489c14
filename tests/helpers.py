"""Shared test helpers: error metrics and device/host marshalling.  No method
arithmetic lives here."""
from __future__ import annotations

import sys

import numpy as np


def normwise_err(got, ref, axes=(-1,)) -> float:
    """max over vectors of ||got - ref||_inf / ||ref||_inf, vectors spanning
    ``axes``; an all-zero reference vector requires an exact zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(got - ref), axis=axes)
    den = np.max(np.abs(ref), axis=axes)
    zero = den == 0
    if np.any(zero & (num != 0)):
        return float("inf")
    return float(np.max(np.where(zero, 0.0, num / np.where(zero, 1.0, den)))) if num.size else 0.0


def matrix_err(got, ref) -> float:
    """Normwise error per (b, head) P x N matrix."""
    return normwise_err(got, ref, axes=(-2, -1))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(arrs, dev, in_dtype="f32"):
    """numpy float32 arrays (alpha, k, v, q) -> device tensors; k, v, q in the
    storage dtype (exact: bf16-representable values)."""
    import torch
    a, k, v, q = arrs
    tin = torch.bfloat16 if in_dtype == "bf16" else torch.float32
    return (torch.from_numpy(np.ascontiguousarray(a)).to(dev),
            torch.from_numpy(np.ascontiguousarray(k)).to(dev).to(tin),
            torch.from_numpy(np.ascontiguousarray(v)).to(dev).to(tin),
            torch.from_numpy(np.ascontiguousarray(q)).to(dev).to(tin))


def raw_bits(t) -> np.ndarray:
    """Bit pattern of a device tensor as a numpy array (uint16 for bf16)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def np_bits(x: np.ndarray, in_dtype: str) -> np.ndarray:
    """Bit pattern the device stores for host values of the input dtype."""
    if in_dtype == "bf16":
        x32 = np.ascontiguousarray(x, dtype=np.float32)
        return (x32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.ascontiguousarray(x, dtype=np.float32)


def unpack_e2m1(packed) -> np.ndarray:
    """MXFP4 copy bytes [..., N/2] -> one E2M1 code per entry [..., N]: entry n
    sits in byte n/2, low nibble first (the library's documented layout)."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out
