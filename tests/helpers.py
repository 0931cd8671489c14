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


# ------------------------------------------------ fp8 recurrent checkpoint
def fp8_ckpt_parts(layer):
    """(codes uint8 [B][Hv][P][N], scales float32 [B][Hv][P]) of a layer's fp8
    checkpoint (rows of N codes and a 16-byte trailer holding the scale)."""
    ck = layer.ckpt.cpu().numpy()
    N = ck.shape[-1] - 16
    sig = np.ascontiguousarray(ck[..., N:N + 4]).view(np.float32)[..., 0]
    return ck[..., :N].copy(), sig.copy()


def fp8_ckpt_values(layer) -> np.ndarray:
    """Values the fp8 checkpoint holds (code value * row scale, float64)."""
    from oracle import stochastic
    return stochastic.fp8_checkpoint_values(*fp8_ckpt_parts(layer))


def set_fp8_ckpt(layer, S) -> np.ndarray:
    """Store S in a layer's fp8 checkpoint (row-scaled e4m3, nearest even, the
    fp8 copy's encoding) and return the values it then holds."""
    import torch
    from oracle import quant, stochastic
    codes, sig = quant.quantize_rows_fp8(np.asarray(S, dtype=np.float32))
    N = codes.shape[-1]
    raw = np.zeros(codes.shape[:-1] + (N + 16,), dtype=np.uint8)
    raw[..., :N] = codes
    raw[..., N:N + 4] = sig.astype(np.float32)[..., None].view(np.uint8)
    layer.ckpt.copy_(torch.from_numpy(raw))
    return stochastic.fp8_checkpoint_values(codes, sig)


def check_fp8_ckpt(layer, S_new, seed, epoch, where, max_frac=2e-3):
    """The fp8 checkpoint a fold stored vs the oracle's stochastic rounding of
    its fp64 fold S_new.  The kernel's fp32 fold and fl32 of the oracle's
    fp64 fold differ by a few ulps: the power-of-two row scales agree except
    in a rare row whose maximum straddles a scale boundary (then by a factor
    2; its codes are not compared), and codes agree except rare entries one
    code apart whose two values straddle a rounding threshold (or that differ
    only in the sign of a zero).  Returns the fraction of such entries."""
    from oracle import stochastic
    codes, sig = fp8_ckpt_parts(layer)
    rc, rs = stochastic.checkpoint_round_fp8(S_new, seed, epoch)
    moved = sig != rs
    assert moved.sum() <= 2, (where, int(moved.sum()))
    assert np.all((sig[moved] == 2 * rs[moved]) | (2 * sig[moved] == rs[moved])), where
    g, r = codes.astype(np.int64), rc.astype(np.int64)
    gm, rm, gs, rsn = g & 0x7F, r & 0x7F, g >> 7, r >> 7
    diff = ((gm != rm) | ((gs != rsn) & (gm != 0))) & ~moved[..., None]
    assert np.all(np.abs(gm - rm)[diff] == 1) and np.all(((gs == rsn) | (gm == 0) | (rm == 0))[diff]), where
    assert diff.sum() <= max(2, max_frac * diff.size), (where, diff.mean())
    return float(diff.mean())
