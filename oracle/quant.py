"""Low-precision encoders for the read copy -- TEST INFRASTRUCTURE ONLY.

The pages keep a high-precision checkpoint for the recurrence and a separate
low-precision copy that only non-flush reads use; at a flush the folded state
is converted independently into both formats ([ru] §06; [ar] "limiting
quantization error"; [zh] method points).  The pages use NVFP4; the formats
here are the ones this library offers (readings):

* bf16: round to nearest, ties to even, from the fp32 value.
* fp8 e4m3fn (OCP 8-bit floating point, E4M3): bias 7, 3 mantissa bits, no
  infinities, NaN = S.1111.111, largest finite 448, subnormal quantum 2^-9.
  Encoding is round to nearest even with saturation to +-448.
  Per-row scale: for each state row r (the N entries that form one output
  element's dot product) sigma_r = fl32(amax_r / 448), or 1 when that is not
  positive (an all-zero row); codes = e4m3(fl32(x / sigma_r)).  All decisions
  are taken in fp32, the precision of the checkpoint the codes come from.

Pins (tests/test_quant_pins.py): bf16 against torch's CPU bfloat16 cast (a
library RNE routine); e4m3 encode against torch's float8_e4m3fn cast on every
in-range value tested, the full 256-entry decode table against torch, and the
format's fixed points (448, 2^-6, 2^-9, ties).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


# ---------------------------------------------------------------- bf16
def bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN -> quiet NaN."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f)
    if np.any(nan):
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040)), r)
    return r.astype(np.uint16)


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# ---------------------------------------------------------------- e4m3fn
def e4m3_encode(x) -> np.ndarray:
    """float values -> OCP e4m3fn codes (uint8), RNE, saturating to +-448."""
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    nan = np.isnan(x)
    ax = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    _, e = np.frexp(ax)                     # ax = m 2^e, m in [0.5, 1)
    E = np.where(ax > 0, e - 1, -6)         # floor(log2 ax)
    E = np.maximum(E, -6)                   # below 2^-6 the quantum stays 2^-9
    quantum = np.ldexp(1.0, E - 3)
    M = np.rint(ax / quantum)               # exact scaling; rint = ties to even
    mag = (8 * E + 48 + M).astype(np.int64) # contiguous code space across binades
    mag = np.minimum(mag, 126)
    code = mag.astype(np.uint8) | sign
    if np.any(nan):
        code = np.where(nan, np.uint8(0x7F) | sign, code)
    return code.astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """OCP e4m3fn codes -> float64 values (exact)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    sub = mf * 2.0 ** -9
    nor = (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7)
    v = np.where(ef == 0, sub, nor)
    v = np.where((ef == 15) & (mf == 7), np.nan, v)
    return s * v


def row_scale_fp32(rows) -> np.ndarray:
    """Per-row scale sigma = fl32(amax / 448), 1 where not positive.  rows [..., N]."""
    r = np.asarray(rows, dtype=np.float32)
    amax = np.max(np.abs(r), axis=-1)
    sig = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    return np.where(sig > 0, sig, np.float32(1.0)).astype(np.float32)


def quantize_rows_fp8(rows):
    """Row-scaled e4m3 quantisation of fp32 rows [..., N].
    Returns (codes uint8 [..., N], sigma float32 [...])."""
    r = np.asarray(rows, dtype=np.float32)
    sig = row_scale_fp32(r)
    y = (r / sig[..., None]).astype(np.float32)      # IEEE fp32 division
    return e4m3_encode(y), sig


def dequantize_rows_fp8(codes, sig) -> np.ndarray:
    return e4m3_decode(codes) * np.asarray(sig, dtype=np.float64)[..., None]


def quantize(S, fmt: str):
    """Quantise an fp32 state [..., P, N] to a read copy.
    fmt 'bf16' -> (bits uint16, None); 'fp8' -> (codes uint8, sigma [..., P])."""
    S32 = np.asarray(S, dtype=np.float32)
    if fmt == "bf16":
        return bf16_bits(S32), None
    if fmt == "fp8":
        return quantize_rows_fp8(S32)
    raise ValueError(fmt)


def dequantize(R, sig, fmt: str) -> np.ndarray:
    if fmt == "bf16":
        return bf16_value(R).astype(np.float64)
    if fmt == "fp8":
        return dequantize_rows_fp8(R, sig)
    raise ValueError(fmt)


def roundtrip(S, fmt: str) -> np.ndarray:
    """deq(Q(fl32(S))) in float64.  'f64' is the identity (no rounding at
    all), 'none' rounds to fp32 only."""
    if fmt == "f64":
        return np.array(S, dtype=np.float64, copy=True)
    if fmt == "none":
        return np.asarray(S, dtype=np.float32).astype(np.float64)
    R, sig = quantize(S, fmt)
    return dequantize(R, sig, fmt)
