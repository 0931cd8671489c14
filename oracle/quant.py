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

* mxfp4 (OCP Microscaling, MXFP4): blocks of 32 consecutive entries of a
  row share one power-of-two scale X = 2^e stored as an E8M0 byte (e + 127);
  each entry is an FP4 E2M1 code (1 sign, 2 exponent bits with bias 1, 1
  mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6).  Reading of the
  scale rule: e = floor(log2 amax_block) - 2 (2 = the largest E2M1 exponent),
  clamped to [-127, 127]; an all-zero block takes e = -127 (E8M0 code 0).
  Codes = e2m1(x / X), round to nearest even, saturating to +-6, sign kept
  (so a small negative entry gives the code of -0).  Scaling by X is exact,
  so these decisions do not depend on the precision they are taken in.
  This stands in for the pages' NVFP4 copy (E2M1 with an E4M3 scale per 16
  entries, an NVIDIA format); MXFP4 is the 4-bit format gfx950 converts
  natively.

Pins (tests/test_quant_pins.py): bf16 against torch's CPU bfloat16 cast (a
library RNE routine); e4m3 encode against torch's float8_e4m3fn cast on every
in-range value tested, the full 256-entry decode table against torch, and the
format's fixed points (448, 2^-6, 2^-9, ties).  E2M1 against brute-force
nearest-even search over its 8 magnitudes and its fixed points; the MX block
scale against the definition's worked cases (amax 6 -> X = 1, amax 1 -> X =
1/4) and a dense sweep of blocks in which every dequantised entry must be
within a quarter of X, plus its relative error, of the input.
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


# ---------------------------------------------------------------- MXFP4
E2M1_MAX = 6.0
E2M1_EMAX = 2
MX_BLOCK = 32


def e2m1_encode(x) -> np.ndarray:
    """float values -> FP4 E2M1 codes (uint8, low 4 bits), RNE, saturating to +-6.

    Below 2 the quantum is 1/2 (the subnormal 0.5 and the binade [1, 2) share
    it); in [2, 4) it is 1, in [4, 6] it is 2.  Codes are contiguous across
    binades, so code = 2 e + rint(|x| / quantum) with e = max(0, floor(log2|x|)).
    """
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(3)
    ax = np.minimum(np.abs(x), E2M1_MAX)
    _, fe = np.frexp(ax)                        # ax = m 2^fe, m in [0.5, 1)
    e = np.where(ax >= 1.0, fe - 1, 0)
    quantum = np.ldexp(1.0, e - 1)
    M = np.rint(ax / quantum)                   # exact scaling; rint = ties to even
    mag = np.minimum(2 * e + M, 7).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def e2m1_decode(code) -> np.ndarray:
    """E2M1 codes -> float64 values (exact): exponent field E (bias 1), mantissa m."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x8, -1.0, 1.0)
    E = (c >> 1) & 0x3
    m = c & 0x1
    v = np.where(E == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, E - 1))
    return s * v


def mx_block_exponent(blocks) -> np.ndarray:
    """Shared exponent e of each block [..., 32]: floor(log2 amax) - 2, clamped
    to [-127, 127]; -127 for an all-zero block."""
    amax = np.max(np.abs(np.asarray(blocks, dtype=np.float64)), axis=-1)
    _, fe = np.frexp(amax)
    e = np.where(amax > 0, fe - 1 - E2M1_EMAX, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_rows_mxfp4(rows):
    """MXFP4 quantisation of fp32 rows [..., N] (N a multiple of 32).
    Returns (codes uint8 [..., N], one E2M1 code per entry; scale codes uint8
    [..., N / 32], E8M0 = e + 127)."""
    r = np.asarray(rows, dtype=np.float32).astype(np.float64)
    n = r.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("MXFP4 rows need a multiple of 32 entries")
    blk = r.reshape(r.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    e = mx_block_exponent(blk)
    codes = e2m1_encode(blk / np.ldexp(1.0, e)[..., None])
    return codes.reshape(r.shape), (e + 127).astype(np.uint8)


def dequantize_rows_mxfp4(codes, scale_codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    n = c.shape[-1]
    blk = e2m1_decode(c).reshape(c.shape[:-1] + (n // MX_BLOCK, MX_BLOCK))
    X = np.ldexp(1.0, np.asarray(scale_codes, dtype=np.int64) - 127)
    return (blk * X[..., None]).reshape(c.shape)


def quantize(S, fmt: str):
    """Quantise an fp32 state [..., P, N] to a read copy.
    fmt 'bf16' -> (bits uint16, None); 'fp8' -> (codes uint8, sigma [..., P]);
    'mxfp4' -> (codes uint8 [..., P, N], E8M0 scale codes uint8 [..., P, N/32])."""
    S32 = np.asarray(S, dtype=np.float32)
    if fmt == "bf16":
        return bf16_bits(S32), None
    if fmt == "fp8":
        return quantize_rows_fp8(S32)
    if fmt == "mxfp4":
        return quantize_rows_mxfp4(S32)
    raise ValueError(fmt)


def dequantize(R, sig, fmt: str) -> np.ndarray:
    if fmt == "bf16":
        return bf16_value(R).astype(np.float64)
    if fmt == "fp8":
        return dequantize_rows_fp8(R, sig)
    if fmt == "mxfp4":
        return dequantize_rows_mxfp4(R, sig)
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
