"""Pins of the oracle's bf16 and OCP fp8 e4m3fn encoders.

Library routines serve as the independent reference: torch's CPU casts to
bfloat16 and float8_e4m3fn both round to nearest even.  torch does not
saturate (it gives NaN above 464), so it is compared on |x| <= 464 only; the
saturating behaviour is pinned by the format's fixed points.
"""
import numpy as np
import torch

from oracle import quant


def _specials32():
    return np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                     1.17549435e-38, 1.4e-45, -1.4e-45, 65504.0, 1e-30], dtype=np.float32)


def test_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-40, 40, 200000))).astype(np.float32)
    # exact ties: low 16 bits = 0x8000, both parities of the kept lsb
    ties = (rng.integers(0, 2 ** 31, 20000, dtype=np.uint64).astype(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = np.concatenate([x, ties.view(np.float32), _specials32()])
    x = x[np.isfinite(x) | np.isinf(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = quant.bf16_bits(x)
    np.testing.assert_array_equal(got, ref)
    back = quant.bf16_value(got)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy())


def _e4m3_grid():
    codes = np.arange(256, dtype=np.uint8)
    vals = quant.e4m3_decode(codes)
    fin = np.isfinite(vals)
    return codes[fin], vals[fin]


def test_e4m3_decode_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = quant.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    np.testing.assert_array_equal(got[m], ref[m])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(300000) * np.exp(rng.uniform(-14, 6.5, 300000))).astype(np.float32)
    _, vals = _e4m3_grid()
    pos = np.unique(np.abs(vals))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)       # exact ties
    x = np.concatenate([x, mids, -mids, pos.astype(np.float32), np.float32([464.0, -464.0, 0.0, -0.0])])
    x = x[np.abs(x) <= 464.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = quant.e4m3_encode(x)
    np.testing.assert_array_equal(got, ref)


def test_e4m3_fixed_points_and_saturation():
    enc = quant.e4m3_encode
    assert enc(448.0) == 0x7E and enc(-448.0) == 0xFE
    assert enc(460.0) == 0x7E and enc(1e6) == 0x7E and enc(-np.inf) == 0xFE
    assert enc(2.0 ** -6) == 0x08 and enc(2.0 ** -9) == 0x01
    assert enc(2.0 ** -10) == 0x00                 # tie between 0 and 2^-9 -> even (0)
    assert enc(3 * 2.0 ** -10) == 0x02             # tie between 1 and 2 quanta -> even
    assert enc(1.0) == 0x38 and enc(1.0625) == 0x38 and enc(1.1875) == 0x3A
    assert enc(np.nan) & 0x7F == 0x7F


def test_row_scaled_fp8_roundtrip_bounds():
    rng = np.random.default_rng(2)
    rows = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-5, 5, (64, 1)))).astype(np.float32)
    rows[3] = 0.0
    codes, sig = quant.quantize_rows_fp8(rows)
    assert sig[3] == 1.0 and np.all(codes[3] == 0)
    amax = np.abs(rows).max(axis=1)
    np.testing.assert_array_equal(sig[amax > 0], (amax[amax > 0] / np.float32(448)).astype(np.float32))
    deq = quant.dequantize_rows_fp8(codes, sig)
    # each row's max maps to (about) 448; relative step of e4m3 normals is 2^-3,
    # so the rounding error is at most 2^-4 relative for normals, and half the
    # subnormal quantum (2^-10 sigma) below 2^-6 sigma
    y = rows / sig[:, None]
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10) * sig[:, None] * (1 + 1e-6)
    assert np.all(np.abs(deq - rows) <= bound)
    assert np.all(np.abs(quant.e4m3_decode(codes)).max(axis=1)[amax > 0] == 448.0)
