"""Pins of the oracle's bf16, OCP fp8 e4m3fn and MXFP4 (E2M1 + E8M0) encoders.

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


# ---------------------------------------------------------------- MXFP4
# The E2M1 value set, from the format's definition (1 sign, 2 exponent bits
# with bias 1, 1 mantissa bit; exponent field 0 is subnormal).
E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_decode_table():
    got = quant.e2m1_decode(np.arange(16, dtype=np.uint8))
    np.testing.assert_array_equal(got[:8], E2M1_MAGNITUDES)
    np.testing.assert_array_equal(got[8:], [-m for m in E2M1_MAGNITUDES])
    assert np.signbit(got[8])                     # code 8 is -0


def _e2m1_brute(x):
    """Nearest E2M1 magnitude by exhaustive search; a tie goes to the code with
    mantissa bit 0 (the even code); saturation at 6; sign of x kept."""
    out = []
    for v in np.asarray(x, dtype=np.float64):
        a = min(abs(v), 6.0)
        d = [abs(a - m) for m in E2M1_MAGNITUDES]
        best = min(d)
        cands = [c for c in range(8) if d[c] == best]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        out.append(c | (8 if np.signbit(v) else 0))
    return np.array(out, dtype=np.uint8)


def test_e2m1_encode_matches_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.uniform(-8, 8, 4000),
        rng.standard_normal(2000) * np.exp(rng.uniform(-6, 3, 2000)),
        np.array(E2M1_MAGNITUDES), -np.array(E2M1_MAGNITUDES),
        (np.array(E2M1_MAGNITUDES[1:]) + np.array(E2M1_MAGNITUDES[:-1])) / 2,       # every tie
        -(np.array(E2M1_MAGNITUDES[1:]) + np.array(E2M1_MAGNITUDES[:-1])) / 2,
        [6.0001, 7.0, 7.999, 1e9, -1e9, -0.0, 0.0, 1e-30, -1e-30]])
    np.testing.assert_array_equal(quant.e2m1_encode(x), _e2m1_brute(x))


def test_e2m1_ties_to_even():
    enc = quant.e2m1_encode
    # ties: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    np.testing.assert_array_equal(enc([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]), [0, 2, 2, 4, 4, 6, 6])
    assert enc(5.01) == 7 and enc(100.0) == 7 and enc(-100.0) == 15
    assert enc(-0.1) == 8                          # rounds to -0


def test_mx_block_exponent_cases():
    ex = lambda amax: int(quant.mx_block_exponent(np.array([[amax] + [0.0] * 31]))[0])
    assert ex(6.0) == 0                            # X = 1: 6 is representable as is
    assert ex(1.0) == -2                           # X = 1/4: 1 -> code of 4.0
    assert ex(4.0) == 0 and ex(7.99) == 0 and ex(8.0) == 1
    assert ex(0.0) == -127                         # all-zero block
    assert ex(2.0 ** -140) == -127                 # clamped to the E8M0 range
    assert ex(2.0 ** 127) == 125


def test_mxfp4_roundtrip_bounds():
    rng = np.random.default_rng(4)
    rows = (rng.standard_normal((96, 128)) * np.exp(rng.uniform(-8, 8, (96, 4))).repeat(32, axis=1)).astype(np.float32)
    rows[5] = 0.0
    rows[7, 32:64] = 0.0
    codes, sc = quant.quantize_rows_mxfp4(rows)
    assert codes.shape == rows.shape and sc.shape == (96, 4)
    assert np.all(codes[5] == 0) and np.all(sc[5] == 0) and sc[7, 1] == 0
    deq = quant.dequantize_rows_mxfp4(codes, sc)
    X = np.ldexp(1.0, sc.astype(np.int64) - 127).repeat(32, axis=1)
    # E2M1 has one mantissa bit: relative error <= 1/4 for normals (saturation
    # between 6X and 8X included), half the subnormal step (X/4) below X
    err = np.abs(deq - rows.astype(np.float64))
    assert np.all(err <= np.maximum(0.25 * np.abs(rows), 0.25 * X))
    # each non-zero block's largest entry lands on code 4.0 or 6.0
    blk = np.abs(quant.e2m1_decode(codes)).reshape(96, 4, 32).max(axis=-1)
    nz = np.abs(rows).reshape(96, 4, 32).max(axis=-1) > 0
    assert np.all(np.isin(blk[nz], [4.0, 6.0]))
