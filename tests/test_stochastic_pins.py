"""Pins of the oracle's fp16 stochastic rounding and its checkpoint path.

* The hash is a bijection of 32-bit words (an LCG step and an invertible
  output permutation): no collisions over 2^20 consecutive inputs, and its
  output bytes are uniform (chi-square).
* Rounding is checked against numpy's own float16 arithmetic: fp16 values
  stay unchanged, every result is one of the two fp16 neighbours of x, and
  the mean over all 65536 draws equals x exactly in the fp16 normal range
  (within 2^-16 of a step below it).
* The checkpoint path reduces to eq.R when every fold result is an fp16
  value (small integers), whatever the draws.
"""
import numpy as np

from oracle import lowprec, recurrence, stochastic as st
from ssm_layer_decode_amd import workloads as W


def test_hash_bijective_and_uniform():
    x = np.arange(1 << 20, dtype=np.uint64) * np.uint64(2654435761) & np.uint64(0xFFFFFFFF)
    h = st.pcg_hash(x)
    assert np.unique(h).size == x.size
    b = (h & np.uint64(0xFF)).astype(np.int64)
    cnt = np.bincount(b, minlength=256)
    exp = x.size / 256
    chi2 = ((cnt - exp) ** 2 / exp).sum()
    assert chi2 < 350                     # 255 degrees of freedom; 1e-4 tail is ~ 330-350
    hi = ((h >> np.uint64(24)) & np.uint64(0xFF)).astype(np.int64)
    cnt = np.bincount(hi, minlength=256)
    assert ((cnt - exp) ** 2 / exp).sum() < 350


def test_uniform16_covers_both_halves_and_changes_with_key():
    g = np.arange(4096, dtype=np.uint64)
    u1 = st.uniform16(st.fold_key(7, 3), g)
    u2 = st.uniform16(st.fold_key(7, 4), g)
    u3 = st.uniform16(st.fold_key(8, 3), g)
    assert u1.min() >= 0 and u1.max() < 65536
    assert np.mean(u1 == u2) < 0.01 and np.mean(u1 == u3) < 0.01
    assert abs(u1.mean() / 65535 - 0.5) < 0.02


def _neighbours_f16(x32):
    """The fp16 values just below and above |x| (numpy float16 arithmetic)."""
    a = np.abs(x32.astype(np.float64))
    h = a.astype(np.float16)                       # nearest
    hd = h.astype(np.float64)
    lo = np.where(hd > a, np.nextafter(h, np.float16(0)), h).astype(np.float64)
    hi = np.where(hd < a, np.nextafter(h, np.float16(np.inf)), h).astype(np.float64)
    return lo, hi


def test_rounding_against_numpy_float16():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        (rng.standard_normal(3000) * np.exp(rng.uniform(-12, 10, 3000))),
        rng.uniform(-1e-4, 1e-4, 1000),                     # fp16 subnormal range
        np.arange(-2048, 2049) * 2.0 ** -5]).astype(np.float32)
    x = x[np.abs(x) < 65504]
    lo, hi = _neighbours_f16(x)
    for u in (0, 1, 12345, 32768, 65535):
        r = np.abs(st.round_f16_stochastic(x, np.full(x.shape, u)))
        assert np.all((r == lo) | (r == hi))
        assert np.all(r.astype(np.float16).astype(np.float64) == r)        # an fp16 value
    exact = x.astype(np.float16).astype(np.float32) == x
    for u in (0, 65535):
        r = st.round_f16_stochastic(x[exact], np.full(exact.sum(), u))
        np.testing.assert_array_equal(r, x[exact].astype(np.float64))
    r = st.round_f16_stochastic(np.float32([-0.0, 0.0, 1e6, -1e6]), np.zeros(4))
    assert np.signbit(r[0]) and not np.signbit(r[1]) and r[2] == 65504 and r[3] == -65504


def test_rounding_is_unbiased_over_all_draws():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200) * np.exp(rng.uniform(-9, 9, 200))).astype(np.float32)
    normal = np.abs(x) >= 2.0 ** -14
    u = np.arange(65536)
    for xi, nm in zip(x, normal):
        mean = st.round_f16_stochastic(np.full(u.shape, xi), u).mean()
        lo, hi = _neighbours_f16(np.float32([xi]))
        if nm:
            assert mean == np.float64(xi), (xi, mean)
        else:
            assert abs(mean - np.float64(xi)) <= (hi[0] - lo[0]) * 2.0 ** -16


def test_f16_checkpoint_path_reduces_to_eqR_on_exact_values():
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=2, dim_v=6, dim_k=8, window=4, dist="integer")
    steps = 14
    ins = [W.decode_inputs_np(sh, 3, t) for t in range(steps)]
    ins = [(np.ones_like(a), k, v, q) for (a, k, v, q) in ins]   # alpha = 1: integer folds
    S0 = np.random.default_rng(2).integers(-4, 5, (2, 4, 6, 8)).astype(np.float64)
    ref, _, _ = recurrence.decode(S0, ins, group=2)
    got, folds = lowprec.split_read_decode(S0, ins, 4, "none", group=2, keep_folds=True, ckpt="f16sr", seed=5)
    np.testing.assert_array_equal(got, ref)


def test_f16_checkpoint_rounds_at_folds_only():
    """Non-integer inputs: the stored checkpoint is an fp16 value after each
    fold and within one fp16 step of the fold's fp32 value; different seeds
    give different roundings."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=8, dim_k=16, window=4, dist="uniform")
    ins = [W.decode_inputs_np(sh, 4, t) for t in range(8)]
    S0 = W.initial_state_np(sh, 1).astype(np.float16).astype(np.float64)
    _, f1 = lowprec.split_read_decode(S0, ins, 4, "none", keep_folds=True, ckpt="f16sr", seed=1)
    _, f2 = lowprec.split_read_decode(S0, ins, 4, "none", keep_folds=True, ckpt="f16sr", seed=2)
    _, fx = lowprec.split_read_decode(S0, ins, 4, "none", keep_folds=True)
    for t in (4, 8):
        assert np.all(f1[t].astype(np.float16).astype(np.float64) == f1[t])
        assert not np.array_equal(f1[t], f2[t])
    lo, hi = _neighbours_f16(fx[4].astype(np.float32))
    a = np.abs(f1[4])
    assert np.all((a == lo) | (a == hi))


def test_rounding_keeps_infinities_and_nan():
    """Infinities stay infinite with their sign, NaN stays NaN, and finite
    values beyond the fp16 range saturate at +-65504, whatever the draw."""
    x = np.array([np.inf, -np.inf, np.nan, 1e6, -1e6, 65504.0, 65519.0, -65535.0], dtype=np.float32)
    for u in (0, 1, 32767, 65535):
        r = st.round_f16_stochastic(x, np.full(x.shape, u))
        assert np.isposinf(r[0]) and np.isneginf(r[1]) and np.isnan(r[2])
        np.testing.assert_array_equal(r[3:], [65504.0, -65504.0, 65504.0, 65504.0, -65504.0])


def test_checkpoint_round_epochs_per_sequence():
    """A per-sequence epoch array rounds each sequence as a scalar epoch
    would; sequences with different epochs draw different numbers."""
    rng = np.random.default_rng(3)
    S = rng.standard_normal((3, 2, 4, 8)) * 3
    ep = np.array([0, 5, 2])
    got = st.checkpoint_round(S, 9, ep)
    for b in range(3):
        np.testing.assert_array_equal(got[b], st.checkpoint_round(S, 9, int(ep[b]))[b])
    assert np.mean(st.checkpoint_round(S, 9, 0) != st.checkpoint_round(S, 9, 1)) > 0.1


# ---------------------------------------------------------------- fp8 (r22)
def _e4m3_grid():
    """All finite non-negative e4m3fn values, ascending (from the code table)."""
    from oracle import quant
    v = quant.e4m3_decode(np.arange(128, dtype=np.uint8))
    return np.unique(v[np.isfinite(v)])


def _neighbours_e4m3(y):
    """Largest e4m3 value <= |y| and smallest >= |y| (saturating at 448), by search."""
    g = _e4m3_grid()
    a = np.minimum(np.abs(np.asarray(y, dtype=np.float64)), 448.0)
    i = np.searchsorted(g, a, side="right") - 1
    lo = g[i]
    hi = np.where(lo == a, lo, g[np.minimum(i + 1, len(g) - 1)])
    return lo, hi


def test_e4m3_rounding_against_the_code_table():
    """Every result is one of the two e4m3 neighbours of |y| found by search
    over the code table, with y's sign; e4m3 values are kept for every draw;
    beyond 448 every draw saturates; zero keeps its sign."""
    rng = np.random.default_rng(11)
    y = np.concatenate([
        rng.standard_normal(3000) * np.exp(rng.uniform(-9, 6, 3000)),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 1000),            # e4m3 subnormal range (step 2^-9)
        np.arange(-300, 301) * 0.75]).astype(np.float32)
    y = y[np.abs(y) <= 448]
    lo, hi = _neighbours_e4m3(y)
    for u in (0, 1, 4321, 32768, 65535):
        r = st.round_e4m3_stochastic(y, np.full(y.shape, u))
        assert np.all((np.abs(r) == lo) | (np.abs(r) == hi))
        assert np.all(np.signbit(r) == np.signbit(y))
    g = _e4m3_grid()
    on = np.concatenate([g, -g]).astype(np.float32)
    for u in (0, 65535):
        np.testing.assert_array_equal(st.round_e4m3_stochastic(on, np.full(on.shape, u)), on.astype(np.float64))
    big = np.float32([448.5, 470.0, 479.9, 1e4, -455.0])
    for u in (0, 65535):
        np.testing.assert_array_equal(st.round_e4m3_stochastic(big, np.full(5, u)), [448, 448, 448, 448, -448])
    r = st.round_e4m3_stochastic(np.float32([-0.0, 0.0]), np.zeros(2))
    assert r[0] == 0 and r[1] == 0 and np.signbit(r[0]) and not np.signbit(r[1])
    # u = 0 rounds every value off the grid up in magnitude; the largest draw rounds down
    off = y[lo != hi]
    lo_off, hi_off = _neighbours_e4m3(off)
    np.testing.assert_array_equal(np.abs(st.round_e4m3_stochastic(off, np.zeros(off.shape))), hi_off)
    frac = (np.abs(off.astype(np.float64)) - lo_off) / (hi_off - lo_off)
    small = frac <= 65535 / 65536
    np.testing.assert_array_equal(np.abs(st.round_e4m3_stochastic(off[small], np.full(small.sum(), 65535))),
                                  lo_off[small])


def test_e4m3_rounding_is_unbiased_over_all_draws():
    """The mean over all 65536 draws is within step * 2^-16 of y, and equals
    y exactly where y's dropped fraction is a multiple of 2^-16."""
    rng = np.random.default_rng(12)
    u = np.arange(65536)
    y = (rng.standard_normal(60) * np.exp(rng.uniform(-8, 5, 60))).astype(np.float32)
    y = y[np.abs(y) < 448]
    for yi in y:
        lo, hi = _neighbours_e4m3(np.float32([yi]))
        mean = np.abs(st.round_e4m3_stochastic(np.full(u.shape, yi), u)).mean()
        assert abs(mean - abs(np.float64(yi))) <= (hi[0] - lo[0]) * 2.0 ** -16, yi
    k = rng.integers(0, 65536, 40)
    e = rng.integers(-6, 8, 40)
    exact = ((8 + k / 65536.0) * np.ldexp(1.0, e - 3)).astype(np.float32)   # 20 significant bits: exact in fp32
    for yi in exact:
        assert np.abs(st.round_e4m3_stochastic(np.full(u.shape, yi), u)).mean() == np.float64(yi), yi


def test_e4m3_rounding_of_non_finite_values_is_nan():
    r = st.round_e4m3_stochastic(np.float32([np.inf, -np.inf, np.nan]), np.zeros(3))
    assert np.all(np.isnan(r))


def test_fp8_checkpoint_keeps_rows_on_the_grid():
    """Rows whose largest magnitude is 448 * 2^s and whose entries are e4m3
    values times 2^s store sigma = 2^s and codes that decode to the row
    exactly, for every seed and epoch."""
    rng = np.random.default_rng(13)
    g = _e4m3_grid()
    vals = rng.choice(np.concatenate([g, -g]), size=(2, 3, 5, 16))
    vals[..., 0] = 448.0
    s = rng.integers(-20, 10, (2, 3, 5))
    S = vals * np.ldexp(1.0, s)[..., None]
    for seed, ep in ((0, 0), (7, 3)):
        codes, sig = st.checkpoint_round_fp8(S, seed, ep)
        np.testing.assert_array_equal(sig, np.ldexp(1.0, s).astype(np.float32))
        np.testing.assert_array_equal(st.fp8_checkpoint_values(codes, sig), S)


def test_fp8_checkpoint_rounding_properties():
    """Random folds: sigma is the smallest power of two with amax <= 448
    sigma (so amax / sigma lies in (224, 448]), every stored value is one of
    the two e4m3 neighbours of y = x / sigma, different seeds and epochs draw
    differently, per-sequence epochs round each sequence as its scalar
    epoch, and a zero row stores sigma = 1."""
    from oracle import quant
    rng = np.random.default_rng(14)
    S = rng.standard_normal((3, 2, 6, 32)) * np.exp(rng.uniform(-5, 5, (3, 2, 6, 1)))
    S[1, 0, 2] = 0.0
    codes, sig = st.checkpoint_round_fp8(S, 4, 0)
    amax = np.abs(S.astype(np.float32)).max(axis=-1).astype(np.float64)
    s = np.log2(sig.astype(np.float64))
    assert np.all(s == np.round(s))                                  # powers of two
    nz = amax > 0
    assert np.all(amax[nz] <= 448 * sig[nz]) and np.all(amax[nz] > 224 * sig[nz])
    assert sig[1, 0, 2] == 1.0
    y = (S.astype(np.float32) / sig[..., None]).astype(np.float32)
    lo, hi = _neighbours_e4m3(y)
    got = np.abs(quant.e4m3_decode(codes))
    assert np.all((got == lo) | (got == hi))
    assert np.mean(codes != st.checkpoint_round_fp8(S, 5, 0)[0]) > 0.05
    assert np.mean(codes != st.checkpoint_round_fp8(S, 4, 1)[0]) > 0.05
    ep = np.array([2, 0, 9])
    per_seq = st.checkpoint_round_fp8(S, 4, ep)[0]
    for b in range(3):
        np.testing.assert_array_equal(per_seq[b], st.checkpoint_round_fp8(S, 4, int(ep[b]))[0][b])


def test_fp8_checkpoint_non_finite_rows():
    """NaN entries are ignored by the row scale and store the NaN code 0x7f;
    an infinite entry makes the row's scale infinite (its finite entries then
    store zero codes, the infinite one NaN); scales of extreme rows are
    clamped to 2^-126 .. 2^127."""
    S = np.zeros((1, 1, 2, 16))
    S[0, 0, 0, :] = np.arange(16) - 7.5
    S[0, 0, 0, 3] = np.nan
    S[0, 0, 1, :] = 1.0
    S[0, 0, 1, 5] = -np.inf
    codes, sig = st.checkpoint_round_fp8(S, 1, 0)
    assert sig[0, 0, 0] == 2.0 ** -5 and codes[0, 0, 0, 3] == 0x7F          # 7.5 / 2^-5 = 240
    assert np.isposinf(sig[0, 0, 1]) and codes[0, 0, 1, 5] == 0x7F
    assert np.all((codes[0, 0, 1, :5] & 0x7F) == 0) and np.all((codes[0, 0, 1, 6:] & 0x7F) == 0)
    np.testing.assert_array_equal(st.fp8_row_scale(np.float32([1e-40, 3e38, 448, 449, 0])),
                                  np.float32([2.0 ** -126, 2.0 ** 120, 1, 2, 1]))


def test_fp8_split_path_stores_the_rounded_fold():
    """The split path with an fp8 checkpoint: the first fold stores the fp8
    rounding (seed, epoch 0) of eq.R's state at that step, the second
    (epoch 1) that of eq.R continued from the stored first one, and flush
    outputs come from the unrounded fold."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=8, dim_k=32, window=4, dist="uniform")
    ins = [W.decode_inputs_np(sh, 6, t) for t in range(8)]
    S0 = W.initial_state_np(sh, 2)
    got, folds = lowprec.split_read_decode(S0, ins, 4, "mxfp4", keep_folds=True, ckpt="fp8sr", seed=3)
    _, _, S4 = recurrence.decode(S0, ins[:4])
    np.testing.assert_array_equal(folds[4], st.fp8_checkpoint_values(*st.checkpoint_round_fp8(S4, 3, 0)))
    o8, _, S8 = recurrence.decode(folds[4], ins[4:8])
    np.testing.assert_array_equal(folds[8], st.fp8_checkpoint_values(*st.checkpoint_round_fp8(S8, 3, 1)))
    np.testing.assert_allclose(got[7], o8[-1], rtol=1e-12, atol=1e-12)
