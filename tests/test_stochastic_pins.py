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
    u1 = st.uniform16(st.launch_key(7, 3), g)
    u2 = st.uniform16(st.launch_key(7, 4), g)
    u3 = st.uniform16(st.launch_key(8, 3), g)
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
