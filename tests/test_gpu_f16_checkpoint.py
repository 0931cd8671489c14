"""GPU parity of the fp16 recurrent checkpoint with stochastic rounding.

The oracle (oracle/stochastic.py) computes the same draws from the same
hash, so the rounding decisions agree except where the kernel's fp32 fold and
the oracle's fp64 fold fall on different sides of a decision threshold (the
decision is taken on the fold's fp32 value on both sides, but the fp32 values
themselves differ by a few units in the last place).  A checkpoint entry may
then differ by one fp16 step; such entries must be rare (<= 1 in 500 here).
Everything read from an unchanged checkpoint (outputs, verification, read
copies) is compared at the fp32 tolerance or bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import lowprec, quant, recurrence, stochastic
from ssm_layer_decode_amd import workloads as W
from tests.helpers import normwise_err, say, to_dev, unpack_e2m1

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ssm_layer_decode_amd import _lib
    _lib.load()
    return torch.device("cuda:0")


def _layer(sh, dev, **kw):
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    return ReplaySSM(LayerConfig.of(sh, ckpt="f16sr", **kw), device=dev)


def _f16(x):
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


def _ulp16(a):
    a = np.abs(a)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -14)
    return np.ldexp(1.0, (e - 10).astype(np.int64))


def _check_ckpt(got, ref, where):
    """fp16 checkpoint vs the oracle's: equal except rare one-step flips."""
    got = np.asarray(got, dtype=np.float64)
    diff = got != ref
    frac = diff.mean()
    step = _ulp16(np.maximum(np.abs(got), np.abs(ref)))
    assert np.all(np.abs(got - ref)[diff] <= step[diff]), where
    # flips are rare independent events: a fraction bound, but at least 2 entries
    assert diff.sum() <= max(2, 2e-3 * diff.size), (where, frac)
    return frac


def _dev_read(layer, fmt):
    """What non-flush steps read, dequantised (float64): the read copy, or the
    fp16 checkpoint itself without one."""
    if fmt == "none":
        return layer.ckpt.float().cpu().numpy().astype(np.float64)
    if fmt == "bf16":
        return layer.read_copy.float().cpu().numpy().astype(np.float64)
    R = layer.read_copy.cpu().numpy()
    if fmt == "mxfp4":
        R = unpack_e2m1(R)
    return quant.dequantize(R, layer.row_scale.cpu().numpy(), fmt)


def _check_copy(layer, S_new, fmt, where):
    """Copy written from the kernel's unrounded fp32 fold vs Q of the oracle's
    fp64 fold, code by code: the two folds' fp32 values can straddle a
    rounding threshold (or, for a row or block maximum, move the fp8 scale by
    a few ulps), so codes may differ by one step in rare entries; fp8 scales
    agree to 2^-20 relative, MXFP4 block exponents exactly (but for a rare
    block)."""
    codes, sc = quant.quantize(S_new, fmt)
    r = codes.astype(np.int64)
    if fmt == "bf16":
        g = layer.read_copy.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
        mask, sbit = 0x7FFF, 15
    elif fmt == "fp8":
        g = layer.read_copy.cpu().numpy().astype(np.int64)
        mask, sbit = 0x7F, 7
        # the kernel's fp32 fold of L + 1 terms carries a few ulps of rounding, so its row
        # maximum, and with it the scale amax / 448, may differ from fl32(fp64 fold) by ~4 ulps
        np.testing.assert_allclose(layer.row_scale.cpu().numpy(), sc, rtol=2.0 ** -20, atol=0)
    else:
        g = unpack_e2m1(layer.read_copy.cpu().numpy()).astype(np.int64)
        mask, sbit = 0x7, 3
        ex = layer.row_scale.cpu().numpy()
        assert (ex != sc).sum() <= 2, where
    gm, rm, gs, rs = g & mask, r & mask, g >> sbit, r >> sbit
    diff = (gm != rm) | ((gs != rs) & (gm != 0))
    if fmt == "mxfp4":
        diff &= ~np.repeat(ex != sc, 32, axis=-1)     # a block whose exponent moved: codes rescaled
    assert np.all(np.abs(gm - rm)[diff] == 1) and np.all(((gs == rs) | (gm == 0) | (rm == 0))[diff]), where
    assert diff.sum() <= max(2, 2e-3 * diff.size), (where, diff.mean())


@pytest.mark.parametrize("fmt,hvpt", [("none", 0), ("none", 4), ("fp8", 0), ("mxfp4", 0), ("mxfp4", 4), ("bf16", 2),
                                      ("mxfp4", 2)])
def test_decode_with_f16_checkpoint(dev, fmt, hvpt):
    """After every fold the oracle restarts from what the GPU stored:
      * fold: eq.R from the previous stored checkpoint through the window
        gives S_new; the flush output is S_new q (1e-5); the stored fp16
        checkpoint is the oracle's stochastic rounding of S_new at the fold's
        epoch (rare one-step flips); the copy is Q(S_new) (rare one-step flips);
      * non-flush: o = gamma deq(R) q + sum_j gamma_{j+1:h} v_j (k_j . q) for the
        read data R the layer holds (the copy, or the fp16 checkpoint), 1e-5."""
    sh = W.Shape(batch=3, n_vheads=4, n_kheads=2, dim_v=16, dim_k=64, window=4, dist="uniform")
    steps, seed = 18, 1234567
    say(f"case: fp16 checkpoint decode copy={fmt} hvpt={hvpt}")
    S0 = _f16(W.initial_state_np(sh, 21, std=0.5))
    layer = _layer(sh, dev, read_copy=fmt, heads_per_tile=hvpt, sr_seed=seed)
    layer.ckpt.copy_(torch.from_numpy(S0.astype(np.float16)))
    if fmt != "none":
        layer.refresh_read_copy()
    ins = [W.decode_inputs_np(sh, 22, t) for t in range(steps)]
    C, Rd = S0, _dev_read(layer, fmt)                 # stored checkpoint and read data at the last fold
    recs, flips = [], []
    for t, x in enumerate(ins, start=1):
        assert np.all(layer.fold_epochs() == (t - 1) // sh.window)     # folds stored so far
        o = layer.decode_step(*to_dev(x, dev)).cpu().numpy()
        if t % sh.window == 0:
            steps_ = [(a, k, v, np.zeros_like(k)) for (a, k, v) in recs] + [x]
            o_ref, _, S_new = recurrence.decode(C, steps_, group=sh.group)
            assert normwise_err(o, o_ref[-1]) <= TOL, t
            epoch = (t - 1) // sh.window
            flips.append(_check_ckpt(layer.ckpt.float().cpu().numpy(),
                                     stochastic.checkpoint_round(S_new, seed, epoch), f"fold at step {t}"))
            if fmt != "none":
                _check_copy(layer, S_new, fmt, f"copy at step {t}")
            C = layer.ckpt.float().cpu().numpy().astype(np.float64)
            Rd = _dev_read(layer, fmt)
            recs = []
        else:
            d = tuple(np.asarray(y)[:, None] for y in x)
            ref = lowprec.split_read_verify(Rd, recs, d, "f64", group=sh.group)[:, 0]
            assert normwise_err(o, ref) <= TOL, (t, normwise_err(o, ref))
            recs.append((x[0], x[1], x[2]))
    assert layer.read_error() == 0
    say(f"  checkpoint entries rounded the other way: {[f'{f:.1e}' for f in flips]}")


def test_verify_and_commit_with_f16_checkpoint(dev):
    """Verification reads the fp16 checkpoint; the fold a commit triggers
    rounds with the commit's launch number."""
    sh = W.Shape(batch=4, n_vheads=4, n_kheads=2, dim_v=16, dim_k=32, window=6, max_draft=4, dist="uniform")
    seed = 99
    say("case: fp16 checkpoint verify + commit")
    S0 = _f16(W.initial_state_np(sh, 31, std=0.5))
    layer = _layer(sh, dev, sr_seed=seed)
    layer.ckpt.copy_(torch.from_numpy(S0.astype(np.float16)))
    recs = [W.decode_inputs_np(sh, 32, t) for t in range(3)]
    for x in recs:
        layer.decode_step(*to_dev(x, dev))
    committed = [(x[0], x[1], x[2]) for x in recs]
    S_ckpt = S0
    for r in range(6):
        T = 4
        drafts = W.draft_inputs_np(sh, 33, r, T)
        O = layer.spec_verify(*to_dev(drafts, dev)).cpu().numpy()
        ref = lowprec.split_read_verify(S_ckpt, committed, drafts, "none", group=sh.group)
        assert normwise_err(O, ref) <= TOL, (r, normwise_err(O, ref))
        # commit the same count for every sequence so the fold happens in lockstep
        a_r = 3 if r % 2 == 0 else 1
        acc = np.full(sh.batch, a_r, dtype=np.int32)
        epoch = layer.fold_epochs()
        layer.commit(torch.from_numpy(acc).to(dev))
        committed += [(drafts[0][:, t], drafts[1][:, t], drafts[2][:, t]) for t in range(a_r)]
        if len(committed) >= sh.window:
            steps = [(a, k, v, np.zeros_like(k)) for (a, k, v) in committed]
            _, _, S_new = recurrence.decode(S_ckpt, steps, group=sh.group)
            S_ckpt = stochastic.checkpoint_round(S_new, seed, epoch)
            _check_ckpt(layer.ckpt.float().cpu().numpy(), S_ckpt, f"commit fold in round {r}")
            assert np.all(layer.fold_epochs() == epoch + 1)
            S_ckpt = layer.ckpt.float().cpu().numpy().astype(np.float64)   # continue from the stored values
            committed = []
    assert layer.read_error() == 0


def test_reset_and_refresh_with_f16_checkpoint(dev):
    sh = W.Shape(batch=3, n_vheads=2, n_kheads=2, dim_v=8, dim_k=64, window=4, dist="uniform")
    say("case: fp16 checkpoint reset + refresh")
    S0 = W.initial_state_np(sh, 41, std=2.0).astype(np.float16)
    for fmt in ("fp8", "mxfp4"):
        layer = _layer(sh, dev, read_copy=fmt)
        layer.ckpt.copy_(torch.from_numpy(S0))
        layer.refresh_read_copy()
        R, sc = quant.quantize(S0.astype(np.float32), fmt)
        got = layer.read_copy.cpu().numpy()
        if fmt == "mxfp4":
            got = unpack_e2m1(got)
        np.testing.assert_array_equal(got & 0x7F if fmt == "fp8" else got, R & 0x7F if fmt == "fp8" else R)
        np.testing.assert_array_equal(layer.row_scale.cpu().numpy(), sc)
        layer.reset(torch.tensor([1], dtype=torch.int32, device=dev))
        ck = layer.ckpt.cpu().numpy()
        assert np.all(ck[1] == 0) and np.array_equal(ck[0], S0[0]) and np.array_equal(ck[2], S0[2])


def test_f16_checkpoint_keeps_infinities_and_nan(dev):
    """A fold whose fp32 result is infinite stays infinite, NaN stays NaN,
    and a finite value beyond the fp16 range saturates at 65504 (the oracle's
    rounding, entry by entry).  L = 1: every decode step folds."""
    sh = W.Shape(batch=1, n_vheads=1, n_kheads=1, dim_v=4, dim_k=16, window=1, dist="uniform")
    say("case: fp16 checkpoint with inf, nan and overflow")
    S0 = np.zeros((1, 1, 4, 16))
    S0[0, 0, 0, :4] = [np.inf, -np.inf, np.nan, 60000.0]
    S0[0, 0, 1, :3] = [-60000.0, 65504.0, 1.0]
    S0[0, 0, 2:] = np.linspace(-3, 3, 32).reshape(2, 16)
    S0 = S0.astype(np.float16).astype(np.float64)       # what the fp16 checkpoint holds
    layer = _layer(sh, dev, sr_seed=5)
    layer.ckpt.copy_(torch.from_numpy(S0.astype(np.float16)))
    a = np.ones((1, 1), dtype=np.float32)
    k = np.zeros((1, 1, 16), dtype=np.float32)
    k[0, 0, :4] = [1.0, 1.0, 1.0, 1.0]
    v = np.array([[[20000.0, -20000.0, 0.5, 0.25]]], dtype=np.float32)
    q = np.zeros((1, 1, 16), dtype=np.float32)
    layer.decode_step(*to_dev((a, k, v, q), dev))
    got = layer.ckpt.float().cpu().numpy().astype(np.float64)
    S1 = S0 + v[..., :, None].astype(np.float64) * k[..., None, :].astype(np.float64)
    ref = stochastic.checkpoint_round(S1, 5, 0)
    assert np.isposinf(got[0, 0, 0, 0]) and np.isneginf(got[0, 0, 0, 1]) and np.isnan(got[0, 0, 0, 2])
    assert got[0, 0, 0, 3] == 65504.0 and got[0, 0, 1, 0] == -65504.0 and got[0, 0, 1, 1] == 45504.0
    np.testing.assert_array_equal(got, ref)
    assert np.all(layer.fold_epochs() == 1)
