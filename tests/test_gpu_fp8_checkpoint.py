"""GPU parity of the fp8 recurrent checkpoint (row-scaled e4m3 with
stochastic rounding, reading r22; always read through a copy).

The oracle (oracle/stochastic.py) computes the same scale and draws, so codes
agree except where the kernel's fp32 fold and the oracle's fp64 fold put y on
different sides of a decision threshold; such entries must be rare and one
code apart (tests/helpers.check_fp8_ckpt).  After every fold the oracle
restarts from what the GPU stored, and everything read from an unchanged
checkpoint (outputs, verification, read copies) is compared at the fp32
tolerance or bit for bit.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import lowprec, quant, recurrence, stochastic
from ssm_layer_decode_amd import workloads as W
from tests.helpers import (check_fp8_ckpt, fp8_ckpt_parts, fp8_ckpt_values, normwise_err, say, set_fp8_ckpt,
                           to_dev, unpack_e2m1)

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
    return ReplaySSM(LayerConfig.of(sh, ckpt="fp8sr", **kw), device=dev)


def _dev_read(layer, fmt):
    """The read copy the layer holds, dequantised (float64)."""
    if fmt == "bf16":
        return layer.read_copy.float().cpu().numpy().astype(np.float64)
    R = layer.read_copy.cpu().numpy()
    if fmt == "mxfp4":
        R = unpack_e2m1(R)
    return quant.dequantize(R, layer.row_scale.cpu().numpy(), fmt)


def _check_copy(layer, S_new, fmt, where):
    """Copy written from the kernel's unrounded fp32 fold vs Q of the oracle's
    fp64 fold: codes equal but for rare one-step entries (the two folds' fp32
    values may straddle a rounding threshold or move a row or block maximum)."""
    codes, sc = quant.quantize(S_new, fmt)
    r = codes.astype(np.int64)
    if fmt == "bf16":
        g = layer.read_copy.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
        mask, sbit = 0x7FFF, 15
    elif fmt == "fp8":
        g = layer.read_copy.cpu().numpy().astype(np.int64)
        mask, sbit = 0x7F, 7
        np.testing.assert_allclose(layer.row_scale.cpu().numpy(), sc, rtol=2.0 ** -20, atol=0)
    else:
        g = unpack_e2m1(layer.read_copy.cpu().numpy()).astype(np.int64)
        mask, sbit = 0x7, 3
        ex = layer.row_scale.cpu().numpy()
        assert (ex != sc).sum() <= 2, where
    gm, rm, gs, rs = g & mask, r & mask, g >> sbit, r >> sbit
    diff = (gm != rm) | ((gs != rs) & (gm != 0))
    if fmt == "mxfp4":
        diff &= ~np.repeat(ex != sc, 32, axis=-1)
    assert np.all(np.abs(gm - rm)[diff] == 1) and np.all(((gs == rs) | (gm == 0) | (rm == 0))[diff]), where
    assert diff.sum() <= max(2, 2e-3 * diff.size), (where, diff.mean())


@pytest.mark.parametrize("fmt,hvpt,P,N,g", [("mxfp4", 0, 16, 64, 2), ("mxfp4", 4, 16, 64, 2),
                                            ("fp8", 0, 16, 64, 2), ("bf16", 0, 16, 64, 2),
                                            ("mxfp4", 0, 128, 128, 1), ("fp8", 0, 128, 128, 4)])
def test_decode_with_fp8_checkpoint(dev, fmt, hvpt, P, N, g):
    """After every fold: the flush output is S_new q (1e-5) for eq.R's S_new
    from the previous stored checkpoint; the stored fp8 checkpoint is the
    oracle's stochastic rounding of S_new at the fold's epoch (rare one-code
    entries); the copy is Q(S_new).  Non-flush outputs equal the replay form
    over the copy the layer holds (1e-5).  The cases cover the two-head
    decode (MXFP4, narrow fp8) and the tile-wide decode (bf16, fp8 of
    128-row heads)."""
    Hv = 4
    sh = W.Shape(batch=3, n_vheads=Hv, n_kheads=Hv // g, dim_v=P, dim_k=N, window=4, dist="uniform")
    steps, seed = 18, 7654321
    say(f"case: fp8 checkpoint decode copy={fmt} hvpt={hvpt} P={P} N={N} g={g}")
    layer = _layer(sh, dev, read_copy=fmt, heads_per_tile=hvpt, sr_seed=seed)
    C = set_fp8_ckpt(layer, W.initial_state_np(sh, 23, std=0.5))
    layer.refresh_read_copy()
    Rd = _dev_read(layer, fmt)
    ins = [W.decode_inputs_np(sh, 24, t) for t in range(steps)]
    recs, flips = [], []
    for t, x in enumerate(ins, start=1):
        assert np.all(layer.fold_epochs() == (t - 1) // sh.window)
        o = layer.decode_step(*to_dev(x, dev)).cpu().numpy()
        if t % sh.window == 0:
            steps_ = [(a, k, v, np.zeros_like(k)) for (a, k, v) in recs] + [x]
            o_ref, _, S_new = recurrence.decode(C, steps_, group=sh.group)
            assert normwise_err(o, o_ref[-1]) <= TOL, t
            flips.append(check_fp8_ckpt(layer, S_new, seed, (t - 1) // sh.window, f"fold at step {t}"))
            _check_copy(layer, S_new, fmt, f"copy at step {t}")
            C = fp8_ckpt_values(layer)
            Rd = _dev_read(layer, fmt)
            recs = []
        else:
            d = tuple(np.asarray(y)[:, None] for y in x)
            ref = lowprec.split_read_verify(Rd, recs, d, "f64", group=sh.group)[:, 0]
            assert normwise_err(o, ref) <= TOL, (t, normwise_err(o, ref))
            recs.append((x[0], x[1], x[2]))
    assert layer.read_error() == 0
    say(f"  checkpoint codes rounded the other way: {[f'{f:.1e}' for f in flips]}")


def test_verify_and_commit_with_fp8_checkpoint(dev):
    """Verification reads the copy; a commit that fills the window folds the
    committed records into the fp8 checkpoint with the next epoch and
    rewrites the copy from the unrounded fold."""
    sh = W.Shape(batch=4, n_vheads=4, n_kheads=2, dim_v=16, dim_k=64, window=6, max_draft=4, dist="uniform")
    seed = 31
    say("case: fp8 checkpoint verify + commit (MXFP4 copy)")
    layer = _layer(sh, dev, read_copy="mxfp4", sr_seed=seed)
    C = set_fp8_ckpt(layer, W.initial_state_np(sh, 33, std=0.5))
    layer.refresh_read_copy()
    recs = [W.decode_inputs_np(sh, 34, t) for t in range(3)]
    for x in recs:
        layer.decode_step(*to_dev(x, dev))
    committed = [(x[0], x[1], x[2]) for x in recs]
    for r in range(6):
        T = 4
        drafts = W.draft_inputs_np(sh, 35, r, T)
        O = layer.spec_verify(*to_dev(drafts, dev)).cpu().numpy()
        ref = lowprec.split_read_verify(_dev_read(layer, "mxfp4"), committed, drafts, "f64", group=sh.group)
        assert normwise_err(O, ref) <= TOL, (r, normwise_err(O, ref))
        a_r = 3 if r % 2 == 0 else 1
        epoch = layer.fold_epochs()
        layer.commit(torch.full((sh.batch,), a_r, dtype=torch.int32, device=dev))
        committed += [(drafts[0][:, t], drafts[1][:, t], drafts[2][:, t]) for t in range(a_r)]
        if len(committed) >= sh.window:
            steps = [(a, k, v, np.zeros_like(k)) for (a, k, v) in committed]
            _, _, S_new = recurrence.decode(C, steps, group=sh.group)
            check_fp8_ckpt(layer, S_new, seed, epoch, f"commit fold in round {r}")
            _check_copy(layer, S_new, "mxfp4", f"copy after the commit fold in round {r}")
            assert np.all(layer.fold_epochs() == epoch + 1)
            C = fp8_ckpt_values(layer)
            committed = []
    assert layer.read_error() == 0


def test_refresh_and_reset_with_fp8_checkpoint(dev):
    """refresh_read_copy quantises the values the fp8 checkpoint holds (their
    fp32 products, code by code); reset zeroes a sequence's rows, scales
    included, and leaves the others."""
    sh = W.Shape(batch=3, n_vheads=2, n_kheads=2, dim_v=8, dim_k=64, window=4, dist="uniform")
    say("case: fp8 checkpoint refresh + reset")
    S0 = W.initial_state_np(sh, 43, std=2.0)
    for fmt in ("bf16", "fp8", "mxfp4"):
        layer = _layer(sh, dev, read_copy=fmt)
        C = set_fp8_ckpt(layer, S0)
        layer.refresh_read_copy()
        R, sc = quant.quantize(C.astype(np.float32), fmt)
        if fmt == "bf16":
            np.testing.assert_array_equal(layer.read_copy.view(torch.int16).cpu().numpy().view(np.uint16), R)
        elif fmt == "fp8":
            got = layer.read_copy.cpu().numpy()
            np.testing.assert_array_equal(np.where(got & 0x7F, got, 0), np.where(R & 0x7F, R, 0))
            np.testing.assert_array_equal(layer.row_scale.cpu().numpy(), sc)
        else:
            np.testing.assert_array_equal(unpack_e2m1(layer.read_copy.cpu().numpy()), R)
            np.testing.assert_array_equal(layer.row_scale.cpu().numpy(), sc)
        before = layer.ckpt.cpu().numpy()
        layer.reset(torch.tensor([1], dtype=torch.int32, device=dev))
        after = layer.ckpt.cpu().numpy()
        assert np.all(after[1] == 0) and np.array_equal(after[0], before[0]) and np.array_equal(after[2], before[2])


def test_fp8_checkpoint_non_finite_and_large_values(dev):
    """L = 1 (every step folds).  Row 0 folds to NaN everywhere: NaN codes,
    scale 1 (NaN entries are left out of the maximum).  Row 1 overflows to
    infinity in one entry (1e30 * 1e30 in fp32): its scale is infinite, the
    infinite entry stores the NaN code and its finite entries zero codes.
    Every row rounds as the oracle rounds it, code for code."""
    sh = W.Shape(batch=1, n_vheads=1, n_kheads=1, dim_v=4, dim_k=16, window=1, dist="uniform")
    say("case: fp8 checkpoint with inf and nan")
    layer = _layer(sh, dev, read_copy="fp8", sr_seed=9)
    S0 = np.zeros((1, 1, 4, 16))
    S0[0, 0, 2:] = np.linspace(-3, 3, 32).reshape(2, 16)
    C = set_fp8_ckpt(layer, S0)
    a = np.ones((1, 1), dtype=np.float32)
    k = np.zeros((1, 1, 16), dtype=np.float32)
    k[0, 0, :2] = [1e30, 1.0]
    v = np.array([[[np.nan, 1e30, 0.5, 0.25]]], dtype=np.float32)
    q = np.zeros((1, 1, 16), dtype=np.float32)
    layer.decode_step(*to_dev((a, k, v, q), dev))
    S1 = C + v[..., :, None].astype(np.float64) * k[..., None, :].astype(np.float64)
    codes, sig = fp8_ckpt_parts(layer)
    rc, rs = stochastic.checkpoint_round_fp8(S1, 9, 0)
    assert np.all(codes[0, 0, 0] == 0x7F) and sig[0, 0, 0] == 1.0
    assert np.isposinf(sig[0, 0, 1]) and codes[0, 0, 1, 0] == 0x7F
    assert np.all((codes[0, 0, 1, 1:] & 0x7F) == 0)
    np.testing.assert_array_equal(np.where(codes & 0x7F, codes, 0), np.where(rc & 0x7F, rc, 0))
    np.testing.assert_array_equal(sig, rs)
    assert np.all(layer.fold_epochs() == 1)


def test_graph_replayed_fp8_fold_draws_new_numbers(dev):
    """A decode step with L = 1 (every step folds) into an fp8 checkpoint is
    captured once and replayed from the same checkpoint and inputs: each
    replay rounds with the next epoch (the oracle's rounding of the same fold
    at epochs 1, 2, ...), so the stored codes differ between replays."""
    sh = W.Shape(batch=3, n_vheads=4, n_kheads=2, dim_v=16, dim_k=64, window=1, dist="uniform")
    seed = 29
    say("case: graph replay of an fp8 fold, epochs 1..5")
    layer = _layer(sh, dev, read_copy="mxfp4", sr_seed=seed)
    C = set_fp8_ckpt(layer, W.initial_state_np(sh, 62, std=0.5))
    ck0 = layer.ckpt.clone()
    x = W.decode_inputs_np(sh, 63, 0)
    xs = [torch.from_numpy(t).to(dev) for t in x]
    o = torch.empty((sh.batch, sh.n_vheads, sh.dim_v), device=dev)
    layer.decode_step(*xs, o)                         # warm-up: epoch 0
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.decode_step(*xs, o)
    torch.cuda.synchronize()
    a, k, v, _ = (np.asarray(t, dtype=np.float64) for t in x)
    kk = np.repeat(k, sh.group, axis=1)
    S1 = a[..., None, None] * C + v[..., :, None] * kk[..., None, :]
    got = []
    for r in range(5):
        layer.ckpt.copy_(ck0)                         # same checkpoint and inputs every replay
        g.replay()
        torch.cuda.synchronize()
        check_fp8_ckpt(layer, S1, seed, r + 1, f"replay {r}")
        assert np.all(layer.fold_epochs() == r + 2)
        got.append(fp8_ckpt_parts(layer)[0])
    for r in range(4):
        assert np.mean(got[r] != got[r + 1]) > 0.05, r
    assert layer.read_error() == 0
