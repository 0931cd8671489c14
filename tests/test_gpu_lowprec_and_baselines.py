"""GPU parity of the read copies and of the in-run baselines.

* Read-copy codes made from the same fp32 checkpoint values must equal the
  oracle's encoders bit for bit (bf16 RNE; e4m3 RNE with per-row scale
  fl32(amax/448), apart from the sign of a zero code; MXFP4 E2M1 codes and
  E8M0 block exponents exactly, zero signs included).
* The split-precision decode must keep an fp32 checkpoint bit-identical to
  the fp32-only run (the copy never feeds the recurrence) and its outputs must
  stay within the copy's rounding bound of the fp64 recurrence.
* Conventional decode (fp32 state) within 1e-5 of the oracle; snapshot verify
  and commit within 1e-5; the quantised-state arms close to the oracle's arm.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import cpu_c, lowprec, quant, recurrence
from ssm_layer_decode_amd import workloads as W
from tests.helpers import matrix_err, normwise_err, say, to_dev, unpack_e2m1

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
    return ReplaySSM(LayerConfig.of(sh, **kw), device=dev)


def _wild_state(sh, seed):
    """fp32 state with row scales spread over many binades, zero rows, ties."""
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k))
    S *= np.exp(rng.uniform(-12, 8, (sh.batch, sh.n_vheads, sh.dim_v, 1)))
    S = S.astype(np.float32)
    S[0, 0, 1] = 0.0
    S[0, 0, 2, :4] = [448.0, -448.0, 1.0, 0.0]        # exact values within a row
    return S


def _codes_equal_up_to_zero_sign(a, b):
    a = np.asarray(a).astype(np.int64)
    b = np.asarray(b).astype(np.int64)
    za = (a & 0x7F) == 0
    zb = (b & 0x7F) == 0
    return np.array_equal(np.where(za, 0, a), np.where(zb, 0, b)) and np.array_equal(za, zb)


@pytest.mark.parametrize("N", [16, 128])
def test_refresh_codes_bit_exact(dev, N):
    sh = W.Shape(batch=2, n_vheads=3, n_kheads=3, dim_v=12, dim_k=N, window=4, dist="uniform")
    S = _wild_state(sh, N)
    for fmt in ("bf16", "fp8"):
        say(f"case: refresh codes {fmt} N={N}")
        layer = _layer(sh, dev, read_copy=fmt)
        layer.ckpt.copy_(torch.from_numpy(S))
        layer.refresh_read_copy()
        R_ref, sig_ref = quant.quantize(S, fmt)
        if fmt == "bf16":
            got = layer.read_copy.view(torch.int16).cpu().numpy().view(np.uint16)
            np.testing.assert_array_equal(got, R_ref)
        else:
            got = layer.read_copy.cpu().numpy()
            sig = layer.row_scale.cpu().numpy()
            np.testing.assert_array_equal(sig, sig_ref)
            assert _codes_equal_up_to_zero_sign(got, R_ref)


def test_fp8_conversion_matches_encoder_on_grid_and_ties(dev):
    """The hardware e4m3 conversion used for the copy rounds like the OCP
    encoder: checked on every representable value, every midpoint and values
    around them (a row whose amax is 448 gives scale 1, so the codes are the
    plain conversion of the values)."""
    codes = np.arange(256, dtype=np.uint8)
    vals = quant.e4m3_decode(codes)
    pos = np.unique(np.abs(vals[np.isfinite(vals)]))
    mids = (pos[1:] + pos[:-1]) / 2
    eps = np.nextafter(mids.astype(np.float32), np.float32(np.inf)) - mids.astype(np.float32)
    xs = np.concatenate([pos, mids, mids + eps, mids - eps, -pos, -mids]).astype(np.float32)
    N = 128
    rows = -(-xs.size // (N - 1))
    S = np.zeros((rows, N), dtype=np.float32)
    flat = np.zeros(rows * (N - 1), dtype=np.float32)
    flat[:xs.size] = xs
    S[:, 1:] = flat.reshape(rows, N - 1)
    S[:, 0] = 448.0                               # fixes every row scale at exactly 1
    P = 4 * (-(-rows // 4))
    Sp = np.zeros((P, N), dtype=np.float32)
    Sp[:rows] = S
    Sp[rows:, 0] = 448.0
    sh = W.Shape(batch=1, n_vheads=1, n_kheads=1, dim_v=P, dim_k=N, window=4, dist="uniform")
    layer = _layer(sh, dev, read_copy="fp8")
    layer.ckpt.copy_(torch.from_numpy(Sp[None, None]))
    layer.refresh_read_copy()
    sig = layer.row_scale.cpu().numpy()[0, 0]
    assert np.all(sig == 1.0)
    got = layer.read_copy.cpu().numpy()[0, 0]
    ref = quant.e4m3_encode(Sp)
    assert _codes_equal_up_to_zero_sign(got, ref)


@pytest.mark.parametrize("N", [32, 64, 128, 256])
def test_mxfp4_refresh_codes_bit_exact(dev, N):
    sh = W.Shape(batch=2, n_vheads=3, n_kheads=3, dim_v=12, dim_k=N, window=4, dist="uniform")
    S = _wild_state(sh, 100 + N)
    S[1, 2, 3, N // 2:] = -0.0                        # a block of negative zeros
    S[1, 2, 4, :32] *= 2.0 ** -100                    # a block near the bottom of the E8M0 range
    S[1, 1, 5, :32] = (S[1, 1, 5, :32] * 2.0 ** -140).astype(np.float32)   # below it: exponent clamped to -127
    say(f"case: refresh codes mxfp4 N={N}")
    layer = _layer(sh, dev, read_copy="mxfp4")
    layer.ckpt.copy_(torch.from_numpy(S))
    layer.refresh_read_copy()
    codes, sc = quant.quantize(S, "mxfp4")
    np.testing.assert_array_equal(unpack_e2m1(layer.read_copy.cpu().numpy()), codes)
    np.testing.assert_array_equal(layer.row_scale.cpu().numpy(), sc)


def test_mxfp4_conversion_grid_and_ties(dev):
    """Every E2M1 magnitude, every midpoint (a tie) and the fp32 neighbours of
    each midpoint, both signs, in blocks whose amax is 6 (so X = 1 and the codes
    are the plain E2M1 rounding of the values)."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
    mids = (mags[1:] + mags[:-1]) / 2
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    xs = np.concatenate([mags, mids, up, dn, np.float32([5.999, 6.0, 7.9])])
    xs = np.concatenate([xs, -xs]).astype(np.float32)
    per = 31                                          # entry 0 of each block holds 6
    nb = -(-xs.size // per)
    blocks = np.zeros((nb, 32), dtype=np.float32)
    flat = np.zeros(nb * per, dtype=np.float32)
    flat[:xs.size] = xs
    blocks[:, 1:] = flat.reshape(nb, per)
    blocks[:, 0] = 6.0
    N = 128
    rows = -(-nb // (N // 32))
    P = 4 * (-(-rows // 4))
    S = np.zeros((P * N // 32, 32), dtype=np.float32)
    S[:, 0] = 6.0
    S[:nb] = blocks
    S = S.reshape(P, N)
    sh = W.Shape(batch=1, n_vheads=1, n_kheads=1, dim_v=P, dim_k=N, window=4, dist="uniform")
    layer = _layer(sh, dev, read_copy="mxfp4")
    layer.ckpt.copy_(torch.from_numpy(S[None, None]))
    layer.refresh_read_copy()
    assert np.all(layer.row_scale.cpu().numpy() == 127)
    got = unpack_e2m1(layer.read_copy.cpu().numpy())[0, 0]
    np.testing.assert_array_equal(got, quant.e2m1_encode(S))


def _copy_codes_equal(layer, C, fmt):
    """The read copy the kernel wrote must be Q(C) bit for bit, C the fp32
    checkpoint it stored from the same fold (e4m3: up to the sign of zero)."""
    R_ref, sc_ref = quant.quantize(C.astype(np.float32), fmt)
    if fmt == "bf16":
        np.testing.assert_array_equal(layer.read_copy.view(torch.int16).cpu().numpy().view(np.uint16), R_ref)
    elif fmt == "fp8":
        assert _codes_equal_up_to_zero_sign(layer.read_copy.cpu().numpy(), R_ref)
        np.testing.assert_array_equal(layer.row_scale.cpu().numpy(), sc_ref)
    else:
        np.testing.assert_array_equal(unpack_e2m1(layer.read_copy.cpu().numpy()), R_ref)
        np.testing.assert_array_equal(layer.row_scale.cpu().numpy(), sc_ref)


def _dev_copy(layer, fmt):
    """Dequantised read copy held by the layer (float64)."""
    if fmt == "bf16":
        return layer.read_copy.float().cpu().numpy().astype(np.float64)
    R = layer.read_copy.cpu().numpy()
    if fmt == "mxfp4":
        R = unpack_e2m1(R)
    return quant.dequantize(R, layer.row_scale.cpu().numpy(), fmt)


def _split_run_against_own_state(dev, sh, plain, split, S0, ins, fmt, truth, ur, ua, A, Z, in_dtype="f32"):
    """Step plain and split layers together.  After every fold the oracle
    restarts from the checkpoint the GPU stored, so every output is compared
    at the fp32 tolerance with the oracle's split path over the same
    checkpoint and copy:
      * fold: stored checkpoint = eq.R from the previous stored checkpoint
        through the window (1e-5), copy codes = Q(stored checkpoint) exactly,
        output = S_new q (1e-5);
      * non-flush: o = gamma deq(R) q + sum_j gamma_{j+1:h} v_j (k_j . q)
        with R = Q(stored checkpoint) (lowprec.split_read_verify, one draft),
        1e-5.
    Also: the split run's fp32 checkpoint equals the fp32-only run's bit for
    bit, fp32-only outputs are within 1e-5 of the fp64 recurrence, and split
    outputs within the copy's rounding bound of it."""
    C = S0.astype(np.float32).astype(np.float64)          # stored checkpoint at the last fold
    recs = []                                             # (alpha, k, v) since that fold
    worst = 0.0
    for t, x in enumerate(ins, start=1):
        o_s = split.decode_step(*to_dev(x, dev, in_dtype)).cpu().numpy()
        o_p = plain.decode_step(*to_dev(x, dev, in_dtype)).cpu().numpy()
        np.testing.assert_array_equal(split.ckpt.cpu().numpy(), plain.ckpt.cpu().numpy())
        assert normwise_err(o_p, truth[t - 1]) <= TOL
        bound = ur * A[t - 1] * (1 + 1e-6) + ua * Z[t - 1] + TOL * np.abs(truth[t - 1]).max(axis=-1, keepdims=True)
        assert np.all(np.abs(o_s - truth[t - 1]) <= bound), (t, np.max(np.abs(o_s - truth[t - 1]) / bound))
        if t % sh.window == 0:
            steps = [(a, k, v, np.zeros_like(k)) for (a, k, v) in recs] + [x]
            o_ref, _, S_new = recurrence.decode(C, steps, group=sh.group)
            e = normwise_err(o_s, o_ref[-1])
            C = split.ckpt.cpu().numpy().astype(np.float64)
            assert matrix_err(C, S_new) <= TOL, t
            _copy_codes_equal(split, C, fmt)
            recs = []
        else:
            d = tuple(np.asarray(y)[:, None] for y in x)
            ref = lowprec.split_read_verify(C, recs, d, fmt, group=sh.group)[:, 0]
            e = normwise_err(o_s, ref)
            recs.append((x[0], x[1], x[2]))
        assert e <= TOL, (t, e)
        worst = max(worst, e)
    return worst


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_split_precision_decode(dev, fmt):
    sh = W.Shape(batch=3, n_vheads=4, n_kheads=2, dim_v=16, dim_k=32, window=4, dist="uniform")
    steps = 26
    S0 = W.initial_state_np(sh, 7, std=0.5)
    say(f"case: split precision {fmt}")
    plain = _layer(sh, dev)
    split = _layer(sh, dev, read_copy=fmt)
    for l in (plain, split):
        l.ckpt.copy_(torch.from_numpy(S0))
    split.refresh_read_copy()
    ins = [W.decode_inputs_np(sh, 3, t) for t in range(steps)]
    truth, _, _ = recurrence.decode(S0, ins, group=sh.group)
    # elementwise read-error bound (unit roundoff u_rel of the format relative
    # to |S_ckpt||q|, u_abs of the row amax times sum|q|, decayed by gamma)
    ur, ua = {"bf16": (2.0 ** -8, 0.0), "fp8": (2.0 ** -4, 2.0 ** -10 / 448),
              "mxfp4": (2.0 ** -2, 2.0 ** -4)}[fmt]
    st = np.stack
    A, Z = cpu_c.split_read_bound(S0, st([x[0] for x in ins]), st([x[1] for x in ins]),
                                  st([x[2] for x in ins]), st([x[3] for x in ins]), sh.window)
    worst = _split_run_against_own_state(dev, sh, plain, split, S0, ins, fmt, truth, ur, ua, A, Z)
    say(f"  worst normwise error against the oracle fed the stored checkpoint: {worst:.2e}")
    assert split.read_error() == 0


def _conv_state(sh, dev, fmt, S0):
    if fmt == "f32":
        return torch.from_numpy(S0.astype(np.float32)).to(dev), None
    if fmt == "bf16":
        return torch.from_numpy(S0.astype(np.float32)).to(dev).to(torch.bfloat16), None
    codes, sig = quant.quantize_rows_fp8(S0.astype(np.float32))
    return torch.from_numpy(codes).to(dev), torch.from_numpy(sig).to(dev)


@pytest.mark.parametrize("N,in_dtype,hvpt", [(16, "f32", 0), (64, "bf16", 1), (128, "f32", 2)])
def test_conventional_decode_fp32(dev, N, in_dtype, hvpt):
    from ssm_layer_decode_amd.replayssm import LayerConfig, convssm_decode_step
    sh = W.Shape(batch=3, n_vheads=4, n_kheads=2, dim_v=20, dim_k=N, window=4, in_dtype=in_dtype,
                 dist="uniform")
    say(f"case: conventional decode N={N} {in_dtype}")
    cfg = LayerConfig.of(sh, heads_per_tile=hvpt)
    S0 = W.initial_state_np(sh, 1, std=0.3)
    state, _ = _conv_state(sh, dev, "f32", S0)
    S = S0.astype(np.float64)
    o = torch.empty((3, 4, 20), device=dev)
    for t in range(18):
        x = W.decode_inputs_np(sh, 2, t)
        a, k, v, q = to_dev(x, dev, in_dtype)
        convssm_decode_step(cfg, state, None, "f32", a, k, v, q, o)
        S, o_ref = recurrence.eqR_step(S, *x, sh.group)
        assert normwise_err(o.cpu().numpy(), o_ref) <= TOL
    assert matrix_err(state.cpu().numpy(), S) <= TOL


def _state_values(state, scale, fmt):
    """Dequantised stored state of the conventional arm (float64)."""
    if fmt == "bf16":
        return state.float().cpu().numpy().astype(np.float64)
    return quant.dequantize_rows_fp8(state.cpu().numpy(), scale.cpu().numpy())


@pytest.mark.parametrize("fmt", ["bf16", "fp8"])
def test_conventional_quantized_state_arm(dev, fmt):
    """The fully quantised comparison arm, one step at a time from the state
    the GPU stored: with D = deq(stored state), the step computes
    S = alpha D + v k^T; its output must be S q at 1e-5 (reading r17: the
    output comes from the unrounded in-register state) and the stored result
    must be Q(S), the oracle's quantiser applied to the fp32 value of S.  The
    kernel's fp32 S may differ from fl32 of the oracle's fp64 S by an ulp,
    so a code may land on the other side of a rounding threshold: such
    entries must be rare and one quantisation step away.  Over 96 steps the
    arm's error against the fp64 recurrence must also track the oracle arm's."""
    from ssm_layer_decode_amd.replayssm import LayerConfig, convssm_decode_step
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=16, dim_k=32, window=16, dist="gdn")
    say(f"case: quantised-state arm {fmt}")
    cfg = LayerConfig.of(sh)
    steps = 96
    S0 = np.zeros((2, 2, 16, 32))
    state, scale = _conv_state(sh, dev, fmt, S0)
    ins = [W.decode_inputs_np(sh, 5, t) for t in range(steps)]
    arm = lowprec.quantized_state_decode(S0, ins, fmt)
    truth, _, _ = recurrence.decode(S0, ins)
    o = torch.empty((2, 2, 16), device=dev)
    got, flips = [], 0
    for x in ins:
        D = _state_values(state, scale, fmt)
        convssm_decode_step(cfg, state, scale, fmt, *to_dev(x, dev), o)
        got.append(o.cpu().numpy())
        S, o_ref = recurrence.eqR_step(D, *x)
        assert normwise_err(got[-1], o_ref) <= TOL, normwise_err(got[-1], o_ref)
        codes, sig = quant.quantize(S, fmt)                  # Q(fl32(S)) by the oracle's encoders
        if fmt == "bf16":
            g = state.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
            r = codes.astype(np.int64)
            gm, rm, gs, rs = g & 0x7FFF, r & 0x7FFF, g >> 15, r >> 15
        else:
            # fp32 fma(a, x, v k) vs fl32 of the fp64 update: the row maximum, and the
            # scale amax / 448 with it, may differ by an ulp or two
            np.testing.assert_allclose(scale.cpu().numpy(), sig, rtol=2.0 ** -20, atol=0)
            g = state.cpu().numpy().astype(np.int64)
            r = codes.astype(np.int64)
            gm, rm, gs, rs = g & 0x7F, r & 0x7F, g >> 7, r >> 7
        diff = (gm != rm) | ((gs != rs) & (gm != 0))
        # one code apart (adjacent magnitudes of one sign, or +-0 and the smallest value)
        assert np.all(np.abs(gm - rm)[diff] == 1) and np.all(((gs == rs) | (gm == 0) | (rm == 0))[diff])
        flips += int(diff.sum())
    n = steps * S0.size
    say(f"  stored codes one step off the oracle's quantiser: {flips} of {n}")
    assert flips <= max(8, 1e-3 * n)
    got = np.stack(got)
    e_arm = np.array([normwise_err(arm[t], truth[t]) for t in range(steps)])
    e_gpu = np.array([normwise_err(got[t], truth[t]) for t in range(steps)])
    assert np.mean(e_gpu) <= 2 * np.mean(e_arm) + 1e-6


@pytest.mark.parametrize("hvpt", [1, 2])
def test_snapshot_verify_commit(dev, hvpt):
    from ssm_layer_decode_amd.replayssm import LayerConfig, convssm_commit, convssm_spec_verify
    sh = W.Shape(batch=5, n_vheads=4, n_kheads=2, dim_v=16, dim_k=32, window=16, max_draft=4,
                 dist="uniform")
    say(f"case: snapshot verify hvpt={hvpt}")
    cfg = LayerConfig.of(sh, heads_per_tile=hvpt)
    ring = sh.max_draft + 1
    S0 = W.initial_state_np(sh, 3)
    states = torch.zeros((5, ring, 4, 16, 32), device=dev)
    states[:, 0] = torch.from_numpy(S0).to(dev)
    cur = torch.zeros(5, dtype=torch.int32, device=dev)
    err = torch.zeros(4, dtype=torch.int32, device=dev)
    S = S0.astype(np.float64)
    for r in range(12):
        T = 4 if r % 3 else 2
        a, k, v, q = W.draft_inputs_np(sh, 0, r, T)
        o = torch.empty((5, T, 4, 16), device=dev)
        convssm_spec_verify(cfg, states, cur, T, *to_dev((a, k, v, q), dev), o)
        O_ref, st = recurrence.verify(S, a, k, v, q, sh.group)
        assert normwise_err(o.cpu().numpy(), O_ref) <= TOL
        acc = W.accepted_np(5, T, 9, r)
        convssm_commit(cfg, cur, torch.from_numpy(acc).to(dev), T, err)
        S = recurrence.commit(st, acc)
        c = cur.cpu().numpy()
        sel = states.cpu().numpy()[np.arange(5), c]
        assert matrix_err(sel, S) <= TOL
    assert int(err.cpu()[0]) == 0


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("hvpt", [2, 4])
def test_split_precision_multi_group_tiles(dev, fmt, hvpt):
    """Read copies with tiles of several key groups: fp32 checkpoint identical
    to the fp32-only run, outputs at 1e-5 of the oracle's split path fed the
    stored checkpoint, copy codes exact."""
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=4, dim_v=16, dim_k=64, window=4, dist="uniform")
    say(f"case: split precision {fmt} hvpt={hvpt}")
    S0 = W.initial_state_np(sh, 9, std=0.5)
    plain = _layer(sh, dev, heads_per_tile=hvpt)
    split = _layer(sh, dev, read_copy=fmt, heads_per_tile=hvpt)
    for l in (plain, split):
        l.ckpt.copy_(torch.from_numpy(S0))
    split.refresh_read_copy()
    ins = [W.decode_inputs_np(sh, 4, t) for t in range(14)]
    truth, _, _ = recurrence.decode(S0, ins, group=sh.group)
    ur, ua = {"bf16": (2.0 ** -8, 0.0), "fp8": (2.0 ** -4, 2.0 ** -10 / 448),
              "mxfp4": (2.0 ** -2, 2.0 ** -4)}[fmt]
    st = np.stack
    A, Z = cpu_c.split_read_bound(S0, st([x[0] for x in ins]), st([x[1] for x in ins]),
                                  st([x[2] for x in ins]), st([x[3] for x in ins]), sh.window)
    _split_run_against_own_state(dev, sh, plain, split, S0, ins, fmt, truth, ur, ua, A, Z)
    assert split.read_error() == 0


@pytest.mark.parametrize("fmt,T", [("bf16", 8), ("fp8", 8), ("mxfp4", 4)])
def test_spec_verify_reads_copy_largest_dims(dev, fmt, T):
    """P = N = 256 with a 16-record window: verification reads the copy of the
    largest supported state rows (MXFP4 at T = 4: its staged queries for 8
    drafts would not fit in shared memory)."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=256, dim_k=256, window=16, max_draft=T,
                 dist="uniform")
    say(f"case: verify with {fmt} copy at P = N = 256, T = {T}")
    S0 = W.initial_state_np(sh, 14, std=0.5)
    layer = _layer(sh, dev, read_copy=fmt)
    layer.ckpt.copy_(torch.from_numpy(S0))
    layer.refresh_read_copy()
    recs = [W.decode_inputs_np(sh, 15, t) for t in range(5)]
    for x in recs:
        layer.decode_step(*to_dev(x, dev))
    drafts = W.draft_inputs_np(sh, 16, T, T)
    O = layer.spec_verify(*to_dev(drafts, dev)).cpu().numpy()
    ref = lowprec.split_read_verify(S0.astype(np.float64), [(x[0], x[1], x[2]) for x in recs], drafts,
                                    fmt, group=sh.group)
    assert normwise_err(O, ref) <= TOL, normwise_err(O, ref)
    layer.commit(torch.zeros(sh.batch, dtype=torch.int32, device=dev))
    assert layer.read_error() == 0


@pytest.mark.parametrize("fmt,hvpt", [("bf16", 1), ("fp8", 2), ("fp8", 4), ("mxfp4", 1), ("mxfp4", 2),
                                      ("mxfp4", 4)])
def test_spec_verify_reads_copy(dev, fmt, hvpt):
    """Verification on the split-precision path reads the copy of the
    checkpoint.  No flush happens before the verify, so the copy is the
    refresh of the given fp32 checkpoint (bit-exact, tested above) and the
    drafts' outputs must match the oracle's split verify to fp32 accuracy;
    the fp32 checkpoint is left untouched."""
    sh = W.Shape(batch=3, n_vheads=4, n_kheads=2, dim_v=16, dim_k=64, window=8, max_draft=4,
                 dist="uniform")
    say(f"case: verify with {fmt} copy hvpt={hvpt}")
    S0 = W.initial_state_np(sh, 11, std=0.5)
    layer = _layer(sh, dev, read_copy=fmt, heads_per_tile=hvpt)
    layer.ckpt.copy_(torch.from_numpy(S0))
    layer.refresh_read_copy()
    recs = [W.decode_inputs_np(sh, 12, t) for t in range(3)]
    for x in recs:
        layer.decode_step(*to_dev(x, dev))
    for T in (4, 2):
        drafts = W.draft_inputs_np(sh, 13, T, T)
        O = layer.spec_verify(*to_dev(drafts, dev)).cpu().numpy()
        ref = lowprec.split_read_verify(S0.astype(np.float64), [(x[0], x[1], x[2]) for x in recs], drafts,
                                        fmt, group=sh.group)
        assert normwise_err(O, ref) <= TOL, (T, normwise_err(O, ref))
        layer.commit(torch.zeros(sh.batch, dtype=torch.int32, device=dev))
    np.testing.assert_array_equal(layer.ckpt.cpu().numpy(), S0.astype(np.float32))
    assert layer.read_error() == 0


def test_chunked_read_probe_indexing(dev):
    """The ceiling probe used by the bench: workgroup c reads 32 KiB chunk c and
    stores, per thread t < write_bytes/16, the xor of the 8 items it loaded
    (items c*2048 + t + 256 u)."""
    import torch
    from ssm_layer_decode_amd.probes import rssm_probe_read_chunked
    chunks, wb = 5, 1024
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2 ** 32, chunks * 8192, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).to(dev)
    dst = torch.zeros(chunks * wb // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    say(f"probe_read_chunked: {chunks} chunks, {wb} B writes")
    rssm_probe_read_chunked(src, dst, wb, sink)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(chunks, wb // 16, 4)
    items = words.reshape(chunks, 8, 256, 4)                 # [chunk][u][thread][word]
    acc = np.bitwise_xor.reduce(np.bitwise_xor.reduce(items, axis=3), axis=1)   # [chunk][thread]
    for w in range(4):
        np.testing.assert_array_equal(got[:, :, w], acc[:, : wb // 16])


@pytest.mark.parametrize("N,P,g,L,in_dtype,fmt", [
    (128, 64, 1, 16, "f32", "mxfp4"),      # the Mamba-2 serving head shape, two key groups per tile
    (128, 64, 1, 16, "f32", "fp8"),
    (128, 128, 2, 16, "bf16", "bf16"),     # two heads of one key group
    (128, 128, 4, 6, "bf16", "fp8"),       # GDN-like grouping
    (64, 20, 1, 5, "f32", "fp8"),          # rows not a multiple of a pass
    (64, 128, 4, 2, "bf16", "mxfp4"),      # one buffered record before each fold
    (128, 4, 2, 3, "f32", "bf16"),         # four rows per head
    (64, 64, 1, 16, "bf16", "mxfp4"),
    (128, 64, 16, 16, "f32", "mxfp4"),     # keys shared by 16 value heads (grouped Mamba-2 keys)
    (128, 64, 16, 16, "f32", "fp8"),
])
def test_two_head_tiles(dev, N, P, g, L, in_dtype, fmt):
    """Tiles of two value heads with a read copy (MXFP4 copies and fp8 copies
    of heads of at most 64 rows take the decode whose non-flush steps give each
    head 128 threads of its own; the others the tile-wide decode): outputs at
    1e-5 of the oracle fed the stored checkpoint, copy codes exact, buffers
    appended as the oracle's buffer model, over several windows."""
    from oracle import bookkeeping
    from tests.helpers import np_bits, raw_bits
    sh = W.Shape(batch=3, n_vheads=2 * g, n_kheads=2, dim_v=P, dim_k=N, window=L, in_dtype=in_dtype,
                  dist="uniform")
    say(f"case: two-head tiles N={N} P={P} g={g} L={L} {in_dtype} {fmt}")
    S0 = W.initial_state_np(sh, 17, std=0.5)
    plain = _layer(sh, dev, heads_per_tile=2)
    split = _layer(sh, dev, read_copy=fmt, heads_per_tile=2)
    assert split.tiles == sh.n_vheads // 2
    for l in (plain, split):
        l.ckpt.copy_(torch.from_numpy(S0))
    split.refresh_read_copy()
    steps = 2 * L + 3
    ins = [W.decode_inputs_np(sh, 18, t) for t in range(steps)]
    bm = bookkeeping.BufferModel(sh.batch, sh.n_vheads, sh.n_kheads, P, N, L, store_dtype=np.float32)
    truth, _, _ = recurrence.decode(S0, ins, group=sh.group)
    ur, ua = {"bf16": (2.0 ** -8, 0.0), "fp8": (2.0 ** -4, 2.0 ** -10 / 448),
              "mxfp4": (2.0 ** -2, 2.0 ** -4)}[fmt]
    st = np.stack
    A, Z = cpu_c.split_read_bound(S0, st([x[0] for x in ins]), st([x[1] for x in ins]),
                                  st([x[2] for x in ins]), st([x[3] for x in ins]), L)
    worst = _split_run_against_own_state(dev, sh, plain, split, S0, ins, fmt, truth, ur, ua, A, Z,
                                         in_dtype=in_dtype)
    for x in ins:
        bm.decode(x[0], x[1], x[2])
    h = steps % L
    np.testing.assert_array_equal(split.count.cpu().numpy(), np.full((sh.batch, split.tiles), h))
    np.testing.assert_array_equal(raw_bits(split.kbuf)[:, :, :h], np_bits(bm.kbuf[:, :, :h], in_dtype))
    np.testing.assert_array_equal(raw_bits(split.vbuf)[:, :, :h], np_bits(bm.vbuf[:, :, :h], in_dtype))
    np.testing.assert_array_equal(split.abuf.cpu().numpy()[:, :, :h], bm.abuf[:, :, :h])
    say(f"  worst normwise error against the oracle fed the stored checkpoint: {worst:.2e}")
    assert split.read_error() == 0
