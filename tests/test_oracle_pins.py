"""Pins of the fp64 oracle against results fixed by the pages and by mathematics.

Each pin computes the expected value by a route other than the oracle's own
step-by-step code:
  * alpha == 1: S_t is S_0 plus one matrix product V^T K of the stacked
    records (exact in integers);
  * constant alpha: geometric weights a^(t-j) from np.power;
  * time-varying alpha: integrating-factor form with cumulative products;
  * eq.U and eq.OT in exact rational arithmetic (brute force), which the pages
    state equal stepping the recurrence;
  * eq.O1 from a zero state.
A dropped decay, an off-by-one decay exponent, a wrong sign, a transposed
outer product or a wrong key-head mapping each fails at least one of these.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import cpu_c, exact, lowprec, quant, recurrence
from ssm_layer_decode_amd import workloads as W


def _stack_steps(sh, seed, steps):
    return [W.decode_inputs_np(sh, seed, t) for t in range(steps)]


def _expand(x, g):
    return np.repeat(x, g, axis=-2)


# --------------------------------------------------------------------- eq.R
def test_alpha_one_integer_closed_form():
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=2, dim_v=6, dim_k=5, window=16, dist="integer")
    steps = 12
    ins = _stack_steps(sh, 11, steps)
    rng = np.random.default_rng(5)
    S0 = rng.integers(-3, 4, (2, 4, 6, 5)).astype(np.float64)
    outs, kept, _ = recurrence.decode(S0, ins, group=sh.group, keep_states=range(1, steps + 1))
    K = np.stack([_expand(k, sh.group) for (_, k, _, _) in ins])      # [t][B][Hv][N]
    V = np.stack([v for (_, _, v, _) in ins])                          # [t][B][Hv][P]
    for t in range(1, steps + 1):
        # S_t = S_0 + sum_{j<=t} v_j k_j^T  as one product over the record axis
        St = S0 + np.einsum("tbhp,tbhn->bhpn", V[:t].astype(np.float64), K[:t].astype(np.float64))
        np.testing.assert_array_equal(kept[t], St)
        q = _expand(ins[t - 1][3], sh.group).astype(np.float64)
        o = np.einsum("bhpn,bhn->bhp", St, q)
        np.testing.assert_array_equal(outs[t - 1], o)


def test_constant_alpha_geometric_closed_form():
    sh = W.Shape(batch=3, n_vheads=2, n_kheads=1, dim_v=4, dim_k=7, window=16, dist="uniform")
    steps = 20
    ins = _stack_steps(sh, 3, steps)
    rng = np.random.default_rng(9)
    a_const = rng.uniform(0.5, 1.0, (3, 2)).astype(np.float32)
    ins = [(a_const, k, v, q) for (_, k, v, q) in ins]
    S0 = rng.standard_normal((3, 2, 4, 7))
    outs, kept, _ = recurrence.decode(S0, ins, group=2, keep_states=[steps])
    a = a_const.astype(np.float64)
    t = steps
    S = np.power(a, t)[..., None, None] * S0
    for j in range(1, t + 1):
        _, k, v, _ = ins[j - 1]
        w = np.power(a, t - j)
        S = S + w[..., None, None] * v.astype(np.float64)[..., :, None] * _expand(k, 2).astype(np.float64)[..., None, :]
    np.testing.assert_allclose(kept[t], S, rtol=1e-12, atol=1e-14)


def test_time_varying_alpha_integrating_factor():
    sh = W.Shape(batch=2, n_vheads=3, n_kheads=3, dim_v=5, dim_k=8, window=16, dist="uniform")
    steps = 24
    ins = _stack_steps(sh, 4, steps)
    S0 = np.random.default_rng(1).standard_normal((2, 3, 5, 8))
    outs, kept, _ = recurrence.decode(S0, ins, group=1, keep_states=range(1, steps + 1))
    A = np.cumprod(np.stack([a.astype(np.float64) for (a, _, _, _) in ins]), axis=0)   # A_t
    acc = S0.copy()
    for t in range(1, steps + 1):
        _, k, v, q = ins[t - 1]
        acc = acc + (v.astype(np.float64)[..., :, None] * k.astype(np.float64)[..., None, :]) / A[t - 1][..., None, None]
        St = A[t - 1][..., None, None] * acc
        np.testing.assert_allclose(kept[t], St, rtol=1e-10, atol=1e-12)
        o = np.einsum("bhpn,bhn->bhp", St, q.astype(np.float64))
        np.testing.assert_allclose(outs[t - 1], o, rtol=1e-9, atol=1e-11)


def test_zero_state_first_output_is_rank_one():
    """eq.O1: from a zero state o_1 = v_1 (k_1 . q_1)."""
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=2, dim_v=16, dim_k=16, window=16, dist="mamba2")
    a, k, v, q = W.decode_inputs_np(sh, 0, 0)
    outs, _, _ = recurrence.decode(np.zeros((2, 4, 16, 16)), [(a, k, v, q)], group=2)
    for b in range(2):
        for h in range(4):
            s = float(np.dot(k[b, h // 2].astype(np.float64), q[b, h // 2].astype(np.float64)))
            np.testing.assert_allclose(outs[0, b, h], s * v[b, h].astype(np.float64), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------- eq.U, eq.OT exact
DYADIC = [Fraction(1, 2), Fraction(3, 4), Fraction(7, 8), Fraction(1)]


def _rational_records(rng, n, P, N):
    recs = []
    for _ in range(n):
        a = DYADIC[rng.integers(0, len(DYADIC))]
        k = [int(x) for x in rng.integers(-3, 4, N)]
        v = [int(x) for x in rng.integers(-3, 4, P)]
        q = [int(x) for x in rng.integers(-3, 4, N)]
        recs.append((a, k, v, q))
    return recs


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_unrolled_window_equals_stepping_exactly(seed):
    """eq.U (whole window from the checkpoint) equals eq.R stepped record by
    record, exactly; and the fp64 numpy stepper reproduces it exactly (dyadic
    inputs keep every fp64 intermediate exact)."""
    rng = np.random.default_rng(seed)
    P, N, H = 3, 4, 7
    S_ckpt = [[Fraction(int(x)) for x in rng.integers(-3, 4, N)] for _ in range(P)]
    recs = _rational_records(rng, H, P, N)
    outs, states = exact.eqR_steps(S_ckpt, recs)
    for h in range(1, H + 1):
        al = [r[0] for r in recs[:h]]
        ks = [r[1] for r in recs[:h]]
        vs = [r[2] for r in recs[:h]]
        assert exact.eqU_state(S_ckpt, al, ks, vs) == states[h - 1]
        assert exact.eqU_output(S_ckpt, al, ks, vs, recs[h - 1][3]) == outs[h - 1]
    # numpy fp64 oracle on the same values (1 sequence, 1 head)
    S0 = np.array([[float(x) for x in row] for row in S_ckpt])[None, None]
    ins = [(np.array([[float(a)]], dtype=np.float32), np.array([[k]], dtype=np.float32),
            np.array([[v]], dtype=np.float32), np.array([[q]], dtype=np.float32)) for (a, k, v, q) in recs]
    o_np, kept, _ = recurrence.decode(S0, ins, keep_states=range(1, H + 1))
    for h in range(1, H + 1):
        assert np.array_equal(o_np[h - 1, 0, 0], np.array([float(x) for x in outs[h - 1]]))
        assert np.array_equal(kept[h][0, 0], np.array([[float(x) for x in row] for row in states[h - 1]]))


@pytest.mark.parametrize("h,T", [(0, 1), (0, 4), (3, 4), (5, 2), (6, 8)])
def test_output_only_chunk_equals_stepping_exactly(h, T):
    """eq.OT with D = diag(gamma_{1:h+t}) and causal W[j,t] = gamma_{j+1:h+t}
    gives each draft's output exactly; so does the numpy verify oracle."""
    rng = np.random.default_rng(100 + 10 * h + T)
    P, N = 3, 5
    S_ckpt = [[Fraction(int(x)) for x in rng.integers(-2, 3, N)] for _ in range(P)]
    committed = _rational_records(rng, h, P, N)
    drafts = _rational_records(rng, T, P, N)
    outs, states = exact.eqR_steps(S_ckpt, committed + drafts)
    # checkpoint-relative state after the committed records
    al = [r[0] for r in committed + drafts]
    ks = [r[1] for r in committed + drafts]
    vs = [r[2] for r in committed + drafts]
    qs = [r[3] for r in drafts]
    got = exact.eqOT_outputs(S_ckpt, al, ks, vs, qs, h)
    for t in range(T):
        assert got[t] == outs[h + t]
    # numpy verify from the committed state (exact for these dyadic values)
    Sc = states[h - 1] if h > 0 else S_ckpt
    Sc_np = np.array([[float(x) for x in row] for row in Sc])[None, None]
    a_d = np.array([[[float(r[0])] for r in drafts]], dtype=np.float32)
    k_d = np.array([[[r[1]] for r in drafts]], dtype=np.float32)
    v_d = np.array([[[r[2]] for r in drafts]], dtype=np.float32)
    q_d = np.array([[[r[3]] for r in drafts]], dtype=np.float32)
    O, _ = recurrence.verify(Sc_np, a_d, k_d, v_d, q_d)
    for t in range(T):
        assert np.array_equal(O[0, t, 0], np.array([float(x) for x in outs[h + t]]))


def test_verify_then_commit_equals_decoding_prefix():
    """Committing a k-prefix of verified drafts leaves the state that decoding
    only those k tokens reaches; the outputs of the drafts are the decode
    outputs ([ru] §05; [zh] method points)."""
    sh = W.Shape(batch=5, n_vheads=4, n_kheads=2, dim_v=8, dim_k=8, window=16, max_draft=4, dist="uniform")
    T = 4
    S0 = W.initial_state_np(sh, 1)
    a, k, v, q = W.draft_inputs_np(sh, 0, 0, T)
    O, states = recurrence.verify(S0, a, k, v, q, group=2)
    acc = np.array([0, 1, 2, 3, 4], dtype=np.int32)
    S_commit = recurrence.commit(states, acc)
    for b in range(5):
        ins = [(a[b:b + 1, t], k[b:b + 1, t], v[b:b + 1, t], q[b:b + 1, t]) for t in range(int(acc[b]))]
        outs, _, S_dec = recurrence.decode(S0[b:b + 1], ins, group=2)
        np.testing.assert_array_equal(S_commit[b], S_dec[0])
        for t in range(int(acc[b])):
            np.testing.assert_array_equal(O[b, t], outs[t, 0])


# ------------------------------------------------------------- C oracle
def test_c_oracle_matches_numpy_stepper():
    sh = W.with_(W.TINY, n_vheads=4, n_kheads=2)
    steps = 40
    ins = _stack_steps(sh, 0, steps)
    S0 = np.random.default_rng(3).standard_normal((sh.batch, 4, sh.dim_v, sh.dim_k))
    o_np, _, S_np = recurrence.decode(S0, ins, group=2)
    a = np.stack([x[0] for x in ins]); k = np.stack([x[1] for x in ins])
    v = np.stack([x[2] for x in ins]); q = np.stack([x[3] for x in ins])
    o_c, S_c = cpu_c.decode(S0, a, k, v, q)
    np.testing.assert_allclose(o_c, o_np, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(S_c, S_np, rtol=1e-13, atol=1e-15)


def test_outputs_are_linear_in_values_and_initial_state():
    """With decays, keys and queries fixed, eq.R's outputs and states are linear
    in (v, S_0): O(a S + b S', a v + b v') = a O(S, v) + b O(S', v').  A term
    that squares, drops or takes |.| of v or S_0 breaks it."""
    sh = W.with_(W.TINY, n_vheads=4, n_kheads=2)
    steps = 24
    rng = np.random.default_rng(11)
    ins = _stack_steps(sh, 2, steps)
    v2 = [rng.standard_normal(x[2].shape).astype(np.float32) for x in ins]
    S0 = rng.standard_normal((sh.batch, 4, sh.dim_v, sh.dim_k))
    S0b = rng.standard_normal(S0.shape)
    ca, cb = 0.75, -1.5
    mix = [(x[0], x[1], (ca * x[2].astype(np.float64) + cb * w.astype(np.float64)), x[3])
           for x, w in zip(ins, v2)]
    o1, _, S1 = recurrence.decode(S0, ins, group=2)
    o2, _, S2 = recurrence.decode(S0b, [(x[0], x[1], w, x[3]) for x, w in zip(ins, v2)], group=2)
    o3, _, S3 = recurrence.decode(ca * S0 + cb * S0b, mix, group=2)
    np.testing.assert_allclose(o3, ca * o1 + cb * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S3, ca * S1 + cb * S2, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- low precision
def test_split_path_with_identity_copy_is_the_recurrence():
    sh = W.with_(W.TINY, dist="uniform", window=5)
    steps = 23
    ins = _stack_steps(sh, 2, steps)
    S0 = W.initial_state_np(sh, 4).astype(np.float64)
    ref, kept, _ = recurrence.decode(S0, ins, keep_states=[5, 10, 15, 20])
    got, folds = lowprec.split_read_decode(S0, ins, 5, "f64", keep_folds=True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    assert sorted(folds) == [5, 10, 15, 20]
    for t in folds:
        np.testing.assert_allclose(folds[t], kept[t], rtol=1e-12, atol=1e-14)
    q_arm = lowprec.quantized_state_decode(S0, ins, "f64")
    np.testing.assert_array_equal(q_arm, ref)


def test_split_path_bf16_error_within_rounding_bound():
    """Non-flush outputs differ from eq.R only through the read copy: the
    difference is gamma_h * (deq(R) - S_ckpt) q, and each bf16 entry is within
    2^-8 relative of fl32(S_ckpt) (half an ulp of an 8-bit significand)."""
    sh = W.with_(W.TINY, dist="uniform", window=4)
    steps = 12
    ins = _stack_steps(sh, 7, steps)
    S0 = W.initial_state_np(sh, 8, std=1.0).astype(np.float64)
    ref, kept, _ = recurrence.decode(S0, ins, keep_states=[4, 8, 12])
    got, _ = lowprec.split_read_decode(S0, ins, 4, "bf16")
    ckpts = {0: S0, 4: kept[4], 8: kept[8]}
    for t in range(1, steps + 1):
        if t % 4 == 0:
            np.testing.assert_allclose(got[t - 1], ref[t - 1], rtol=1e-12, atol=1e-14)
            continue
        base = 4 * ((t - 1) // 4)
        gam = np.prod(np.stack([ins[j][0] for j in range(base, t)]).astype(np.float64), axis=0)
        q = ins[t - 1][3].astype(np.float64)
        bound = gam[..., None] * np.einsum("bhpn,bhn->bhp", np.abs(ckpts[base]) * (2.0 ** -8 + 2.0 ** -23), np.abs(q))
        assert np.all(np.abs(got[t - 1] - ref[t - 1]) <= bound * (1 + 1e-9) + 1e-15)


def test_quantized_state_arm_outputs_unrounded_state_and_feeds_rounding_back():
    """Reading r17 on hand-worked dyadic numbers (P = 1, N = 2, bf16 state).
    Step 1 from zero: alpha = 1, k = (1, 0), v = 1 + 2^-10, q = (1, 0), so
    S_1 = (1 + 2^-10, 0), which bf16 (8 significand bits) stores as (1, 0).
    The output is taken from the unrounded S_1: o_1 = 1 + 2^-10 (from the
    stored state it would be 1).  Step 2: alpha = 1/2, k = (0, 1), v = 1,
    q = (1, 1) starts from the stored (1, 0): S_2 = (1/2, 1), o_2 = 3/2
    (without the rounding fed back it would be 3/2 + 2^-11)."""
    a1, k1, v1, q1 = [[1.0]], [[[1.0, 0.0]]], [[[1.0 + 2.0 ** -10]]], [[[1.0, 0.0]]]
    a2, k2, v2, q2 = [[0.5]], [[[0.0, 1.0]]], [[[1.0]]], [[[1.0, 1.0]]]
    steps = [tuple(np.array(x, dtype=np.float64) for x in st) for st in
             ((a1, k1, v1, q1), (a2, k2, v2, q2))]
    o = lowprec.quantized_state_decode(np.zeros((1, 1, 1, 2)), steps, "bf16")
    assert o[0, 0, 0, 0] == 1.0 + 2.0 ** -10
    assert o[1, 0, 0, 0] == 1.5
    # the exact recurrence differs from the arm exactly by the fed-back rounding
    ref, _, _ = recurrence.decode(np.zeros((1, 1, 1, 2)), steps)
    assert ref[1, 0, 0, 0] == 1.5 + 2.0 ** -11 and ref[0, 0, 0, 0] == o[0, 0, 0, 0]


def test_quantized_state_error_accumulates_split_error_does_not():
    """The pages' claim about feedback ([ru] §02 and §06): rounding the stored
    state every step accumulates, rounding only the read copy does not.  Checked
    on the oracle itself with fp8 at a tiny size."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=16, dim_k=16, window=16, dist="gdn")
    steps = 256
    ins = _stack_steps(sh, 1, steps)
    S0 = np.zeros((2, 2, 16, 16))
    ref, _, _ = recurrence.decode(S0, ins)
    split, _ = lowprec.split_read_decode(S0, ins, 16, "fp8")
    qarm = lowprec.quantized_state_decode(S0, ins, "fp8")

    def err(x):
        return np.max(np.abs(x - ref), axis=(1, 2, 3)) / np.max(np.abs(ref), axis=(1, 2, 3))
    e_s, e_q = err(split), err(qarm)
    assert np.mean(e_s[128:]) < np.mean(e_q[128:])
    assert np.max(e_s[192:]) <= 2.0 * np.max(e_s[32:96]) + 1e-12


def test_split_read_bound_routine_and_oracle_path_obey_it():
    """The C bound routine equals a brute-force numpy evaluation from the
    stepper's own checkpoints, and the oracle's split path stays within it
    for both read formats (bf16: |R-S| <= 2^-8|S|; e4m3 row-scaled:
    |R-S| <= 2^-4|S| + 2^-10 amax/448)."""
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=2, dim_v=8, dim_k=16, window=5, dist="gdn")
    steps = 23
    ins = _stack_steps(sh, 8, steps)
    S0 = W.initial_state_np(sh, 2, std=0.4).astype(np.float64)
    a = np.stack([x[0] for x in ins]); k = np.stack([x[1] for x in ins])
    v = np.stack([x[2] for x in ins]); q = np.stack([x[3] for x in ins])
    A, Z = cpu_c.split_read_bound(S0, a, k, v, q, sh.window)
    truth, kept, _ = recurrence.decode(S0, ins, group=2, keep_states=range(1, steps + 1))
    ck, gam = S0, np.ones((2, 4))
    for t in range(1, steps + 1):
        gam = gam * a[t - 1].astype(np.float64)
        qq = np.repeat(q[t - 1].astype(np.float64), 2, axis=1)
        if t % sh.window == 0:
            assert np.all(A[t - 1] == 0) and np.all(Z[t - 1] == 0)
            ck, gam = kept[t], np.ones((2, 4))
            continue
        A_ref = gam[..., None] * np.einsum("bhpn,bhn->bhp", np.abs(ck), np.abs(qq))
        Z_ref = gam[..., None] * np.abs(ck).max(axis=-1) * np.abs(qq).sum(axis=-1)[..., None]
        np.testing.assert_allclose(A[t - 1], A_ref, rtol=1e-12)
        np.testing.assert_allclose(Z[t - 1], Z_ref, rtol=1e-12)
    for fmt, ur, ua in (("bf16", 2.0 ** -8, 0.0), ("fp8", 2.0 ** -4, 2.0 ** -10 / 448)):
        got, _ = lowprec.split_read_decode(S0, ins, sh.window, fmt, group=2)
        slack = 2.0 ** -22 * np.abs(truth).max(axis=-1, keepdims=True)   # fp32 rounding of S_ckpt
        assert np.all(np.abs(got - truth) <= ur * A * (1 + 2.0 ** -20) + ua * Z + slack)


def test_split_read_bound_mxfp4():
    """The oracle's MXFP4 split path stays within the same bound with E2M1's
    unit roundoff: |R-S| <= 2^-2 |S| + 2^-4 amax (half the subnormal step of a
    block, X/4, with X <= amax(block)/4 <= amax(row)/4)."""
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=2, dim_v=8, dim_k=64, window=5, dist="gdn")
    steps = 17
    ins = _stack_steps(sh, 9, steps)
    S0 = W.initial_state_np(sh, 3, std=0.4).astype(np.float64)
    a = np.stack([x[0] for x in ins]); k = np.stack([x[1] for x in ins])
    v = np.stack([x[2] for x in ins]); q = np.stack([x[3] for x in ins])
    A, Z = cpu_c.split_read_bound(S0, a, k, v, q, sh.window)
    truth, _, _ = recurrence.decode(S0, ins, group=2)
    got, _ = lowprec.split_read_decode(S0, ins, sh.window, "mxfp4", group=2)
    slack = 2.0 ** -22 * np.abs(truth).max(axis=-1, keepdims=True)
    assert np.all(np.abs(got - truth) <= 2.0 ** -2 * A * (1 + 2.0 ** -20) + 2.0 ** -4 * Z + slack)
    # and the copy is not trivially exact: the error is a visible share of the bound
    assert np.max(np.abs(got - truth)) > 1e-3 * np.max(2.0 ** -2 * A + 2.0 ** -4 * Z)


def test_split_read_verify_reduces_to_stepping():
    """With the identity copy the split verify equals stepping eq.R through the
    committed records and then the drafts; with a real copy, and no flush
    inside the window, draft t's output equals the split decode output of the
    same token (both read the same copy of the same checkpoint)."""
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=2, dim_v=6, dim_k=32, window=12, max_draft=4, dist="uniform")
    S0 = W.initial_state_np(sh, 5, std=0.5).astype(np.float64)
    recs = _stack_steps(sh, 6, 3)
    a, k, v, q = W.draft_inputs_np(sh, 7, 0, 4)
    got = lowprec.split_read_verify(S0, [(x[0], x[1], x[2]) for x in recs], (a, k, v, q), "f64", group=2)
    _, _, S_h = recurrence.decode(S0, recs, group=2)
    ref, _ = recurrence.verify(S_h, a, k, v, q, group=2)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13 * np.abs(ref).max())
    steps = recs + [(a[:, t], k[:, t], v[:, t], q[:, t]) for t in range(4)]
    for fmt in ("bf16", "fp8", "mxfp4"):
        ver = lowprec.split_read_verify(S0, [(x[0], x[1], x[2]) for x in recs], (a, k, v, q), fmt, group=2)
        dec, _ = lowprec.split_read_decode(S0, steps, sh.window, fmt, group=2)
        np.testing.assert_allclose(ver, np.moveaxis(dec[3:], 0, 1), rtol=1e-12, atol=1e-13 * np.abs(ref).max())


@pytest.mark.parametrize("h0,T", [(0, 37), (5, 3), (5, 11), (0, 16), (3, 29)])
def test_prefill_equals_token_by_token_decoding(h0, T):
    """Prefill's outputs are eq.R's (stepped here with zero queries for the
    buffered records, whose outputs are not returned); its new checkpoint is
    the state decoding reaches at the last window boundary; the buffer model
    keeps the last (h0 + T) mod L records."""
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=2, dim_v=5, dim_k=6, window=8, max_draft=0, dist="uniform")
    L = sh.window
    S0 = W.initial_state_np(sh, 3).astype(np.float64)
    buf = _stack_steps(sh, 4, h0)
    a, k, v, q = W.draft_inputs_np(sh, 5, 0, T)
    O, S_new, folds = recurrence.prefill(S0, [(x[0], x[1], x[2]) for x in buf], (a, k, v, q), L, group=2)
    steps = [(x[0], x[1], x[2], np.zeros_like(x[1])) for x in buf] + [(a[:, t], k[:, t], v[:, t], q[:, t]) for t in range(T)]
    ref, kept, _ = recurrence.decode(S0, steps, group=2, keep_states=range(1, len(steps) + 1))
    np.testing.assert_allclose(O, np.moveaxis(ref[h0:], 0, 1), rtol=1e-12, atol=1e-13)
    assert folds == (h0 + T) // L
    if folds:
        np.testing.assert_allclose(S_new, kept[folds * L], rtol=1e-12, atol=1e-13)
    else:
        np.testing.assert_array_equal(S_new, S0)
    from oracle import bookkeeping
    bm = bookkeeping.BufferModel(2, 4, 2, 5, 6, L)
    for x in buf:
        bm.decode(x[0], x[1], x[2])
    f = bm.prefill(a, k, v)
    assert np.all(f == folds) and np.all(bm.count == (h0 + T) % L)
    hp = (h0 + T) % L
    if hp:
        np.testing.assert_array_equal(bm.vbuf[:, :, :hp], np.moveaxis(v[:, T - hp:], 1, 2))
