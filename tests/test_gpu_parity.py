"""GPU parity of the ReplaySSM kernels against the fp64 oracle, through the C ABI.

Tolerances (stated before measuring): outputs and checkpoints of the fp32 paths
within a normwise relative error of 1e-5 of the fp64 oracle (per output vector,
per P x N checkpoint matrix); buffer contents, pointers and the error word
bit-exact; integer inputs with alpha = 1 bit-exact.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import recurrence
from oracle.bookkeeping import BufferModel
from ssm_layer_decode_amd import workloads as W
from tests.helpers import matrix_err, normwise_err, np_bits, raw_bits, say, to_dev

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ssm_layer_decode_amd import _lib
    _lib.load()                       # fails loudly if the library is missing
    return torch.device("cuda:0")


def _layer(sh, dev, **kw):
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    return ReplaySSM(LayerConfig.of(sh, **kw), device=dev)


def _model(sh):
    dt = np.uint16 if sh.in_dtype == "bf16" else np.float32
    return BufferModel(sh.batch, sh.n_vheads, sh.n_kheads, sh.dim_v, sh.dim_k, sh.window,
                       sh.max_draft, store_dtype=dt)


def _check_buffers(layer, model, sh):
    counts = layer.count.cpu().numpy()
    assert np.all(counts == model.count[:, None]), (counts, model.count)
    kb, vb, ab = raw_bits(layer.kbuf), raw_bits(layer.vbuf), layer.abuf.cpu().numpy()
    for b in range(sh.batch):
        h = int(model.count[b])
        assert kb[b, :, :h].tobytes() == model.kbuf[b, :, :h].tobytes()
        assert vb[b, :, :h].tobytes() == model.vbuf[b, :, :h].tobytes()
        assert ab[b, :, :h].tobytes() == model.abuf[b, :, :h].tobytes()


def run_decode(sh, steps, dev, seed=0, S0=None, check_every=1, tol=TOL, exact=False, **kw):
    """Decode `steps` steps on the GPU and step the oracle alongside."""
    layer = _layer(sh, dev, **kw)
    g = sh.group
    S = np.zeros((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k))
    if S0 is not None:
        layer.ckpt.copy_(torch.from_numpy(S0.astype(np.float32)))
        S = S0.astype(np.float32).astype(np.float64)
    model = _model(sh)
    worst_o = worst_s = 0.0
    nflush = 0
    for t in range(1, steps + 1):
        a, k, v, q = W.decode_inputs_np(sh, seed, t - 1)
        o = layer.decode_step(*to_dev((a, k, v, q), dev, sh.in_dtype))
        S, o_ref = recurrence.eqR_step(S, a, k, v, q, g)
        folded = model.decode(a, np_bits(k, sh.in_dtype), np_bits(v, sh.in_dtype))
        got = o.cpu().numpy()
        if exact:
            assert np.array_equal(got, o_ref), f"step {t}: outputs not bit-exact"
        else:
            e = normwise_err(got, o_ref)
            worst_o = max(worst_o, e)
            assert e <= tol, f"step {t}: output error {e:.3e}"
        if folded.any():
            nflush += 1
            ck = layer.ckpt.cpu().numpy()
            if exact:
                assert np.array_equal(ck, S), f"step {t}: checkpoint not bit-exact"
            else:
                es = matrix_err(ck, S)
                worst_s = max(worst_s, es)
                assert es <= tol, f"step {t}: checkpoint error {es:.3e}"
        if t % check_every == 0 or t == steps:
            _check_buffers(layer, model, sh)
    assert layer.read_error() == 0
    return layer, model, S, worst_o, worst_s, nflush


def test_tiny_workload(dev):
    """Tiny correctness workload: batch 2, 2 heads, P = N = 16, 64 steps, L = 16."""
    say("case: tiny workload, 64 steps")
    _, _, _, eo, es, nf = run_decode(W.TINY, W.TINY_STEPS, dev)
    assert nf == 4
    say(f"  max output err {eo:.2e}, checkpoint err {es:.2e}")


def test_integer_inputs_are_bit_exact(dev):
    """alpha = 1 and integer k, q, v keep every fp32 intermediate exact, so the
    GPU must reproduce the oracle bit for bit whatever its summation order."""
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=2, dim_v=16, dim_k=16, window=8, dist="integer")
    say("case: integer inputs, 40 steps, L = 8")
    run_decode(sh, 40, dev, exact=True)


@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hvpt", [1, 3])
def test_ragged_shapes(dev, N, in_dtype, hvpt):
    """Rows that do not fill the row groups (P = 20), a key group of 3 split
    over tiles or kept whole, a window of 5 with a partial last window."""
    sh = W.Shape(batch=3, n_vheads=6, n_kheads=2, dim_v=20, dim_k=N, window=5, in_dtype=in_dtype,
                 dist="uniform")
    say(f"case: ragged N={N} {in_dtype} hvpt={hvpt}")
    S0 = W.initial_state_np(sh, 3, std=0.5)
    run_decode(sh, 23, dev, S0=S0, heads_per_tile=hvpt)


@pytest.mark.parametrize("N", [32, 128, 256])
def test_wide_key_dims(dev, N):
    sh = W.Shape(batch=2, n_vheads=4, n_kheads=4, dim_v=32, dim_k=N, window=6, dist="uniform")
    say(f"case: key dim {N}")
    run_decode(sh, 14, dev, S0=W.initial_state_np(sh, 5))


def test_window_one_is_conventional(dev):
    """L = 1: every step folds its own record (conventional decoding)."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=1, dim_v=16, dim_k=32, window=1, dist="uniform")
    say("case: L = 1")
    _, _, _, _, _, nf = run_decode(sh, 9, dev)
    assert nf == 9


def test_long_window_pure_replay(dev):
    """L = 32 with 31 steps never folds: every output is replay from S_0."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=16, dim_k=64, window=32, dist="uniform")
    say("case: L = 32, 31 steps")
    layer, _, _, _, _, nf = run_decode(sh, 31, dev, S0=W.initial_state_np(sh, 9))
    assert nf == 0
    np.testing.assert_array_equal(layer.ckpt.cpu().numpy(), W.initial_state_np(sh, 9))


def test_gdn_shaped_small(dev):
    """Gated-DeltaNet-shaped scalar-decay layer (4 value heads per key group,
    K = V = 128, bf16 inputs) at a small batch, whole key group per tile and
    split over tiles."""
    sh = W.with_(W.GDN, batch=3, n_vheads=8, n_kheads=2)
    for hvpt in (1, 2, 4):
        say(f"case: gdn small hvpt={hvpt}")
        run_decode(sh, 35, dev, heads_per_tile=hvpt, check_every=7)


@pytest.mark.parametrize("hvpt", [0, 4, 8])
def test_grouped_keys_sixteen_heads(dev, hvpt):
    """Mamba-2 head dims with keys shared by groups of 16 value heads (the
    window sweep's grouped case): the default two-head tiles and tiles of 4
    and 8 heads, all inside the group (a whole group of 1024 rows exceeds the
    shared memory and is refused); decode over two windows, then verify and
    commit rounds."""
    sh = W.Shape(batch=2, n_vheads=32, n_kheads=2, dim_v=64, dim_k=128, window=16, max_draft=4,
                 dist="uniform")
    say(f"case: grouped keys g=16 hvpt={hvpt}")
    run_decode(sh, 35, dev, S0=W.initial_state_np(sh, 6), heads_per_tile=hvpt, check_every=5)
    run_spec(sh, 12, dev, S0=W.initial_state_np(sh, 7), heads_per_tile=hvpt)


def test_explicit_flush_materialises_state(dev):
    sh = W.Shape(batch=3, n_vheads=4, n_kheads=2, dim_v=16, dim_k=32, window=8, dist="uniform")
    say("case: explicit flush")
    layer, model, S, _, _, _ = run_decode(sh, 11, dev, S0=W.initial_state_np(sh, 2))
    layer.flush()
    model.flush()
    es = matrix_err(layer.ckpt.cpu().numpy(), S)
    assert es <= TOL, es
    assert np.all(layer.count.cpu().numpy() == 0)
    ck = layer.ckpt.clone()
    layer.flush()                                  # empty buffers: untouched
    assert torch.equal(ck, layer.ckpt)


def test_reset_listed_sequences(dev):
    sh = W.Shape(batch=4, n_vheads=2, n_kheads=2, dim_v=16, dim_k=16, window=4, dist="uniform")
    layer, _, _, _, _, _ = run_decode(sh, 6, dev, S0=W.initial_state_np(sh, 1))
    before = layer.ckpt.cpu().numpy()
    layer.reset(torch.tensor([1, 3], dtype=torch.int32, device=dev))
    after = layer.ckpt.cpu().numpy()
    cnt = layer.count.cpu().numpy()
    assert np.all(after[[1, 3]] == 0) and np.array_equal(after[[0, 2]], before[[0, 2]])
    assert np.all(cnt[[1, 3]] == 0) and np.all(cnt[[0, 2]] == 2)
    layer.reset(torch.tensor([7], dtype=torch.int32, device=dev))   # out of range: flagged only
    assert layer.read_error(clear=True) == 1
    assert np.array_equal(layer.ckpt.cpu().numpy(), after)


def test_device_error_paths(dev):
    """A corrupted pointer is detected on the device: the tile is left
    untouched and the error word says why."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=16, dim_k=16, window=4, max_draft=2,
                 dist="uniform")
    layer = _layer(sh, dev)
    layer.count[1, :] = 4                               # outside 0..L-1
    ins = to_dev(W.decode_inputs_np(sh, 0, 0), dev)
    o = torch.full((2, 2, 16), 7.0, device=dev)
    layer.decode_step(*ins, o)
    assert layer.read_error(clear=True) == 1
    assert torch.all(o[1] == 7.0) and not torch.all(o[0] == 7.0)
    assert np.all(layer.count.cpu().numpy()[1] == 4)
    layer.count[1, :] = 0
    a, k, v, q = to_dev(W.draft_inputs_np(sh, 0, 0, 2), dev)
    layer.spec_verify(a, k, v, q)
    layer.commit(torch.tensor([1, 3], dtype=torch.int32, device=dev))   # 3 > T
    assert layer.read_error(clear=True) == 2
    cnt = layer.count.cpu().numpy()
    assert np.all(cnt[0] == 2) and np.all(cnt[1] == 0)


def test_decode_is_bitwise_reproducible(dev):
    sh = W.with_(W.TINY, n_vheads=4, n_kheads=2, dist="uniform")
    outs = []
    for _ in range(2):
        layer = _layer(sh, dev)
        os_ = []
        for t in range(20):
            os_.append(layer.decode_step(*to_dev(W.decode_inputs_np(sh, 4, t), dev)).cpu().numpy())
        outs.append((np.stack(os_), layer.ckpt.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


# ------------------------------------------------------------- speculative
def run_spec(sh, rounds, dev, seed=0, S0=None, decode_between=True, accept=None, **kw):
    """Alternate verify(T)+commit(accepted) with plain decode steps; compare
    draft outputs, pointers, buffers and folded checkpoints with the oracle.
    accept(r, Tr) gives round r's accepted lengths (default: seeded uniform)."""
    layer = _layer(sh, dev, **kw)
    g = sh.group
    T = sh.max_draft
    S = np.zeros((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k))
    if S0 is not None:
        layer.ckpt.copy_(torch.from_numpy(S0.astype(np.float32)))
        S = S0.astype(np.float32).astype(np.float64)
    model = _model(sh)
    worst = 0.0
    for r in range(rounds):
        Tr = 1 + (r % T) if r % 3 == 2 else T           # also exercise T < T_max
        a, k, v, q = W.draft_inputs_np(sh, seed, r, Tr)
        O = layer.spec_verify(*to_dev((a, k, v, q), dev, sh.in_dtype))
        O_ref, states = recurrence.verify(S, a, k, v, q, g)
        e = normwise_err(O.cpu().numpy(), O_ref)
        worst = max(worst, e)
        assert e <= TOL, f"round {r}: verify error {e:.3e}"
        model.verify(a, np_bits(k, sh.in_dtype), np_bits(v, sh.in_dtype))
        _check_buffers(layer, model, sh)                  # drafts appended, pointer unchanged
        acc = W.accepted_np(sh.batch, Tr, seed + 1, r) if accept is None else accept(r, Tr)
        layer.commit(torch.from_numpy(acc).to(dev))
        folded = model.commit(acc)
        S = recurrence.commit(states, acc)
        _check_buffers(layer, model, sh)
        if folded.any():
            ck = layer.ckpt.cpu().numpy()
            es = matrix_err(ck[folded], S[folded])
            assert es <= TOL, f"round {r}: folded checkpoint error {es:.3e}"
        if decode_between and r % 4 == 3:
            x = W.decode_inputs_np(sh, seed + 7, r)
            o = layer.decode_step(*to_dev(x, dev, sh.in_dtype))
            S, o_ref = recurrence.eqR_step(S, *x, g)
            model.decode(x[0], np_bits(x[1], sh.in_dtype), np_bits(x[2], sh.in_dtype))
            e = normwise_err(o.cpu().numpy(), o_ref)
            assert e <= TOL, f"round {r}: decode error {e:.3e}"
    layer.flush()
    es = matrix_err(layer.ckpt.cpu().numpy(), S)
    assert es <= TOL, f"final flush error {es:.3e}"
    assert layer.read_error() == 0
    return worst


@pytest.mark.parametrize("hvpt", [1, 2])
def test_spec_verify_commit(dev, hvpt):
    sh = W.Shape(batch=6, n_vheads=4, n_kheads=2, dim_v=16, dim_k=32, window=8, max_draft=4,
                 dist="uniform")
    say(f"case: spec verify/commit hvpt={hvpt}")
    run_spec(sh, 30, dev, S0=W.initial_state_np(sh, 1), heads_per_tile=hvpt)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_spec_larger_drafts(dev, in_dtype):
    sh = W.Shape(batch=3, n_vheads=2, n_kheads=1, dim_v=24, dim_k=64, window=5, max_draft=8,
                 in_dtype=in_dtype, dist="uniform")
    say(f"case: spec T_max = 8 {in_dtype}")
    run_spec(sh, 16, dev, S0=W.initial_state_np(sh, 2))


def test_spec_window32_drafts8_wide_keys(dev):
    """Capacity C = 40 at N = 128: every key pass of the verify kernel holds
    committed records or drafts, and commits fold up to 39 records."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=16, dim_k=128, window=32, max_draft=8,
                 dist="uniform")
    say("case: spec L = 32, T_max = 8, N = 128")
    run_spec(sh, 30, dev, S0=W.initial_state_np(sh, 3))


def test_long_window_wide_keys(dev):
    """L = 32 at N = 128: the decode kernel's four key passes all hold records."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=16, dim_k=128, window=32, dist="uniform")
    say("case: L = 32, N = 128, 70 steps")
    _, _, _, _, _, nf = run_decode(sh, 70, dev, S0=W.initial_state_np(sh, 4))
    assert nf == 2


def test_verify_with_one_draft_equals_decode(dev):
    """T = 1 reduces to a decode step (same output, same appended record)."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=16, dim_k=32, window=8, max_draft=1,
                 dist="uniform")
    A = _layer(sh, dev)
    Bl = _layer(sh, dev)
    for t in range(5):
        x = W.decode_inputs_np(sh, 0, t)
        A.decode_step(*to_dev(x, dev))
        Bl.decode_step(*to_dev(x, dev))
    x = W.decode_inputs_np(sh, 0, 5)
    oa = A.decode_step(*to_dev(x, dev))
    a, k, v, q = (y[:, None] for y in x)
    ob = Bl.spec_verify(*to_dev((a, k, v, q), dev))
    Bl.commit(torch.ones(2, dtype=torch.int32, device=dev))
    assert normwise_err(ob[:, 0].cpu().numpy(), oa.cpu().numpy()) <= TOL
    assert torch.equal(A.count, Bl.count) and torch.equal(A.kbuf, Bl.kbuf) and torch.equal(A.vbuf, Bl.vbuf)


@pytest.mark.parametrize("all_accepted", [True, False])
def test_commit_fold_list_longer_than_its_grid(dev, all_accepted):
    """20480 tiles (160 sequences x 128 one-head tiles): when every draft is
    accepted, every tile folds at the same commit, so the fold list is longer
    than the commit's fixed fold grid and workgroups take several tiles; with
    seeded acceptances the list is partial and changes every commit."""
    sh = W.Shape(batch=160, n_vheads=128, n_kheads=128, dim_v=16, dim_k=16, window=4, max_draft=4,
                 dist="uniform")
    say(f"case: commit fold list over 20480 tiles, all accepted={all_accepted}")
    accept = (lambda r, Tr: np.full(sh.batch, Tr, dtype=np.int32)) if all_accepted else None
    run_spec(sh, 7, dev, S0=W.initial_state_np(sh, 12, std=0.5), accept=accept)


# ------------------------------------------------------- largest supported sizes
@pytest.mark.parametrize("P,N,L,T", [(256, 256, 16, 8), (256, 128, 32, 8), (128, 256, 32, 8)])
def test_largest_head_dims_windows_and_drafts(dev, P, N, L, T):
    """The largest value and key dims together with the largest windows and
    draft counts whose tiles still fit in shared memory: decode over two
    whole windows and a partial one, then verify/commit rounds with T drafts."""
    sh = W.Shape(batch=2, n_vheads=2, n_kheads=2, dim_v=P, dim_k=N, window=L, max_draft=T,
                 dist="uniform")
    say(f"case: largest dims P={P} N={N} L={L} T={T}")
    _, _, _, _, _, nf = run_decode(sh, 2 * L + 3, dev, S0=W.initial_state_np(sh, 8, std=0.5))
    assert nf == 2
    run_spec(sh, 10, dev, S0=W.initial_state_np(sh, 9, std=0.5))


@pytest.mark.parametrize("hk,N,L,T", [(2, 128, 8, 2), (8, 32, 4, 4)])
def test_largest_tiles(dev, hk, N, L, T):
    """1024-row tiles (4 heads of P = 256): inside one key group of 4 heads, or
    over 4 key groups of one head each."""
    sh = W.Shape(batch=2, n_vheads=8, n_kheads=hk, dim_v=256, dim_k=N, window=L, max_draft=T,
                 dist="uniform")
    say(f"case: 1024-row tiles Hk={hk} N={N} L={L} T={T}")
    run_decode(sh, 3 * L + 1, dev, S0=W.initial_state_np(sh, 10, std=0.5), heads_per_tile=4)
    run_spec(sh, 10, dev, S0=W.initial_state_np(sh, 11, std=0.5), heads_per_tile=4)


# ------------------------------------------------------- tiles of several key groups
@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("g,hvpt", [(1, 2), (1, 4), (2, 4), (2, 6)])
def test_tiles_spanning_key_groups(dev, N, in_dtype, g, hvpt):
    """A workgroup tile of several whole key groups (each group's scores and
    q slices kept apart) must give the same results as one group per tile."""
    Hv = 12
    sh = W.Shape(batch=3, n_vheads=Hv, n_kheads=Hv // g, dim_v=20, dim_k=N, window=5,
                 in_dtype=in_dtype, dist="uniform")
    say(f"case: multi-group tiles g={g} hvpt={hvpt} N={N} {in_dtype}")
    run_decode(sh, 17, dev, S0=W.initial_state_np(sh, 6, std=0.5), heads_per_tile=hvpt)


@pytest.mark.parametrize("g,hvpt", [(1, 2), (2, 4)])
def test_spec_with_tiles_spanning_key_groups(dev, g, hvpt):
    sh = W.Shape(batch=4, n_vheads=8, n_kheads=8 // g, dim_v=16, dim_k=32, window=6, max_draft=4,
                 dist="uniform")
    say(f"case: spec multi-group tiles g={g} hvpt={hvpt}")
    run_spec(sh, 14, dev, S0=W.initial_state_np(sh, 4), heads_per_tile=hvpt)
