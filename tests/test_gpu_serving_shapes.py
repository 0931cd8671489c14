"""Full serving shapes on the GPU, in the launch configuration bench.py times.

The oracle cannot step every (sequence, head) pair of a 1-2 GiB state in
seconds, so each test runs the whole batch on the GPU and checks a seeded
sample of pairs element by element against the fp64 recurrence (outputs at
every step, checkpoints after every fold), plus properties that hold for every
pair (pointer copies bit-exact, no device error).

Workloads:
  * Mamba-2-style layer: batch 256, 128 heads, P = 64, N = 128, L = 16,
    256 steps, fp32 (ReplaySSM and the conventional fused decode).
  * Gated-DeltaNet-shaped layer: batch 256, 64 value heads sharing 16 key
    heads, K = V = 128, L = 16, 512 steps, bf16 k/q/v.
  * Speculative verify/commit: Mamba-2 shape, batch 512, T = 4, accepted
    lengths uniform in 0..4, random initial checkpoint (ReplaySSM and the
    snapshot baseline).
  * Long decode: batch 64, 64 heads, P = N = 128, 4096 steps, fp32 checkpoint
    with a bf16, fp8 or MXFP4 read copy, against the fully quantised-state arms
    (bf16, fp8).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import cpu_c, recurrence
from ssm_layer_decode_amd import workloads as W
from tests.helpers import matrix_err, normwise_err, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ssm_layer_decode_amd import _lib
    _lib.load()
    return torch.device("cuda:0")


def _sample(B, H, n, seed):
    rng = np.random.default_rng(seed)
    b = rng.choice(B, size=n, replace=(n > B))
    h = rng.integers(0, H, n)
    return b, h


class Sampled:
    """fp64 eq.R for a set of (b, h) pairs, fed from device inputs."""

    def __init__(self, dev, sh, b, h, S0=None):
        self.g = sh.group
        self.bi = torch.as_tensor(b, device=dev, dtype=torch.long)
        self.hi = torch.as_tensor(h, device=dev, dtype=torch.long)
        self.ki = self.hi // self.g
        n = len(b)
        self.S = np.zeros((n, 1, sh.dim_v, sh.dim_k)) if S0 is None else S0[:, None].astype(np.float64)

    def pick(self, a, k, v, q):
        f = lambda x: x.float().cpu().numpy()
        return (f(a[self.bi, self.hi])[:, None], f(k[self.bi, self.ki])[:, None],
                f(v[self.bi, self.hi])[:, None], f(q[self.bi, self.ki])[:, None])

    def step(self, a, k, v, q):
        self.S, o = recurrence.eqR_step(self.S, *self.pick(a, k, v, q))
        return o[:, 0]

    def out(self, o):
        return o[self.bi, self.hi].cpu().numpy()

    def state(self, S):
        return S[self.bi, self.hi].float().cpu().numpy()


def test_mamba2_serving_shape(dev):
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM, convssm_decode_step
    sh, steps = W.MAMBA2, W.MAMBA2_STEPS
    say(f"case: mamba2 serving shape B={sh.batch}, {steps} steps")
    cfg = LayerConfig.of(sh)
    layer = ReplaySSM(cfg, device=dev)
    conv = torch.zeros((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k), device=dev)
    oc = torch.empty((sh.batch, sh.n_vheads, sh.dim_v), device=dev)
    b, h = _sample(sh.batch, sh.n_vheads, 24, 1)
    ref = Sampled(dev, sh, b, h)
    worst = [0.0, 0.0, 0.0]
    for t in range(steps):
        a, k, v, q = W.decode_inputs_torch(sh, 0, t, device=dev)
        o = layer.decode_step(a, k, v, q)
        convssm_decode_step(cfg, conv, None, "f32", a, k, v, q, oc)
        o_ref = ref.step(a, k, v, q)
        worst[0] = max(worst[0], normwise_err(ref.out(o), o_ref))
        worst[1] = max(worst[1], normwise_err(ref.out(oc), o_ref))
        if (t + 1) % sh.window == 0:
            worst[2] = max(worst[2], matrix_err(ref.state(layer.ckpt), ref.S[:, 0]))
            assert int(layer.count.max()) == 0 and int(layer.count.min()) == 0
        else:
            assert int(layer.count.min()) == int(layer.count.max()) == (t + 1) % sh.window
        assert max(worst) <= TOL, (t, worst)
    assert matrix_err(ref.state(conv), ref.S[:, 0]) <= TOL
    assert layer.read_error() == 0
    say(f"  worst errors: replay out {worst[0]:.2e}, conventional out {worst[1]:.2e}, checkpoint {worst[2]:.2e}")


def test_gdn_serving_shape(dev):
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    sh, steps = W.GDN, W.GDN_STEPS
    say(f"case: gdn serving shape B={sh.batch}, {steps} steps, bf16 inputs")
    layer = ReplaySSM(LayerConfig.of(sh), device=dev)
    b, h = _sample(sh.batch, sh.n_vheads, 24, 2)
    ref = Sampled(dev, sh, b, h)
    worst = 0.0
    for t in range(steps):
        a, k, v, q = W.decode_inputs_torch(sh, 0, t, device=dev)
        o = layer.decode_step(a, k, v, q)
        worst = max(worst, normwise_err(ref.out(o), ref.step(a, k, v, q)))
        if (t + 1) % sh.window == 0:
            worst = max(worst, matrix_err(ref.state(layer.ckpt), ref.S[:, 0]))
        assert worst <= TOL, (t, worst)
    # buffered records of the sampled pairs are bit copies of the inputs: run a
    # few more steps and compare slots 0..h-1
    kept = []
    for t in range(steps, steps + 5):
        x = W.decode_inputs_torch(sh, 0, t, device=dev)
        layer.decode_step(*x)
        kept.append(x)
    for j, (a, k, v, q) in enumerate(kept):
        assert torch.equal(layer.kbuf[:, :, j], k) and torch.equal(layer.vbuf[:, :, j], v)
        assert torch.equal(layer.abuf[:, :, j], a)
    assert int(layer.count.min()) == int(layer.count.max()) == 5
    assert layer.read_error() == 0
    say(f"  worst error {worst:.2e}")


def test_spec_serving_shape(dev):
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM, convssm_commit, convssm_spec_verify
    sh, T = W.SPEC, W.SPEC_T
    rounds = 40
    say(f"case: spec serving shape B={sh.batch}, T={T}, {rounds} rounds (replay + snapshot)")
    cfg = LayerConfig.of(sh)
    layer = ReplaySSM(cfg, device=dev)
    S0 = W.initial_state_torch(sh, 1, device=dev)
    layer.ckpt.copy_(S0)
    ring = sh.max_draft + 1
    snaps = torch.zeros((sh.batch, ring, sh.n_vheads, sh.dim_v, sh.dim_k), device=dev)
    snaps[:, 0] = S0
    cur = torch.zeros(sh.batch, dtype=torch.int32, device=dev)
    err = torch.zeros(4, dtype=torch.int32, device=dev)
    b, h = _sample(sh.batch, sh.n_vheads, 16, 3)
    ref = Sampled(dev, sh, b, h, S0=S0[torch.as_tensor(b, device=dev), torch.as_tensor(h, device=dev)].cpu().numpy())
    ar_idx = torch.arange(len(b), device=dev)
    count = np.zeros(sh.batch, dtype=np.int64)
    worst = [0.0, 0.0, 0.0]
    folds = 0
    for r in range(rounds):
        a, k, v, q = W.draft_inputs_torch(sh, 0, r, T, device=dev)
        O = layer.spec_verify(a, k, v, q)
        Os = torch.empty_like(O)
        convssm_spec_verify(cfg, snaps, cur, T, a, k, v, q, Os)
        pa, pk, pv, pq = (x[ref.bi] for x in (a, k, v, q))
        f = lambda x: x.float().cpu().numpy()
        # per-pair draft arrays [n][T][1][...]
        ar = f(pa[ar_idx, :, ref.hi])[:, :, None]
        kr = f(pk[ar_idx, :, ref.ki])[:, :, None]
        vr = f(pv[ar_idx, :, ref.hi])[:, :, None]
        qr = f(pq[ar_idx, :, ref.ki])[:, :, None]
        O_ref, states = recurrence.verify(ref.S, ar, kr, vr, qr)
        got = O[ref.bi, :, ref.hi].cpu().numpy()
        gots = Os[ref.bi, :, ref.hi].cpu().numpy()
        worst[0] = max(worst[0], normwise_err(got, O_ref[:, :, 0]))
        worst[1] = max(worst[1], normwise_err(gots, O_ref[:, :, 0]))
        acc = W.accepted_torch(sh.batch, T, 1, r, device=dev)
        layer.commit(acc)
        convssm_commit(cfg, cur, acc, T, err)
        acc_np = acc.cpu().numpy()
        ref.S = recurrence.commit(states, acc_np[b])
        count += acc_np
        fold = count >= sh.window
        folds += int(fold.sum())
        count[fold] = 0
        cnt = layer.count.cpu().numpy()
        assert np.all(cnt == count[:, None]), f"round {r}: pointers differ"
        folded_s = fold[b]
        if folded_s.any():
            worst[2] = max(worst[2], matrix_err(ref.state(layer.ckpt)[folded_s], ref.S[folded_s, 0]))
        assert max(worst) <= TOL, (r, worst)
    layer.flush()
    assert matrix_err(ref.state(layer.ckpt), ref.S[:, 0]) <= TOL
    sel = snaps[ref.bi, cur[ref.bi].long(), ref.hi].cpu().numpy()
    assert matrix_err(sel, ref.S[:, 0]) <= TOL
    assert layer.read_error() == 0 and int(err[0]) == 0
    assert folds > 0
    say(f"  worst errors: replay verify {worst[0]:.2e}, snapshot verify {worst[1]:.2e}, "
        f"folded checkpoints {worst[2]:.2e}; {folds} folds")


def _kl_rows(p_logits, q_logits):
    p = p_logits - p_logits.max(axis=-1, keepdims=True)
    q = q_logits - q_logits.max(axis=-1, keepdims=True)
    lp = p - np.log(np.exp(p).sum(axis=-1, keepdims=True))
    lq = q - np.log(np.exp(q).sum(axis=-1, keepdims=True))
    return np.sum(np.exp(lp) * (lp - lq), axis=-1)


def test_long_decode_split_precision(dev):
    """Split precision over 4096 steps: the fp32 checkpoint is unaffected by
    the read copy, the read error stays flat in t, and it is below that of
    rounding the stored state every step ([ru] §06; [ar] quantisation section)."""
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM, convssm_decode_step
    from oracle import quant
    sh, steps = W.LONG, W.LONG_STEPS
    say(f"case: long decode B={sh.batch}, {steps} steps, read copies bf16/fp8 vs quantised state")
    plain = ReplaySSM(LayerConfig.of(sh), device=dev)
    split = {f: ReplaySSM(LayerConfig.of(sh, read_copy=f), device=dev) for f in ("bf16", "fp8", "mxfp4")}
    # fp16 checkpoint with stochastic rounding, read directly or through an MXFP4 copy
    f16 = {f: ReplaySSM(LayerConfig.of(sh, read_copy=f, ckpt="f16sr", sr_seed=11), device=dev)
           for f in ("none", "mxfp4")}
    # fp8 checkpoint with stochastic rounding, read through a bf16 or an MXFP4 copy
    f8 = {f: ReplaySSM(LayerConfig.of(sh, read_copy=f, ckpt="fp8sr", sr_seed=13), device=dev)
          for f in ("bf16", "mxfp4")}
    cfg = LayerConfig.of(sh)
    qstate = {"bf16": torch.zeros((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k), dtype=torch.bfloat16, device=dev),
              "fp8": torch.zeros((sh.batch, sh.n_vheads, sh.dim_v, sh.dim_k), dtype=torch.uint8, device=dev)}
    qscale = torch.ones((sh.batch, sh.n_vheads, sh.dim_v), device=dev)
    seqs = torch.tensor([5, 42], device=dev)
    arms = ["plain", "split-bf16", "split-fp8", "split-mxfp4", "f16sr", "f16sr-mxfp4", "fp8sr-bf16", "fp8sr-mxfp4",
            "qstate-bf16", "qstate-fp8"]
    outs = {m: np.zeros((steps, 2, sh.n_vheads, sh.dim_v), dtype=np.float32) for m in arms}
    ins = {n: np.zeros((steps, 2) + s, dtype=np.float32) for n, s in
           (("a", (sh.n_vheads,)), ("k", (sh.n_kheads, sh.dim_k)), ("v", (sh.n_vheads, sh.dim_v)),
            ("q", (sh.n_kheads, sh.dim_k)))}
    o = torch.empty((sh.batch, sh.n_vheads, sh.dim_v), device=dev)
    chunk = 256
    buf = {m: torch.empty((chunk, 2, sh.n_vheads, sh.dim_v), device=dev) for m in arms}
    ibuf = {n: torch.empty((chunk, 2) + ins[n].shape[2:], device=dev) for n in ins}
    for t in range(steps):
        a, k, v, q = W.decode_inputs_torch(sh, 0, t, device=dev)
        i = t % chunk
        for n, x in zip("akvq", (a, k, v, q)):
            ibuf[n][i] = x[seqs]
        buf["plain"][i] = plain.decode_step(a, k, v, q, o)[seqs]
        buf["split-mxfp4"][i] = split["mxfp4"].decode_step(a, k, v, q, o)[seqs]
        buf["f16sr"][i] = f16["none"].decode_step(a, k, v, q, o)[seqs]
        buf["f16sr-mxfp4"][i] = f16["mxfp4"].decode_step(a, k, v, q, o)[seqs]
        for f in ("bf16", "mxfp4"):
            buf[f"fp8sr-{f}"][i] = f8[f].decode_step(a, k, v, q, o)[seqs]
        for f in ("bf16", "fp8"):
            buf[f"split-{f}"][i] = split[f].decode_step(a, k, v, q, o)[seqs]
            convssm_decode_step(cfg, qstate[f], qscale if f == "fp8" else None, f, a, k, v, q, o)
            buf[f"qstate-{f}"][i] = o[seqs]
        if i == chunk - 1:
            for m in arms:
                outs[m][t - chunk + 1:t + 1] = buf[m].cpu().numpy()
            for n in ins:
                ins[n][t - chunk + 1:t + 1] = ibuf[n].cpu().numpy()
        if t in (15, 1023, steps - 1):
            for f in ("bf16", "fp8", "mxfp4"):
                assert torch.equal(split[f].ckpt, plain.ckpt), f"step {t}: {f} split checkpoint differs"
    for l in [plain, *split.values(), *f16.values(), *f8.values()]:
        assert l.read_error() == 0
    truth, _ = cpu_c.decode(np.zeros((2, sh.n_vheads, sh.dim_v, sh.dim_k)), ins["a"], ins["k"], ins["v"], ins["q"])
    err = {m: np.array([normwise_err(outs[m][t], truth[t]) for t in range(steps)]) for m in arms}
    proj = W.projection_np(sh.n_vheads * sh.dim_v, W.LONG_VOCAB, seed=2)
    lr = truth.reshape(steps * 2, -1) @ proj
    c = 1.0 / lr.std()
    kl = {m: _kl_rows(c * lr, c * (outs[m].reshape(steps * 2, -1).astype(np.float64) @ proj)) for m in arms[1:]}
    for m in arms:
        early, late = err[m][512:1024].max(), err[m][3584:].max()
        say(f"  {m:12s} max err {err[m].max():.3e}  [512,1024) {early:.3e}  [3584,4096) {late:.3e}"
            + (f"  KL mean {kl[m].mean():.3e} max {kl[m].max():.3e}" if m in kl else ""))
    assert err["plain"].max() <= TOL
    # Read-error bound per output element: each copy entry is within the
    # format's unit roundoff (bf16 RNE 2^-8 relative; e4m3 row-scaled 2^-4
    # relative or 2^-10 of the row scale), so
    #   |o - o_exact| <= u_rel * g (|S_ckpt||q|) + u_abs * g amax sum|q|
    # plus the fp32 path's own tolerance.  KL of the projected outputs is
    # bounded by 2 u_rel^2 (second-order expansion of KL in the logit error).
    A, Z = cpu_c.split_read_bound(None, ins["a"], ins["k"], ins["v"], ins["q"], sh.window)
    slack = TOL * np.abs(truth).max(axis=-1, keepdims=True)
    for f, ur, ua in (("bf16", 2.0 ** -8, 0.0), ("fp8", 2.0 ** -4, 2.0 ** -10 / 448),
                      ("mxfp4", 2.0 ** -2, 2.0 ** -4)):
        m = f"split-{f}"
        bound = ur * A * (1 + 1e-6) + ua * Z + slack
        ratio = np.abs(outs[m].astype(np.float64) - truth) / bound
        # flush steps output the fp32 fold (no copy read), and during the first
        # window the checkpoint and its copy are still zero: there the error is
        # the fp32 path's and the bound only its slack.  The copy's rounding
        # shows on the non-flush steps after the first window.
        idx = np.arange(steps)
        nonflush = (idx + 1) % sh.window != 0
        read = nonflush & (idx >= sh.window)
        say(f"  {m}: largest error / bound {ratio.max():.3f} (<= 1 required); non-flush steps after the "
            f"first window {ratio[read].max():.3f}; first window {ratio[idx < sh.window].max():.3f}; "
            f"flush steps {ratio[~nonflush].max():.3f}; KL mean / (2 u^2) {kl[m].mean() / (2 * ur ** 2):.2e}")
        assert ratio.max() <= 1.0, f"{m}: read error exceeds its rounding bound"
        assert kl[m].mean() <= 2 * ur ** 2
        assert err[m][3584:].max() <= 2 * err[m][512:1024].max()
        if f"qstate-{f}" in kl:
            assert kl[m].mean() <= kl[f"qstate-{f}"].mean()
    # fp16 checkpoint, stochastic rounding at folds only ([ru] §06: close to
    # FP32): its rounding does feed the recurrence, once per window.  Required:
    # error flat in t, and KL below that of re-rounding the stored state to bf16
    # at every step.  With an MXFP4 copy on top, the two errors add: to second
    # order KL is a quadratic form d^T F d of the logit error, and
    # (a+b)^T F (a+b) <= 2 a^T F a + 2 b^T F b.
    for m in ("f16sr", "f16sr-mxfp4"):
        say(f"  {m}: KL mean {kl[m].mean():.3e}; qstate-bf16 {kl['qstate-bf16'].mean():.3e}, "
            f"split-mxfp4 {kl['split-mxfp4'].mean():.3e}")
        assert err[m][3584:].max() <= 2 * err[m][512:1024].max()
    assert kl["f16sr"].mean() <= kl["qstate-bf16"].mean()
    assert kl["f16sr-mxfp4"].mean() <= 2 * kl["split-mxfp4"].mean() + 2 * kl["f16sr"].mean()
    # fp8 checkpoint ([ar] section on limiting quantization error: low-precision
    # reads with an FP8 recurrence), rounded stochastically once per window:
    # error flat in t; through a bf16 copy (whose own error is small) its KL is
    # below that of rounding the stored state to fp8 at every step; with an
    # MXFP4 copy the two errors add as above.
    for m in ("fp8sr-bf16", "fp8sr-mxfp4"):
        say(f"  {m}: KL mean {kl[m].mean():.3e}; qstate-fp8 {kl['qstate-fp8'].mean():.3e}, "
            f"split-mxfp4 {kl['split-mxfp4'].mean():.3e}")
        assert err[m][3584:].max() <= 2 * err[m][512:1024].max()
    assert kl["fp8sr-bf16"].mean() <= kl["qstate-fp8"].mean()
    assert kl["fp8sr-mxfp4"].mean() <= 2 * kl["split-mxfp4"].mean() + 2 * kl["fp8sr-bf16"].mean()
