"""Decode, verify and commit captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed.  The library records no memsets and keeps no device-side state
beyond the caller's buffers, so every replay must equal the same calls made
eagerly on a twin layer, bit for bit (same kernels in the same order), with
eager work and synchronisations between the replays.  The captured layer's
commit work area starts out holding garbage: every commit clears its own list
count first.  With an fp16 checkpoint every fold takes its stochastic-rounding
epoch from a per-tile device counter, so replays draw new numbers and still
equal the eager twin; a replayed fold is also checked against the oracle's
rounding at each epoch."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import stochastic
from ssm_layer_decode_amd import _lib
from ssm_layer_decode_amd import workloads as W
from tests.helpers import say, set_fp8_ckpt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    return torch.device("cuda:0")


def _pair(sh, dev, S0, read_copy="none", ckpt="f32"):
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    out = []
    for _ in range(2):
        layer = ReplaySSM(LayerConfig.of(sh, read_copy=read_copy, ckpt=ckpt, sr_seed=17), device=dev)
        if ckpt == "fp8sr":
            set_fp8_ckpt(layer, S0.numpy())
        else:
            layer.ckpt.copy_(S0.to(layer.ckpt.dtype))
        if read_copy != "none":
            layer.refresh_read_copy()
        out.append(layer)
    return out


def _same(A, B):
    pairs = [(A.ckpt, B.ckpt), (A.count, B.count), (A.kbuf, B.kbuf), (A.vbuf, B.vbuf), (A.abuf, B.abuf)]
    if A.read_copy is not None:
        pairs.append((A.read_copy, B.read_copy))
    if A.row_scale is not None:
        pairs.append((A.row_scale, B.row_scale))
    if A.folds is not None:
        pairs.append((A.folds, B.folds))
    return all(torch.equal(x, y) for x, y in pairs)


@pytest.mark.parametrize("B,Hv,Hk,copy,ckpt", [(4, 4, 2, "none", "f32"), (160, 128, 128, "none", "f32"),
                                               (4, 4, 2, "fp8", "f32"), (4, 4, 1, "mxfp4", "f32"),
                                               (6, 4, 4, "bf16", "f32"), (4, 4, 2, "none", "f16sr"),
                                               (4, 4, 1, "mxfp4", "f16sr"), (4, 4, 1, "mxfp4", "fp8sr"),
                                               (4, 4, 2, "bf16", "fp8sr")])
def test_graph_replay_matches_eager(dev, B, Hv, Hk, copy, ckpt):
    """The second shape has 20480 tiles, more than the commit's fold grid;
    with a read copy, folds rewrite the copy and verify reads it; with an
    fp16 or fp8 checkpoint, each replayed fold rounds with the next epoch."""
    sh = W.Shape(batch=B, n_vheads=Hv, n_kheads=Hk, dim_v=16, dim_k=32, window=4, max_draft=2,
                 dist="uniform")
    T = sh.max_draft
    say(f"case: graph replay B={B} Hv={Hv} Hk={Hk} copy={copy} ckpt={ckpt}")
    S0 = torch.from_numpy(W.initial_state_np(sh, 21, std=0.5))
    A, E = _pair(sh, dev, S0, copy, ckpt)
    x0 = [t.to(dev) for t in map(torch.from_numpy, W.decode_inputs_np(sh, 22, 0))]
    d0 = [t.to(dev) for t in map(torch.from_numpy, W.draft_inputs_np(sh, 23, 0, T))]
    acc0 = torch.zeros(B, dtype=torch.int32, device=dev)
    # static buffers the graph reads and writes
    xs = [t.clone() for t in x0]
    ds = [t.clone() for t in d0]
    acc_s = acc0.clone()
    o_s = torch.empty((B, Hv, sh.dim_v), device=dev)
    O_s = torch.empty((B, T, Hv, sh.dim_v), device=dev)
    # warm-up (loads the kernels' code objects), the same on both layers
    for L_ in (A, E):
        L_.decode_step(*x0)
        L_.spec_verify(*d0)
        L_.commit(acc0)
    A.work.fill_(123456789)                              # not zeroed: each commit clears its count
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.decode_step(*xs, o_s)
        A.spec_verify(*ds, O_s)
        A.commit(acc_s)
    torch.cuda.synchronize()
    assert _same(A, E)                                   # capture runs nothing
    for r in range(8):
        x = [t.to(dev) for t in map(torch.from_numpy, W.decode_inputs_np(sh, 30, r))]
        d = [t.to(dev) for t in map(torch.from_numpy, W.draft_inputs_np(sh, 31, r, T))]
        acc = torch.from_numpy(W.accepted_np(B, T, 32, r)).to(dev)
        for s_, t_ in zip(xs + ds + [acc_s], x + d + [acc]):
            s_.copy_(t_)
        g.replay()
        o_e = E.decode_step(*x)
        O_e = E.spec_verify(*d)
        E.commit(acc)
        torch.cuda.synchronize()
        assert torch.equal(o_s, o_e) and torch.equal(O_s, O_e), r
        assert _same(A, E), r
        if r % 3 == 1:                                   # eager work on the captured layer too
            y = [t.to(dev) for t in map(torch.from_numpy, W.decode_inputs_np(sh, 33, r))]
            assert torch.equal(A.decode_step(*y), E.decode_step(*y))
            torch.cuda.synchronize()
    assert A.read_error() == 0 and E.read_error() == 0
    assert int(A.count.sum()) >= 0 and np.isfinite(A.ckpt.cpu().numpy()).all()


def test_graph_replayed_fold_draws_new_numbers(dev):
    """One decode step of an fp16-checkpoint layer with a window of one record
    (every step folds) is captured once and replayed from the same checkpoint
    and inputs: each replay must round with the next epoch -- the oracle's
    rounding of the same fold at epochs 0, 1, 2, ... -- so the stored
    checkpoints differ between replays."""
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    sh = W.Shape(batch=3, n_vheads=4, n_kheads=2, dim_v=16, dim_k=32, window=1, dist="uniform")
    seed = 23
    say("case: graph replay of an fp16 fold, epochs 0..5")
    S0 = W.initial_state_np(sh, 60, std=0.5).astype(np.float16)
    layer = ReplaySSM(LayerConfig.of(sh, ckpt="f16sr", sr_seed=seed), device=dev)
    S0_dev = torch.from_numpy(S0).to(dev)
    x = W.decode_inputs_np(sh, 61, 0)
    xs = [torch.from_numpy(t).to(dev) for t in x]
    o = torch.empty((sh.batch, sh.n_vheads, sh.dim_v), device=dev)
    layer.ckpt.copy_(S0_dev)
    layer.decode_step(*xs, o)                         # warm-up: epoch 0
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.decode_step(*xs, o)
    torch.cuda.synchronize()
    # the fold in fp64: S1 = alpha S0 + v k^T (window of one record)
    a, k, v, _ = (np.asarray(t, dtype=np.float64) for t in x)
    kk = np.repeat(k, sh.group, axis=1)
    S1 = a[..., None, None] * S0.astype(np.float64) + v[..., :, None] * kk[..., None, :]
    got = []
    for r in range(5):
        layer.ckpt.copy_(S0_dev)                      # same checkpoint and inputs every replay
        g.replay()
        torch.cuda.synchronize()
        ck = layer.ckpt.float().cpu().numpy().astype(np.float64)
        ref = stochastic.checkpoint_round(S1, seed, r + 1)
        diff = ck != ref
        # the kernel's fp32 fold may cross a rounding threshold the fp64 fold does not: rare
        assert diff.sum() <= max(2, 2e-3 * diff.size), (r, diff.mean())
        assert np.all(layer.fold_epochs() == r + 2)
        got.append(ck)
    for r in range(4):
        assert np.mean(got[r] != got[r + 1]) > 0.05, r  # new draws, not the captured ones
    assert layer.read_error() == 0
