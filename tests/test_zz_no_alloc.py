"""replayssm_commit_static, the commit that allocates nothing: the fold list
lives in the library's own device array instead of the caller's work buffer.
Its results must equal replayssm_commit's bit for bit (same kernels, same
order): twin layers take the same verify/commit rounds, one committing with
its work buffer, the other (created without one) with the static array.  Two
runs in a row, the second on a smaller layer, so the array holds the first
run's list when the second starts."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from ssm_layer_decode_amd import _lib
from ssm_layer_decode_amd import workloads as W
from tests.helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    return torch.device("cuda:0")


def _same(A, E):
    pairs = [(A.ckpt, E.ckpt), (A.count, E.count), (A.kbuf, E.kbuf), (A.vbuf, E.vbuf), (A.abuf, E.abuf)]
    for n in ("read_copy", "row_scale", "folds"):
        if getattr(A, n) is not None:
            pairs.append((getattr(A, n), getattr(E, n)))
    return all(torch.equal(x, y) for x, y in pairs)


def _run(dev, sh, rounds, seed, **kw):
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    cfg = LayerConfig.of(sh, sr_seed=5, **kw)
    A = ReplaySSM(cfg, device=dev)
    E = ReplaySSM(cfg, device=dev, commit_work=False)
    assert E.work is None
    S0 = torch.from_numpy(W.initial_state_np(sh, seed, std=0.5))
    for L_ in (A, E):
        L_.ckpt.copy_(S0.to(L_.ckpt.dtype))
        if cfg.read_copy != "none":
            L_.refresh_read_copy()
    T = sh.max_draft
    folded = 0
    for r in range(rounds):
        d = [torch.from_numpy(x).to(dev) for x in W.draft_inputs_np(sh, seed + 1, r, T)]
        oa, oe = A.spec_verify(*d), E.spec_verify(*d)
        acc = torch.from_numpy(W.accepted_np(sh.batch, T, seed + 2, r)).to(dev)
        before = A.count.clone()
        A.commit(acc)
        E.commit_static(acc)
        torch.cuda.synchronize()
        folded += int(((before[:, 0] + acc) >= sh.window).sum())
        assert torch.equal(oa, oe), r
        assert _same(A, E), r
    assert A.read_error() == 0 and E.read_error() == 0
    assert folded > 0
    return folded


def test_commit_static_matches_commit(dev):
    big = W.Shape(batch=96, n_vheads=8, n_kheads=4, dim_v=16, dim_k=32, window=4, max_draft=4, dist="uniform")
    small = W.Shape(batch=5, n_vheads=4, n_kheads=2, dim_v=16, dim_k=32, window=4, max_draft=4, dist="uniform")
    say("case: static commit, 96 sequences x 8 heads")
    n1 = _run(dev, big, 10, 70)
    say("case: static commit, then 5 sequences x 4 heads (the array holds the larger list)")
    n2 = _run(dev, small, 10, 80)
    say(f"  folded sequences: {n1}, then {n2}")


@pytest.mark.parametrize("copy,ckpt", [("fp8", "f32"), ("mxfp4", "f16sr")])
def test_commit_static_with_copy_and_fp16_checkpoint(dev, copy, ckpt):
    sh = W.Shape(batch=7, n_vheads=4, n_kheads=2, dim_v=16, dim_k=64, window=6, max_draft=4, dist="uniform")
    say(f"case: static commit with {copy} copy, {ckpt} checkpoint")
    _run(dev, sh, 8, 90, read_copy=copy, ckpt=ckpt)
