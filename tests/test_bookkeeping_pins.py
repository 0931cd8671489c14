"""Pins of the integer buffer/pointer model against the pages' schedule."""
import numpy as np
import pytest

from oracle.bookkeeping import BufferModel
from ssm_layer_decode_amd import workloads as W


def test_tiny_workload_flushes_four_times_at_window_ends():
    """64 decode steps with L = 16 give 4 flushes (tiny correctness workload),
    at steps 16, 32, 48, 64: the fold happens on the step whose append fills
    the 16-record buffer ([ar] how ReplaySSM works; [ru] §03)."""
    sh = W.TINY
    m = BufferModel(sh.batch, sh.n_vheads, sh.n_kheads, sh.dim_v, sh.dim_k, sh.window)
    flush_steps = []
    for t in range(1, W.TINY_STEPS + 1):
        a, k, v, q = W.decode_inputs_np(sh, 0, t - 1)
        f = m.decode(a, k, v)
        assert f.all() or not f.any()
        if f.all():
            flush_steps.append(t)
        assert list(m.count) == [t % 16] * sh.batch
    assert flush_steps == [16, 32, 48, 64]


def test_buffer_holds_exact_input_copies():
    sh = W.Shape(batch=3, n_vheads=4, n_kheads=2, dim_v=5, dim_k=6, window=8, dist="uniform")
    m = BufferModel(3, 4, 2, 5, 6, 8)
    recs = []
    for t in range(5):
        a, k, v, q = W.decode_inputs_np(sh, 9, t)
        m.decode(a, k, v)
        recs.append((a, k, v))
    for j, (a, k, v) in enumerate(recs):
        assert m.kbuf[:, :, j].tobytes() == k.tobytes()
        assert m.vbuf[:, :, j].tobytes() == v.tobytes()
        assert m.abuf[:, :, j].tobytes() == a.tobytes()


def test_spec_verify_commit_schedule():
    """Drafts go after the committed records; commit advances the pointer by
    the accepted length and folds once it reaches L ([ru] §05; [zh] method
    points).  Readings: capacity L + T_max; commit folds everything committed."""
    L, T = 16, 4
    m = BufferModel(3, 2, 2, 4, 4, L, max_draft=T)
    m.count[:] = [0, 13, 15]
    rng = np.random.default_rng(0)
    a = rng.random((3, T, 2)).astype(np.float32)
    k = rng.random((3, T, 2, 4)).astype(np.float32)
    v = rng.random((3, T, 2, 4)).astype(np.float32)
    m.verify(a, k, v)
    assert list(m.count) == [0, 13, 15]            # verify never moves the pointer
    assert m.kbuf[1, :, 13:17].tobytes() == k[1].transpose(1, 0, 2).tobytes()
    f = m.commit(np.array([4, 3, 0]))
    assert list(f) == [False, True, False]
    assert list(m.count) == [4, 0, 15]
    m.verify(a, k, v)
    f = m.commit(np.array([0, 0, 1]))
    assert list(f) == [False, False, True]
    assert list(m.count) == [4, 0, 0]
    # slots of rejected drafts are stale: the next append overwrites slot 4
    a1, k1, v1 = a[:, 0], k[:, 0], v[:, 0]
    m.decode(a1, k1, v1)
    assert m.kbuf[0, :, 4].tobytes() == k1[0].tobytes()


def test_commit_without_verify_is_rejected():
    m = BufferModel(1, 1, 1, 2, 2, 4, max_draft=2)
    with pytest.raises(AssertionError):
        m.commit(np.array([1]))


def test_flush_folds_only_nonempty():
    m = BufferModel(3, 1, 1, 2, 2, 4)
    m.count[:] = [0, 2, 3]
    assert list(m.flush()) == [False, True, True]
    assert list(m.count) == [0, 0, 0]
