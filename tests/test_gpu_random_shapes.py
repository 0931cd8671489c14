"""Seeded random-shape parity sweep through the C ABI against the fp64 oracle.

Each case draws one layer shape from the ranges the library accepts (key dims
16-256, value dims 4-96 in steps of 4, one to four value heads per key head,
windows 1-32, 0-8 drafts, fp32 or bf16 inputs, default or explicit tiles of
part of a key group or of several key groups), skips it on the host when its
tiles exceed shared memory, and then runs decode steps over whole and partial
windows (eq.R stepped by the oracle) and, with drafts, verify/commit rounds
(verify = eq.R continued on a copy, commit = the state after the accepted
prefix) with pointers and buffers compared bit for bit.

A second sweep draws read copies (bf16, fp8, MXFP4) and the fp16 checkpoint:
verification of drafts from a refreshed copy must match the oracle's
split-precision verify, which reads the copy the same way.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import lowprec
from ssm_layer_decode_amd import _lib
from ssm_layer_decode_amd import workloads as W
from ssm_layer_decode_amd.replayssm import LayerConfig, replayssm_query_sizes
from tests.helpers import normwise_err, say, set_fp8_ckpt, to_dev
from tests.test_gpu_parity import TOL, _layer, run_decode, run_spec

pytestmark = pytest.mark.gpu

# RSSM_RANDOM_SCALE multiplies the number of cases for longer sweeps
_SCALE = max(1, int(os.environ.get("RSSM_RANDOM_SCALE", "1")))
N_FP32_CASES = 96 * _SCALE
N_COPY_CASES = 48 * _SCALE


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _lib.load()
    return torch.device("cuda:0")


def _tile_choices(Hv, g):
    """Explicit tiles the library accepts: divisors of g, or multiples of g dividing Hv."""
    part = [d for d in range(1, g + 1) if g % d == 0]
    whole = [m for m in range(2 * g, Hv + 1, g) if Hv % m == 0]
    return part + whole


def _supported(sh, **kw):
    try:
        replayssm_query_sizes(LayerConfig.of(sh, **kw))
        return True
    except _lib.RssmError:
        return False


def _draw_fp32_case(i):
    rng = np.random.default_rng(9100 + i)
    while True:
        N = int(rng.choice([16, 32, 64, 128, 256]))
        P = 4 * int(rng.integers(1, 25))
        g = int(rng.integers(1, 5))
        Hk = int(rng.integers(1, 4))
        Hv = g * Hk
        L = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 32]))
        T = int(rng.choice([0, 1, 2, 3, 4, 8]))
        in_dtype = str(rng.choice(["f32", "bf16"]))
        B = int(rng.integers(1, 4))
        tiles = _tile_choices(Hv, g)
        hvpt = 0 if rng.random() < 0.5 else int(rng.choice(tiles))
        sh = W.Shape(batch=B, n_vheads=Hv, n_kheads=Hk, dim_v=P, dim_k=N, window=L, max_draft=T,
                     in_dtype=in_dtype, dist="uniform")
        if hvpt * P <= 1024 and _supported(sh, heads_per_tile=hvpt):
            return sh, hvpt


@pytest.mark.parametrize("i", range(N_FP32_CASES))
def test_random_shape_fp32(dev, i):
    sh, hvpt = _draw_fp32_case(i)
    L, T = sh.window, sh.max_draft
    say(f"case {i}: B={sh.batch} Hv={sh.n_vheads} Hk={sh.n_kheads} P={sh.dim_v} N={sh.dim_k} "
        f"L={L} T={T} {sh.in_dtype} hvpt={hvpt}")
    S0 = W.initial_state_np(sh, 300 + i, std=0.5)
    steps = 2 * L + 1 + i % 3
    _, _, _, _, _, nf = run_decode(sh, steps, dev, seed=i, S0=S0, heads_per_tile=hvpt)
    assert nf == steps // L
    if T > 0:
        run_spec(sh, 6 + i % 4, dev, seed=i, S0=S0, heads_per_tile=hvpt)


def _draw_copy_case(i):
    rng = np.random.default_rng(9700 + i)
    rng_fp8 = np.random.default_rng(19700 + i)            # drawn apart: the other draws stay as they were
    while True:
        N = int(rng.choice([32, 64, 128, 256]))
        P = 4 * int(rng.integers(1, 17))
        g = int(rng.integers(1, 5))
        Hk = int(rng.integers(1, 3))
        Hv = g * Hk
        L = int(rng.choice([4, 8, 16]))
        T = int(rng.choice([1, 2, 4, 8]))
        in_dtype = str(rng.choice(["f32", "bf16"]))
        fmt = str(rng.choice(["bf16", "fp8", "mxfp4", "f16sr"]))
        hvpt = 0 if rng.random() < 0.6 else int(rng.choice(_tile_choices(Hv, g)))
        sh = W.Shape(batch=int(rng.integers(1, 4)), n_vheads=Hv, n_kheads=Hk, dim_v=P, dim_k=N,
                     window=L, max_draft=T, in_dtype=in_dtype, dist="uniform")
        kw = dict(ckpt="f16sr") if fmt == "f16sr" else dict(read_copy=fmt)
        if fmt != "f16sr" and rng_fp8.random() < 0.3:
            kw["ckpt"] = "fp8sr"                           # an fp8 checkpoint under the copy
        if hvpt * P <= 1024 and _supported(sh, heads_per_tile=hvpt, **kw):
            return sh, fmt, kw, hvpt


@pytest.mark.parametrize("i", range(N_COPY_CASES))
def test_random_shape_verify_reads_copy(dev, i):
    """No fold happens before the verify, so the copy (or the fp16 checkpoint)
    is exactly what the oracle's split verify reads."""
    sh, fmt, kw, hvpt = _draw_copy_case(i)
    T = sh.max_draft
    say(f"case {i}: B={sh.batch} Hv={sh.n_vheads} Hk={sh.n_kheads} P={sh.dim_v} N={sh.dim_k} "
        f"L={sh.window} T={T} {sh.in_dtype} {fmt} ckpt={kw.get('ckpt', 'f32')} hvpt={hvpt}")
    S0 = W.initial_state_np(sh, 400 + i, std=0.5)
    if fmt == "f16sr":
        S0 = S0.astype(np.float16).astype(np.float64)
    layer = _layer(sh, dev, heads_per_tile=hvpt, **kw)
    if kw.get("ckpt") == "fp8sr":
        S0 = set_fp8_ckpt(layer, S0)                    # the values the fp8 checkpoint holds
    else:
        layer.ckpt.copy_(torch.from_numpy(S0))
    if fmt != "f16sr":
        layer.refresh_read_copy()
    nrec = min(sh.window - 1, 1 + i % 3)
    recs = [W.decode_inputs_np(sh, 500 + i, t) for t in range(nrec)]
    for x in recs:
        layer.decode_step(*to_dev(x, dev, sh.in_dtype))
    drafts = W.draft_inputs_np(sh, 600 + i, T, T)
    O = layer.spec_verify(*to_dev(drafts, dev, sh.in_dtype)).cpu().numpy()
    read = "none" if fmt == "f16sr" else fmt          # fp16 checkpoint entries are exact fp32 values
    ref = lowprec.split_read_verify(S0.astype(np.float64), [(x[0], x[1], x[2]) for x in recs], drafts,
                                    read, group=sh.group)
    e = normwise_err(O, ref)
    assert e <= TOL, e
    layer.commit(torch.zeros(sh.batch, dtype=torch.int32, device=dev))
    assert layer.read_error() == 0
