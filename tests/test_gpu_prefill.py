"""GPU parity of prefill: a prompt of T tokens after h0 buffered records.

Against the oracle (recurrence.prefill, pinned to token-by-token decoding):
outputs within the fp32 tolerance; the checkpoint at the last window boundary
(fp32 within tolerance, or its stochastic fp16 rounding with the prefill's
launch number, up to the rare one-step flips of an fp32-vs-fp64 fold); the
record count and the buffered records bit for bit; the read copy equal to the
encoding of the stored checkpoint; and decoding after the prefill continuing
eq.R.  Cases include key groups split over several tiles with records already
buffered (the key appends run after the prefill kernel for that reason), and
both kernels: the matrix-core one (16-record windows, P and N multiples of
16) and the VALU one (other windows).
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import bookkeeping, quant, recurrence, stochastic
from ssm_layer_decode_amd import workloads as W
from tests.helpers import (check_fp8_ckpt, fp8_ckpt_values, matrix_err, normwise_err, raw_bits, np_bits, say,
                           set_fp8_ckpt, to_dev, unpack_e2m1)

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ssm_layer_decode_amd import _lib
    _lib.load()
    return torch.device("cuda:0")


def _ulp16(a):
    a = np.abs(a)
    e = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -14)
    return np.ldexp(1.0, (e - 10).astype(np.int64))


CASES = [
    # (Hv, Hk, P, N, L, h0, T, in_dtype, ckpt, copy, hvpt)
    (4, 4, 16, 32, 8, 0, 37, "f32", "f32", "none", 0),
    (4, 2, 20, 32, 8, 3, 5, "f32", "f32", "none", 0),          # no window completed
    (4, 2, 16, 64, 8, 5, 11, "bf16", "f32", "none", 0),
    (8, 2, 12, 32, 6, 4, 29, "f32", "f32", "none", 2),          # key group split over tiles, h0 > 0, folds
    (8, 2, 12, 32, 6, 2, 16, "bf16", "f32", "none", 8),         # tile of two whole key groups
    (4, 4, 64, 128, 16, 7, 41, "f32", "f32", "fp8", 0),
    (4, 4, 32, 128, 16, 0, 32, "f32", "f16sr", "none", 0),
    (4, 2, 16, 64, 8, 2, 23, "f32", "f16sr", "mxfp4", 0),
    (2, 2, 128, 128, 16, 9, 20, "bf16", "f32", "bf16", 0),      # 16 rows per thread
    (2, 1, 8, 16, 4, 1, 9, "f32", "f32", "none", 0),
    (3, 3, 32, 256, 32, 30, 40, "f32", "f32", "none", 0),       # chunks split a 32-record window
    # L = 16 with P, N multiples of 16 take the matrix-core kernel (the cases above with L = 16 too)
    (8, 2, 48, 64, 16, 5, 40, "f32", "f32", "none", 2),         # one wave without a p block; split key group
    (32, 2, 64, 128, 16, 5, 40, "f32", "f32", "none", 0),      # keys shared by 16 heads, Mamba-2 head dims
    (32, 2, 64, 128, 16, 0, 37, "bf16", "f16sr", "mxfp4", 4),  # the same with 4-head tiles and a copy
    (16, 1, 128, 128, 16, 11, 33, "f32", "f32", "none", 0),    # two p blocks per wave with fp32 inputs
    (2, 1, 16, 16, 16, 3, 21, "bf16", "f32", "none", 0),
    (2, 2, 256, 64, 16, 0, 35, "f32", "f16sr", "mxfp4", 0),     # four p blocks per wave
    (2, 2, 128, 128, 16, 4, 33, "f32", "f32", "none", 0),       # two p blocks, fp32 inputs loaded item by item
    (2, 2, 64, 256, 16, 2, 30, "f32", "f32", "none", 0),        # 16 column groups per row
    # fp8 checkpoint (read through a copy): the matrix-core kernel and the VALU kernel
    (4, 4, 64, 128, 16, 3, 37, "f32", "fp8sr", "mxfp4", 0),
    (4, 2, 32, 64, 16, 0, 16, "bf16", "fp8sr", "fp8", 2),
    (4, 2, 16, 64, 8, 2, 23, "f32", "fp8sr", "mxfp4", 0),
    (2, 2, 128, 128, 16, 4, 33, "f32", "fp8sr", "bf16", 0),
]


def _prefill_supported(P, N, L):
    """The library's prefill limits: the matrix-core kernel for 16-record
    windows with P, N multiples of 16 and at most 16 state blocks per wave,
    else the VALU kernel (up to 16 rows per thread); LDS within 64 KiB."""
    npb = 1 if P <= 64 else 2 if P <= 128 else 4
    if L == 16 and P % 16 == 0 and N % 16 == 0 and npb * (N // 16) <= 16:
        lds = (16 * (N + 4) + 16 * (N + 16) + 16 * (64 * npb + 16) + 16 + 5 * 16 * 17 + 2 * 16 + 4) * 4
    else:
        rpp, npr = 1024 // N, 2
        while npr * rpp < P and npr < 16:
            npr *= 2
        if npr * rpp < P:
            return False
        lds = (L * N + L * P + ((L + 3) & ~3) + 16 * N + L * 16 + 16 * P + 4) * 4
    return lds <= 64 * 1024


def _random_cases(n, seed=8800):
    """Seeded layer shapes, prompt lengths and buffered-record counts that the
    library accepts (half with 16-record windows, the matrix-core path)."""
    from ssm_layer_decode_amd import _lib
    from ssm_layer_decode_amd.replayssm import LayerConfig, replayssm_query_sizes
    rng = np.random.default_rng(seed)
    rng_fp8 = np.random.default_rng(seed + 1)
    out = []
    while len(out) < n:
        N = int(rng.choice([16, 32, 64, 128, 256]))
        P = (16 * int(rng.integers(1, 9))) if rng.random() < 0.5 else 4 * int(rng.integers(1, 33))
        L = 16 if rng.random() < 0.5 else int(rng.choice([1, 2, 4, 5, 8, 32]))
        g, Hk = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        Hv = g * Hk
        T, h0 = int(rng.integers(1, 41)), int(rng.integers(0, L))
        in_dtype = str(rng.choice(["f32", "bf16"]))
        ckpt = "f16sr" if rng.random() < 0.3 else "f32"
        copy = "none" if rng.random() < 0.6 else str(rng.choice(["bf16", "fp8", "mxfp4"]))
        if ckpt == "f32" and copy != "none" and rng_fp8.random() < 0.4:
            ckpt = "fp8sr"                                 # drawn apart: the other draws stay as they were
        tiles = [d for d in range(1, g + 1) if g % d == 0] + [m for m in range(2 * g, Hv + 1, g) if Hv % m == 0]
        hvpt = 0 if rng.random() < 0.6 else int(rng.choice(tiles))
        if (copy == "mxfp4" and N < 32) or hvpt * P > 1024 or not _prefill_supported(P, N, L):
            continue
        sh = W.Shape(batch=3, n_vheads=Hv, n_kheads=Hk, dim_v=P, dim_k=N, window=L, in_dtype=in_dtype)
        try:
            replayssm_query_sizes(LayerConfig.of(sh, read_copy=copy, ckpt=ckpt, heads_per_tile=hvpt))
        except _lib.RssmError:
            continue
        out.append((Hv, Hk, P, N, L, h0, T, in_dtype, ckpt, copy, hvpt))
    return out


@pytest.mark.parametrize("Hv,Hk,P,N,L,h0,T,in_dtype,ckpt,copy,hvpt", CASES)
def test_prefill_matches_oracle(dev, Hv, Hk, P, N, L, h0, T, in_dtype, ckpt, copy, hvpt):
    _check_prefill(dev, Hv, Hk, P, N, L, h0, T, in_dtype, ckpt, copy, hvpt)


@pytest.mark.parametrize("Hv,Hk,P,N,L,h0,T,in_dtype,ckpt,copy,hvpt",
                         _random_cases(40 * max(1, int(os.environ.get("RSSM_RANDOM_SCALE", "1")))))
def test_prefill_random_shapes(dev, Hv, Hk, P, N, L, h0, T, in_dtype, ckpt, copy, hvpt):
    _check_prefill(dev, Hv, Hk, P, N, L, h0, T, in_dtype, ckpt, copy, hvpt)


def _check_prefill(dev, Hv, Hk, P, N, L, h0, T, in_dtype, ckpt, copy, hvpt):
    from ssm_layer_decode_amd.replayssm import LayerConfig, ReplaySSM
    sh = W.Shape(batch=3, n_vheads=Hv, n_kheads=Hk, dim_v=P, dim_k=N, window=L, in_dtype=in_dtype,
                 dist="uniform")
    g = sh.group
    seed = 77
    say(f"case: prefill Hv={Hv} Hk={Hk} P={P} N={N} L={L} h0={h0} T={T} {in_dtype} ckpt={ckpt} copy={copy} hvpt={hvpt}")
    S0 = W.initial_state_np(sh, 50 + N, std=0.5)
    if ckpt == "f16sr":
        S0 = S0.astype(np.float16).astype(np.float64)
    layer = ReplaySSM(LayerConfig.of(sh, read_copy=copy, ckpt=ckpt, sr_seed=seed, heads_per_tile=hvpt), device=dev)
    if ckpt == "fp8sr":
        S0 = set_fp8_ckpt(layer, S0)                  # the values the fp8 checkpoint holds
    else:
        layer.ckpt.copy_(torch.from_numpy(S0).to(layer.ckpt.dtype))
    if copy != "none":
        layer.refresh_read_copy()
    bm = bookkeeping.BufferModel(3, Hv, Hk, P, N, L, store_dtype=np.float32)
    buffered = [W.decode_inputs_np(sh, 51, t) for t in range(h0)]
    for x in buffered:
        layer.decode_step(*to_dev(x, dev, in_dtype))
        bm.decode(x[0], x[1], x[2])
    a, k, v, q = W.draft_inputs_np(sh, 52, 0, T)
    epoch = layer.fold_epochs() if ckpt != "f32" else None
    O = layer.prefill(*to_dev((a, k, v, q), dev, in_dtype)).cpu().numpy()
    bm.prefill(a, k, v)
    O_ref, S_new, folds = recurrence.prefill(S0, [(x[0], x[1], x[2]) for x in buffered], (a, k, v, q), L, group=g)
    assert normwise_err(O, O_ref) <= TOL, normwise_err(O, O_ref)
    ck = fp8_ckpt_values(layer) if ckpt == "fp8sr" else layer.ckpt.float().cpu().numpy().astype(np.float64)
    if folds == 0:
        np.testing.assert_array_equal(ck, S0)
    elif ckpt == "f32":
        assert matrix_err(ck, S_new) <= TOL
    elif ckpt == "fp8sr":
        check_fp8_ckpt(layer, S_new, seed, epoch, "prefill fold")
    else:
        ref = stochastic.checkpoint_round(S_new, seed, epoch)
        diff = ck != ref
        assert np.all(np.abs(ck - ref)[diff] <= _ulp16(np.maximum(np.abs(ck), np.abs(ref)))[diff])
        assert diff.sum() <= max(2, 2e-3 * diff.size), diff.mean()   # rare flips; at least 2 allowed
    cnt = layer.count.cpu().numpy()
    assert np.all(cnt == (h0 + T) % L)
    hp = (h0 + T) % L
    np.testing.assert_array_equal(raw_bits(layer.kbuf)[:, :, :hp], np_bits(bm.kbuf[:, :, :hp], in_dtype))
    np.testing.assert_array_equal(raw_bits(layer.vbuf)[:, :, :hp], np_bits(bm.vbuf[:, :, :hp], in_dtype))
    np.testing.assert_array_equal(layer.abuf.cpu().numpy()[:, :, :hp], bm.abuf[:, :, :hp])
    if copy != "none":
        R, sc = quant.quantize(ck.astype(np.float32), copy)
        got = layer.read_copy
        if copy == "bf16":
            np.testing.assert_array_equal(raw_bits(got), R)
        elif copy == "fp8":
            gr = got.cpu().numpy().astype(np.int64)
            np.testing.assert_array_equal(np.where((gr & 0x7F) == 0, 0, gr), np.where((R & 0x7F) == 0, 0, R))
            np.testing.assert_array_equal(layer.row_scale.cpu().numpy(), sc)
        else:
            np.testing.assert_array_equal(unpack_e2m1(got.cpu().numpy()), R)
            np.testing.assert_array_equal(layer.row_scale.cpu().numpy(), sc)
    # decoding continues from the prefilled state (fp32 paths: eq.R over everything)
    if ckpt == "f32" and copy == "none":
        more = [W.decode_inputs_np(sh, 53, t) for t in range(L + 3)]
        steps = [(x[0], x[1], x[2], np.zeros_like(x[1])) for x in buffered] + \
                [(a[:, t], k[:, t], v[:, t], q[:, t]) for t in range(T)] + more
        ref, _, _ = recurrence.decode(S0, steps, group=g)
        for i, x in enumerate(more):
            o = layer.decode_step(*to_dev(x, dev, in_dtype)).cpu().numpy()
            assert normwise_err(o, ref[h0 + T + i]) <= TOL, i
    assert layer.read_error() == 0
    if ckpt != "f32":
        assert np.all(layer.fold_epochs() == epoch + (1 if folds else 0))   # a prefill stores one fold
