"""fp16 and fp8 checkpoints with stochastic rounding -- TEST INFRASTRUCTURE ONLY.

The pages note that keeping the recurrent checkpoint in FP16 with stochastic
rounding stays close to FP32 ([ru] §06, last paragraph; [ar] section on
limiting quantization error mentions FP16 or FP8 recurrence with
low-precision reads).  They give no rounding recipe, so this library's
definition (a reading, stated once here and in include/replayssm.h):

* Random bits.  The random numbers cannot be passed in (one per state entry
  per fold), so both sides compute them from one published counter-based
  hash: ``pcg_hash`` of Jarzynski and Olano, "Hash Functions for GPU
  Rendering" (JCGT 2020) -- an LCG step followed by PCG's RXS-M-XS output
  permutation on 32 bits.  For a fold with epoch E -- the number of folds
  the sequence stored before it (every call that writes the checkpoint, one
  fold each: a decode step that fills the window, a flush, a commit that
  folds, a prefill that completes a window; counted per sequence from 0) --
  and the layer's seed s:
      key = h(lo32(s) ^ h(hi32(s) ^ h(lo32(E) ^ h(hi32(E)))))
  and checkpoint entry g (its flat index in [B][Hv][P][N]) draws
      w = h(key ^ (g >> 1));  u16 = low 16 bits of w if g is even, else high.
* Rounding.  For the fp32 value x of the folded entry (the decision is taken
  in fp32, the kernel's precision): a = |x|, e = max(floor(log2 a), -14)
  (-14 also for a = 0), q = 2^(e - 10) the fp16 spacing at a, m = a / q,
  f = floor(m), p = m - f (all exact).  The result is (f + 1) q if
  u16 / 2^16 < p, else f q; saturated at 65504; with the sign of x.  An
  infinity stays infinite and NaN stays NaN.  So the expected result over
  u16 equals x exactly wherever p is a multiple of 2^-16 (the whole fp16
  normal range).

parity pins (tests/test_stochastic_pins.py): the hash is a bijection with
uniform output bytes; rounding leaves fp16 values unchanged, always returns
one of the two fp16 neighbours (found by numpy's float16 arithmetic), and its
mean over all 65536 draws equals x exactly in the normal range; the
checkpoint path reduces to eq.R when every fold result is an fp16 value.
fp8: every result is one of the two neighbours of |y| found by search over
the e4m3 code table, grid values are kept and values beyond 448 saturate for
every draw, u = 0 rounds every off-grid value up and the largest draw rounds
down; the mean over all draws is within step * 2^-16 of y and exact where the
dropped fraction is a multiple of 2^-16; rows on the grid (amax 448 * 2^s)
store sigma = 2^s and decode exactly; sigma is the smallest power of two with
amax <= 448 sigma; the split path stores the rounding of eq.R's fold with
epochs 0, 1, ...
"""
from __future__ import annotations

import numpy as np

M32 = 0xFFFFFFFF


def pcg_hash(x):
    """32-bit pcg_hash (uint32 in, uint32 out), vectorised."""
    x = np.asarray(x, dtype=np.uint64) & np.uint64(M32)
    state = (x * np.uint64(747796405) + np.uint64(2891336453)) & np.uint64(M32)
    shift = (state >> np.uint64(28)) + np.uint64(4)
    word = (((state >> shift) ^ state) * np.uint64(277803737)) & np.uint64(M32)
    return ((word >> np.uint64(22)) ^ word).astype(np.uint64) & np.uint64(M32)


def fold_key(seed: int, epoch: int) -> int:
    """Key of one fold from the layer seed and the fold's epoch."""
    h = lambda v: int(pcg_hash(np.uint64(v & M32)))
    return h((seed & M32) ^ h(((seed >> 32) & M32) ^ h((epoch & M32) ^ h((epoch >> 32) & M32))))


def uniform16(key: int, g):
    """16-bit draw of checkpoint entry g (flat index) under `key`."""
    g = np.asarray(g, dtype=np.uint64)
    w = pcg_hash(np.uint64(key) ^ ((g >> np.uint64(1)) & np.uint64(M32)))
    return np.where((g & np.uint64(1)) == 0, w & np.uint64(0xFFFF), w >> np.uint64(16)).astype(np.int64)


F16_MAX = 65504.0


def round_f16_stochastic(x32, u16):
    """fp32 values -> fp16 values (as float64), stochastic rounding with the
    16-bit draws u16 (same shape)."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    _, fe = np.frexp(a)                           # a = m 2^fe, m in [0.5, 1)
    e = np.where(a > 0, fe - 1, -14)
    e = np.maximum(e, -14)
    q = np.ldexp(1.0, e - 10)
    with np.errstate(invalid="ignore"):          # inf and nan: replaced below
        m = a / q
        f = np.floor(m)
        p = m - f
        up = (np.asarray(u16, dtype=np.float64) / 65536.0) < p
        r = np.minimum((f + up) * q, F16_MAX)
    r = np.where(np.isinf(a), np.inf, r)
    r = np.where(np.signbit(x), -r, r)
    return np.where(np.isnan(x), np.nan, r)


def checkpoint_round(S_new, seed: int, epoch):
    """Stochastic fp16 rounding of a whole folded checkpoint [B][Hv][P][N]
    (fp64 fold; the decision is taken on its fp32 value).  epoch: the fold's
    epoch, one for all sequences or one per sequence ([B])."""
    S32 = np.asarray(S_new, dtype=np.float64).astype(np.float32)
    g = np.arange(S32.size, dtype=np.uint64).reshape(S32.shape)
    ep = np.broadcast_to(np.asarray(epoch, dtype=np.int64), S32.shape[:1])
    u = np.empty(S32.shape, dtype=np.int64)
    for b in range(S32.shape[0]):
        u[b] = uniform16(fold_key(seed, int(ep[b])), g[b])
    return round_f16_stochastic(S32, u)


# ------------------------------------------------------------------ fp8
# The fp8 recurrent checkpoint ([ar] section on limiting quantization error:
# low-precision reads with an FP16 or FP8 recurrence; no recipe given).  This
# library's reading: each checkpoint row is stored as OCP e4m3fn codes with
# one scale sigma = 2^s, the smallest power of two with amax <= 448 sigma
# (amax the row's largest magnitude, NaN entries ignored; s clamped to
# [-126, 127]; sigma = 1 for a row with no nonzero entry, +inf for a row with
# an infinite entry), so that y = x / sigma is exact, as for the power-of-two
# block scales of the MX formats; the code of entry x is the stochastic
# rounding of y between its two neighbouring e4m3 values, with the same draws
# as the fp16 checkpoint.
E4M3_MAX = 448.0


def fp8_row_scale(amax32):
    """sigma = 2^s, the smallest power of two with amax <= 448 sigma: with
    amax = m 2^E (m in [1, 2)), s = E - 8, plus 1 if m > 1.75; s in
    [-126, 127]; 1 where amax is 0, +inf where it is infinite."""
    a = np.asarray(amax32, dtype=np.float32).astype(np.float64)
    fin = np.isfinite(a) & (a > 0)
    ac = np.where(fin, a, 1.0)
    m, e = np.frexp(ac)                           # ac = m 2^e, m in [0.5, 1)
    s = (e - 1) - 8 + (2.0 * m > 1.75)
    s = np.clip(s, -126, 127)
    sig = np.where(fin, np.ldexp(1.0, s), 1.0)
    sig = np.where(np.isinf(a), np.inf, sig)
    return sig.astype(np.float32)


def round_e4m3_stochastic(y32, u16):
    """fp32 values already divided by their row scale -> e4m3fn values (as
    float64), stochastic rounding with the 16-bit draws u16: up to the next
    e4m3 step iff u16 / 2^16 < p, p the dropped fraction of the step at |y|
    (steps 2^(e-3), e = max(floor(log2|y|), -6)); saturating at 448, sign
    kept.  e4m3fn has no infinity: a non-finite y gives NaN."""
    y = np.asarray(y32, dtype=np.float32).astype(np.float64)
    fin = np.isfinite(y)
    a = np.where(fin, np.abs(y), 0.0)
    _, fe = np.frexp(a)                           # a = m 2^fe, m in [0.5, 1)
    e = np.maximum(np.where(a > 0, fe - 1, -6), -6)
    q = np.ldexp(1.0, e - 3)
    m = a / q
    f = np.floor(m)
    p = m - f
    up = (np.asarray(u16, dtype=np.float64) / 65536.0) < p
    r = np.minimum((f + up) * q, E4M3_MAX)
    r = np.where(np.signbit(y), -r, r)
    return np.where(fin, r, np.nan)


def checkpoint_round_fp8(S_new, seed: int, epoch):
    """Stochastic e4m3 rounding of a whole folded checkpoint [B][Hv][P][N]
    (fp64 fold; scale and decision taken on its fp32 values).  Returns
    (codes uint8 [B][Hv][P][N], sigma float32 [B][Hv][P]); a NaN code is 0x7f.
    epoch: one for all sequences or one per sequence ([B])."""
    from . import quant
    with np.errstate(over="ignore"):                  # fl32: values beyond the fp32 range become infinite
        S32 = np.asarray(S_new, dtype=np.float64).astype(np.float32)
    with np.errstate(invalid="ignore"):
        amax = np.max(np.where(np.isnan(S32), np.float32(0.0), np.abs(S32)), axis=-1)
        sig = fp8_row_scale(amax)
        # y = x / sigma: exact for a power of two (in float64, then to fp32: exact
        # but for results below the fp32 normal range, which round as fp32 does)
        y = (S32.astype(np.float64) / sig[..., None].astype(np.float64)).astype(np.float32)
    g = np.arange(S32.size, dtype=np.uint64).reshape(S32.shape)
    ep = np.broadcast_to(np.asarray(epoch, dtype=np.int64), S32.shape[:1])
    u = np.empty(S32.shape, dtype=np.int64)
    for b in range(S32.shape[0]):
        u[b] = uniform16(fold_key(seed, int(ep[b])), g[b])
    vals = round_e4m3_stochastic(y, u)
    codes = quant.e4m3_encode(vals)               # exact: every value is an e4m3 value
    codes = np.where(np.isnan(vals), np.uint8(0x7F), codes).astype(np.uint8)
    return codes, sig


def fp8_checkpoint_values(codes, sig):
    """Stored fp8 checkpoint -> its values (float64, exact products)."""
    from . import quant
    return quant.e4m3_decode(codes) * np.asarray(sig, dtype=np.float64)[..., None]

