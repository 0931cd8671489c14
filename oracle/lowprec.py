"""Split-precision read path and the fully quantised arm -- TEST INFRASTRUCTURE ONLY.

Split precision ([ru] §06; [ar] "limiting quantization error"; [zh] method
points): the recurrence keeps a high-precision checkpoint; a low-precision
copy is written next to it at every flush, from the same folded state, and is
read only by the non-flush output computation.  Its rounding therefore touches
the outputs of the current window and never re-enters the recurrence.

This is an approximation, so the oracle follows the algorithm's steps (in
fp64 arithmetic; quantisation decisions in fp32, the precision of the
checkpoint the copy is made from):

  1. the checkpoint evolves exactly as in the fp32 path (eq.R / eq.U folds);
  2. each fold also produces R = Q(S_new);
  3. a non-flush step outputs gamma_h * (deq(R) q) + sum_j gamma_{j+1:h} v_j (k_j . q)
     (eq.U applied to q, with eq.O1 per record);
  4. a flush step outputs S_new q from the high-precision fold.

The fully quantised arm ([ru] §02 problem 3 and §06; [ar] same section) is
conventional decoding whose stored state is Q(S) after every step, so the
rounding of step t feeds step t+1.  Its output at step t is taken from the
unrounded in-register S_t (reading adopted so that feedback through the stored
state is the only difference from the split path).

parity: pinned by reduction -- with Q the identity both functions equal eq.R
(tests/test_oracle_pins.py); the quantiser itself is pinned in quant.py.
"""
from __future__ import annotations

import numpy as np

from . import quant
from .recurrence import eqR_step, _expand_keys


def split_read_decode(S0, step_inputs, window: int, fmt: str, group: int = 1,
                      keep_folds: bool = False, ckpt: str = "exact", seed: int = 0, epoch0: int = 0):
    """Outputs of the split-precision path over ``step_inputs``.

    S0 [B][Hv][P][N]; the read copy of S0 is Q(S0) (as after a refresh).
    fmt 'none' | 'bf16' | 'fp8' | 'mxfp4'.  ckpt 'exact': the checkpoint
    keeps each fold's fp64 value; 'f16sr': it stores the fold rounded to fp16
    stochastically (stochastic.checkpoint_round) with epoch epoch0 + i for
    the i-th fold of the run (counted from 0; all sequences fold together);
    'fp8sr': it stores the fold as row-scaled e4m3 codes rounded
    stochastically (stochastic.checkpoint_round_fp8, same epochs; an fp8
    checkpoint is always read through a copy, fmt != 'none').  The read
    copy is always made from the unrounded fold, and a flush step's output
    from the unrounded fold too.  Returns (outputs [steps][B][Hv][P], folds)
    where folds maps the 1-based flush step to the stored checkpoint.
    """
    from . import stochastic
    S_ckpt = np.array(S0, dtype=np.float64, copy=True)
    R = quant.roundtrip(S_ckpt, fmt)
    recs = []                       # (alpha, k expanded to value heads, v)
    outs, folds = [], {}
    nfold = 0
    for t, (a, k, v, q) in enumerate(step_inputs, start=1):
        a = np.asarray(a, dtype=np.float64)
        kk = _expand_keys(np.asarray(k, dtype=np.float64), group)
        vv = np.asarray(v, dtype=np.float64)
        qq = _expand_keys(np.asarray(q, dtype=np.float64), group)
        recs.append((a, kk, vv))
        h = len(recs)
        if h == window:
            S = S_ckpt
            for (aj, kj, vj) in recs:           # fold = eq.R over the window
                S = aj[..., None, None] * S + vj[..., :, None] * kj[..., None, :]
            recs = []
            outs.append(np.matmul(S, qq[..., :, None])[..., 0])
            if ckpt == "exact":
                S_ckpt = S
            elif ckpt == "f16sr":
                S_ckpt = stochastic.checkpoint_round(S, seed, epoch0 + nfold)
            else:
                S_ckpt = stochastic.fp8_checkpoint_values(*stochastic.checkpoint_round_fp8(S, seed, epoch0 + nfold))
            nfold += 1
            # without a copy, non-flush steps read the stored checkpoint
            R = S_ckpt if (fmt == "none" and ckpt != "exact") else quant.roundtrip(S, fmt)
            if keep_folds:
                folds[t] = S_ckpt.copy()
        else:
            gam = np.ones_like(a)
            for (aj, _, _) in recs:
                gam = gam * aj
            o = gam[..., None] * np.matmul(R, qq[..., :, None])[..., 0]
            c = np.ones_like(a)                 # gamma_{j+1:h}, walking back from j = h
            for (aj, kj, vj) in reversed(recs):
                s = np.sum(kj * qq, axis=-1)
                o = o + (c * s)[..., None] * vj
                c = c * aj
            outs.append(o)
    return np.stack(outs), folds


def split_read_verify(S_ckpt, records, drafts, fmt: str, group: int = 1):
    """Output-only verification of T drafts on the split-precision path
    ([zh] method points, the T-query chunk; [ru] §05 and §06).

    S_ckpt [B][Hv][P][N]: the high-precision checkpoint; its read copy is
    Q(S_ckpt).  records: the (alpha, k, v) step inputs committed since the
    checkpoint, oldest first (h of them).  drafts: (alpha [B][T][Hv],
    k [B][T][Hk][N], v [B][T][Hv][P], q [B][T][Hk][N]).  Column t (1-based)
    is the unrolled window at position h + t applied to q_t, with deq(R) in
    place of S_ckpt -- the same steps as a non-flush decode output.
    Returns O [B][T][Hv][P].
    """
    R = quant.roundtrip(np.asarray(S_ckpt, dtype=np.float64), fmt)
    recs = [(np.asarray(a, dtype=np.float64), _expand_keys(np.asarray(k, dtype=np.float64), group),
             np.asarray(v, dtype=np.float64)) for (a, k, v) in records]
    da, dk, dv, dq = (np.asarray(x, dtype=np.float64) for x in drafts)
    T = da.shape[1]
    cols = []
    for t in range(T):
        recs.append((da[:, t], _expand_keys(dk[:, t], group), dv[:, t]))
        qq = _expand_keys(dq[:, t], group)
        gam = np.ones_like(da[:, t])
        for (aj, _, _) in recs:
            gam = gam * aj
        o = gam[..., None] * np.matmul(R, qq[..., :, None])[..., 0]
        c = np.ones_like(gam)
        for (aj, kj, vj) in reversed(recs):
            o = o + (c * np.sum(kj * qq, axis=-1))[..., None] * vj
            c = c * aj
        cols.append(o)
    return np.stack(cols, axis=1)


def quantized_state_decode(S0, step_inputs, fmt: str, group: int = 1):
    """Conventional decoding with the stored state rounded to ``fmt`` after
    every step.  Returns outputs [steps][B][Hv][P]."""
    Sq = quant.roundtrip(np.asarray(S0, dtype=np.float64), fmt)
    outs = []
    for (a, k, v, q) in step_inputs:
        S, o = eqR_step(Sq, a, k, v, q, group)
        outs.append(o)
        Sq = quant.roundtrip(S, fmt)
    return np.stack(outs)
