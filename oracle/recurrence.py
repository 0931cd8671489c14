"""eq.R in fp64, stepped one token at a time -- TEST INFRASTRUCTURE ONLY.

ReplaySSM is an exact reorganisation of the recurrence: its outputs agree with
conventional decoding up to floating-point rounding ([ru] §03; [ar] "how
ReplaySSM works"; [zh] method points).  The oracle for every fp32 path is
therefore the plain definition ([ru] §01):

    S_t = a_t * S_{t-1} + v_t k_t^T          (S is P x N: value dim x key dim)
    o_t = S_t q_t

for every (sequence b, value head h) independently, with key/query head
floor(h / group) shared by the ``group`` value heads of a key group ([zh] method
points: K^T Q is shared by the value heads of a group).

Speculative verification ([ru] §05; [ar] rollback section; [zh] method points):
the T draft outputs are those of eq.R continued from the committed state
through drafts 1..t, and committing an accepted prefix of length a leaves the
state eq.R reaches after exactly those a drafts; the other drafts leave no trace.

Pins (tests/test_oracle_pins.py): alpha == 1 integer closed form (sum of outer
products, exact), constant-alpha geometric closed form, integrating-factor form
for time-varying alpha, rational brute force of eq.U, zero-state eq.O1,
verify/commit against plain decoding.
"""
from __future__ import annotations

import numpy as np


def _expand_keys(x: np.ndarray, group: int) -> np.ndarray:
    """Map key-head arrays [..., Hk, N] to value heads [..., Hv, N] (head h uses
    key head h // group)."""
    return np.repeat(x, group, axis=-2)


def eqR_step(S, alpha, k, v, q, group: int = 1):
    """One eq.R step for all (b, h) at once, in fp64.

    S      [B][Hv][P][N] float64 (not modified)
    alpha  [B][Hv];  k, q [B][Hk][N];  v [B][Hv][P]
    Returns (S_t, o_t) with o_t [B][Hv][P].
    """
    a = np.asarray(alpha, dtype=np.float64)
    kk = _expand_keys(np.asarray(k, dtype=np.float64), group)
    qq = _expand_keys(np.asarray(q, dtype=np.float64), group)
    vv = np.asarray(v, dtype=np.float64)
    S_new = a[..., None, None] * S + vv[..., :, None] * kk[..., None, :]
    o = np.matmul(S_new, qq[..., :, None])[..., 0]
    return S_new, o


def decode(S0, step_inputs, group: int = 1, keep_states=None):
    """Run eq.R over a sequence of steps.

    S0          [B][Hv][P][N] initial state (any float dtype; used in fp64)
    step_inputs iterable of (alpha, k, v, q) per step
    keep_states set of 1-based step numbers whose state S_t is returned
    Returns (outputs [steps][B][Hv][P] fp64, {t: S_t}, final S).
    """
    S = np.array(S0, dtype=np.float64, copy=True)
    outs, kept = [], {}
    keep_states = set(keep_states or ())
    for t, (a, k, v, q) in enumerate(step_inputs, start=1):
        S, o = eqR_step(S, a, k, v, q, group)
        outs.append(o)
        if t in keep_states:
            kept[t] = S.copy()
    return np.stack(outs) if outs else np.zeros((0,)), kept, S


def verify(S_committed, alpha, k, v, q, group: int = 1):
    """Outputs of T draft tokens evaluated from the committed state.

    S_committed [B][Hv][P][N];  alpha [B][T][Hv];  k, q [B][T][Hk][N];
    v [B][T][Hv][P].
    Returns (O [B][T][Hv][P], states [T+1][B][Hv][P][N]) where states[t] is the
    state after the first t drafts (states[0] = S_committed).
    """
    S = np.array(S_committed, dtype=np.float64, copy=True)
    T = alpha.shape[1]
    outs, states = [], [S.copy()]
    for t in range(T):
        S, o = eqR_step(S, alpha[:, t], k[:, t], v[:, t], q[:, t], group)
        outs.append(o)
        states.append(S.copy())
    return np.stack(outs, axis=1), np.stack(states)


def commit(states, accepted):
    """State after committing ``accepted[b]`` drafts of sequence b: the eq.R
    state after exactly that prefix ([ru] §05: the accepted prefix is kept by
    moving the buffer pointer; rejected drafts are simply ignored)."""
    acc = np.asarray(accepted)
    B = acc.shape[0]
    return np.stack([states[int(acc[b]), b] for b in range(B)])


def prefill(S_ckpt, buffered, prompt, window: int, group: int = 1):
    """Prefill of T prompt tokens into the checkpoint and buffer ([zh] method
    points: the unrolled form is the chunkwise form prefill kernels use; [ru]
    §03 for the window).  Reading: prefill leaves exactly the state that
    decoding the prompt token by token would leave -- the records buffered
    since the checkpoint, then the prompt, folded window by window.

    S_ckpt    [B][Hv][P][N] checkpoint;  buffered  the h0 records (alpha, k, v)
              already in the buffer (same h0 for every sequence), oldest first;
    prompt    (alpha [B][T][Hv], k [B][T][Hk][N], v [B][T][Hv][P], q [B][T][Hk][N]).
    Returns (O [B][T][Hv][P] -- eq.R outputs of the prompt tokens,
             S_new -- the state after the last complete window (S_ckpt if none),
             folds -- the number of windows completed).
    """
    a, k, v, q = (np.asarray(x) for x in prompt)
    T = a.shape[1]
    h0 = len(buffered)
    S = np.array(S_ckpt, dtype=np.float64, copy=True)
    zero_q = None
    for (aj, kj, vj) in buffered:
        zero_q = np.zeros_like(np.asarray(kj, dtype=np.float64)) if zero_q is None else zero_q
        S, _ = eqR_step(S, aj, kj, vj, zero_q, group)
    folds = (h0 + T) // window
    last = folds * window - h0            # prompt tokens up to the last window boundary
    S_new = np.array(S_ckpt, dtype=np.float64, copy=True) if folds == 0 else None
    outs = []
    for t in range(T):
        S, o = eqR_step(S, a[:, t], k[:, t], v[:, t], q[:, t], group)
        outs.append(o)
        if folds and t + 1 == last:
            S_new = S.copy()
    return np.stack(outs, axis=1), S_new, folds
