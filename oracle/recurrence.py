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
