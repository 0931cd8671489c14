"""Exact rational forms of eq.R, eq.U and eq.OT -- TEST INFRASTRUCTURE ONLY.

Pure-Python ``fractions.Fraction`` arithmetic on one (sequence, head) pair with
tiny shapes.  These serve as brute-force pins:

* ``eqR_steps``: eq.R ([ru] §01) stepped exactly.
* ``eqU_state`` / ``eqU_output``: the unrolled window ([ru] §03; [zh] method
  points).  The pages write gamma_h for the decay since the checkpoint and
  gamma_{j+1:h} for the decay a record receives after it was appended; the
  reading used here (the only one under which eq.U equals eq.R) is
      gamma_{a:b} = prod_{i=a..b} alpha_i   (empty product = 1),
      gamma_h     = gamma_{1:h}.
* ``eqOT_outputs``: the T-query output-only chunk ([zh] method points).  The
  card names D and W without defining them; the causal reading used is
      Q = [q_{h+1} .. q_{h+T}],  D = diag(gamma_{1:h+t}),
      W[j, t] = gamma_{j+1:h+t} if j <= h+t else 0,
  with K, V the h committed records followed by the T drafts.

Matrices are lists of rows (P rows of N entries), vectors are lists.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Sequence


def _F(x) -> Fraction:
    return x if isinstance(x, Fraction) else Fraction(x)


def zeros(P: int, N: int):
    return [[Fraction(0)] * N for _ in range(P)]


def matvec(S, q):
    return [sum((_F(s) * _F(x) for s, x in zip(row, q)), Fraction(0)) for row in S]


def dot(a, b) -> Fraction:
    return sum((_F(x) * _F(y) for x, y in zip(a, b)), Fraction(0))


def gamma(alphas: Sequence, a: int, b: int) -> Fraction:
    """prod_{i=a..b} alphas[i-1] for 1-based a..b; empty product is 1."""
    g = Fraction(1)
    for i in range(a, b + 1):
        g *= _F(alphas[i - 1])
    return g


def eqR_steps(S0, records):
    """eq.R over records [(alpha, k, v, q), ...]; returns (outputs, states)."""
    S = [[_F(x) for x in row] for row in S0]
    outs, states = [], []
    for a, k, v, q in records:
        a = _F(a)
        S = [[a * S[p][n] + _F(v[p]) * _F(k[n]) for n in range(len(k))] for p in range(len(v))]
        outs.append(matvec(S, q))
        states.append([row[:] for row in S])
    return outs, states


def eqU_state(S_ckpt, alphas, ks, vs):
    """State after h records appended since the checkpoint, by eq.U."""
    h = len(alphas)
    P, N = len(S_ckpt), len(S_ckpt[0])
    gh = gamma(alphas, 1, h)
    S = [[gh * _F(S_ckpt[p][n]) for n in range(N)] for p in range(P)]
    for j in range(1, h + 1):
        c = gamma(alphas, j + 1, h)
        for p in range(P):
            for n in range(N):
                S[p][n] += c * _F(vs[j - 1][p]) * _F(ks[j - 1][n])
    return S


def eqU_output(S_ckpt, alphas, ks, vs, q):
    """Output at window position h without forming the state: the checkpoint
    term scaled by gamma_h plus every record contributing v_j (k_j . q) scaled
    by gamma_{j+1:h} (eq.U applied to q, with eq.O1 for each record)."""
    h = len(alphas)
    y = matvec(S_ckpt, q)
    gh = gamma(alphas, 1, h)
    o = [gh * yp for yp in y]
    for j in range(1, h + 1):
        s = dot(ks[j - 1], q)
        c = gamma(alphas, j + 1, h)
        for p in range(len(o)):
            o[p] += c * s * _F(vs[j - 1][p])
    return o


def eqOT_outputs(S_ckpt, alphas, ks, vs, qs, h: int):
    """Outputs of the T drafts by eq.OT.  ``alphas/ks/vs`` hold the h committed
    records followed by the T drafts (h + T entries); ``qs`` holds the T draft
    queries.  Returns a list of T output vectors (column t of O)."""
    T = len(qs)
    P = len(S_ckpt)
    outs = []
    for t in range(1, T + 1):
        q = qs[t - 1]
        D = gamma(alphas, 1, h + t)
        y = matvec(S_ckpt, q)
        col = [D * yp for yp in y]
        for j in range(1, h + T + 1):
            if j > h + t:
                continue          # W[j, t] = 0: drafts after t are invisible
            W = gamma(alphas, j + 1, h + t)
            s = dot(ks[j - 1], q)
            for p in range(P):
                col[p] += W * s * _F(vs[j - 1][p])
        outs.append(col)
    return outs
