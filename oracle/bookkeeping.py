"""Integer model of the record buffer and its pointer -- TEST INFRASTRUCTURE ONLY.

Compared bit-exactly with the device.  The rules follow the pages:

* State = checkpoint + buffer of recent input records (alpha_j, v_j, k_j); q is
  not a record ([ru] §03; [zh] method points).
* Non-flush step: append the current record ([ru] §03; [ar] "how ReplaySSM
  works").  The buffer holds L = 16 records ([ar] same section); the flush
  happens on the step whose append fills it, folds the records into the
  checkpoint and clears the buffer ([ru] §03; [zh] method points).  Reading
  adopted: the fill and the fold happen in the same call, so 64 steps at L = 16
  give exactly 4 flushes (steps 16, 32, 48, 64).
* Speculative decoding: the T draft records are appended after the committed
  ones before verification; the accepted prefix is committed by advancing the
  buffer pointer; records past the pointer are ignored and overwritten later
  ([ru] §05; [ar] rollback section; [zh] method points).
  Readings adopted (the pages are silent): capacity C = L + T_max; commit folds
  every committed record as soon as the pointer reaches L or more.
* ``flush()`` folds whatever is buffered (pointer > 0) and clears the buffer.

Buffers are modelled at storage granularity: k per key head [B][Hk][C][N],
v per value head [B][Hv][C][P], alpha per value head [B][Hv][C].  Only slots
[0, h_b) carry meaning; the model stores exact copies of the input values
(their bit patterns, whatever the storage dtype).
"""
from __future__ import annotations

import numpy as np


class BufferModel:
    def __init__(self, batch, n_vheads, n_kheads, dim_v, dim_k, window, max_draft=0,
                 store_dtype=np.float32):
        self.B, self.Hv, self.Hk = batch, n_vheads, n_kheads
        self.P, self.N, self.L, self.Tmax = dim_v, dim_k, window, max_draft
        self.C = window + max_draft
        self.count = np.zeros(batch, dtype=np.int32)
        self.kbuf = np.zeros((batch, n_kheads, self.C, dim_k), dtype=store_dtype)
        self.vbuf = np.zeros((batch, n_vheads, self.C, dim_v), dtype=store_dtype)
        self.abuf = np.zeros((batch, n_vheads, self.C), dtype=np.float32)
        self.pending_T = None

    # -- calls -----------------------------------------------------------
    def prefill(self, alpha, k, v):
        """Append T prompt records per sequence (alpha [B][T][Hv], k [B][T][Hk][N],
        v [B][T][Hv][P]) exactly as T decode steps would: the buffer keeps the
        records after the last window boundary.  Returns int[B]: windows folded."""
        folds = np.zeros(self.B, dtype=np.int32)
        for t in range(np.asarray(alpha).shape[1]):
            folds += self.decode(np.asarray(alpha)[:, t], np.asarray(k)[:, t], np.asarray(v)[:, t])
        return folds

    def decode(self, alpha, k, v):
        """Append one record per sequence.  Returns bool[B]: which sequences
        folded (flushed) on this step."""
        assert self.pending_T is None
        folded = np.zeros(self.B, dtype=bool)
        for b in range(self.B):
            h = int(self.count[b])
            assert 0 <= h < self.L
            self.kbuf[b, :, h] = k[b]
            self.vbuf[b, :, h] = v[b]
            self.abuf[b, :, h] = alpha[b]
            h += 1
            if h == self.L:
                folded[b] = True
                h = 0
            self.count[b] = h
        return folded

    def verify(self, alpha, k, v):
        """Append T drafts after the committed records; pointer unchanged.
        alpha [B][T][Hv], k [B][T][Hk][N], v [B][T][Hv][P]."""
        assert self.pending_T is None
        T = alpha.shape[1]
        assert 1 <= T <= self.Tmax
        for b in range(self.B):
            h = int(self.count[b])
            assert h + T <= self.C
            for t in range(T):
                self.kbuf[b, :, h + t] = k[b, t]
                self.vbuf[b, :, h + t] = v[b, t]
                self.abuf[b, :, h + t] = alpha[b, t]
        self.pending_T = T
        return T

    def commit(self, accepted):
        """Advance the pointer by accepted[b] (0..T).  Returns bool[B]: which
        sequences folded."""
        T = self.pending_T
        assert T is not None
        folded = np.zeros(self.B, dtype=bool)
        for b in range(self.B):
            a = int(accepted[b])
            assert 0 <= a <= T
            h = int(self.count[b]) + a
            if h >= self.L:
                folded[b] = True
                h = 0
            self.count[b] = h
        self.pending_T = None
        return folded

    def flush(self):
        assert self.pending_T is None
        folded = self.count > 0
        self.count[:] = 0
        return folded

    # -- views for comparison ----------------------------------------------
    def live_slots(self, b):
        return int(self.count[b])
