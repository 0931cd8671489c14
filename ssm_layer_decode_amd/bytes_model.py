"""Algorithmic HBM bytes of the ReplaySSM decode path and of its baselines.

These are the bytes the method itself must move (no re-reads an implementation
adds).  Traffic model of the pages ([ru] §04; [ar] "reducing state traffic";
[zh] method points): over a window of L tokens conventional decoding reads and
writes the state L times each; ReplaySSM reads its checkpoint every step, writes
it once per window, and otherwise writes only the new input record.

Per decode step and sequence (one layer), ReplaySSM moves:
  * the checkpoint read (fp32 or fp16, or the low-precision read copy on
    non-flush steps),
  * 1/L of a checkpoint write (plus the read copy's refresh when present),
  * the h earlier records of the window (h = 0..L-1, mean (L-1)/2),
  * the new record read from the step inputs, and its write into the buffer on
    the L-1 non-flush steps of a window (a flush clears the buffer, so its
    record is never stored),
  * q read and o write.
Conventional decoding moves the state read + write, k, v, alpha, q reads and the
o write.  The per-tile pointer words (8 bytes per workgroup) are left out.
"""
from __future__ import annotations

from dataclasses import dataclass


def _esize(dtype: str) -> int:
    return {"f32": 4, "bf16": 2}[dtype]


@dataclass(frozen=True)
class Dims:
    n_vheads: int
    n_kheads: int
    dim_v: int
    dim_k: int
    window: int
    in_dtype: str = "f32"
    read_copy: str = "none"     # "none" | "bf16" | "fp8" | "mxfp4"
    ckpt: str = "f32"           # "f32" | "f16sr" | "fp8sr"

    @staticmethod
    def of(shape) -> "Dims":
        return Dims(shape.n_vheads, shape.n_kheads, shape.dim_v, shape.dim_k, shape.window,
                    shape.in_dtype, getattr(shape, "read_copy", "none"), getattr(shape, "ckpt", "f32"))


def fp32_state_bytes(d: Dims) -> int:
    """fp32 state of one sequence (the conventional baseline's state)."""
    return d.n_vheads * d.dim_v * d.dim_k * 4


def state_bytes(d: Dims) -> int:
    """Checkpoint of one sequence: fp32, fp16, or e4m3 codes plus one fp32
    scale per row for the fp8 checkpoint (its rows' other 12 trailer bytes are
    never read or written)."""
    if d.ckpt == "fp8sr":
        return d.n_vheads * d.dim_v * (d.dim_k + 4)
    return d.n_vheads * d.dim_v * d.dim_k * (2 if d.ckpt == "f16sr" else 4)


def copy_bytes(d: Dims) -> int:
    """Low-precision read copy of one sequence (codes + per-row scales)."""
    if d.read_copy == "none":
        return 0
    if d.read_copy == "bf16":
        return d.n_vheads * d.dim_v * d.dim_k * 2
    if d.read_copy == "fp8":
        return d.n_vheads * d.dim_v * d.dim_k + d.n_vheads * d.dim_v * 4
    if d.read_copy == "mxfp4":          # E2M1 codes + one E8M0 byte per 32 entries
        return d.n_vheads * d.dim_v * d.dim_k // 2 + d.n_vheads * d.dim_v * (d.dim_k // 32)
    raise ValueError(d.read_copy)


def record_bytes(d: Dims) -> int:
    """One buffered input record (alpha, k, v) of one sequence."""
    e = _esize(d.in_dtype)
    return d.n_kheads * d.dim_k * e + d.n_vheads * d.dim_v * e + d.n_vheads * 4


def q_bytes(d: Dims, T: int = 1) -> int:
    return T * d.n_kheads * d.dim_k * _esize(d.in_dtype)


def o_bytes(d: Dims, T: int = 1) -> int:
    return T * d.n_vheads * d.dim_v * 4


def replay_step_bytes(d: Dims, h: int) -> int:
    """Bytes of one decode step of one sequence that starts with h buffered
    records (h = L-1 is the flush step)."""
    L = d.window
    flush = (h + 1 == L)
    S, R = state_bytes(d), copy_bytes(d)
    b = 0
    if flush or R == 0:
        b += S                          # checkpoint read
    else:
        b += R                          # low-precision copy read
    if flush:
        b += S + R                      # checkpoint (and copy) written once
    b += h * record_bytes(d)            # earlier records
    b += record_bytes(d)                # new record read from the step inputs
    if not flush:
        b += record_bytes(d)            # ... and appended to the buffer
    b += q_bytes(d) + o_bytes(d)
    return b


def replay_bytes_per_token(d: Dims) -> float:
    """Window-averaged bytes per decode step per sequence."""
    L = d.window
    return sum(replay_step_bytes(d, h) for h in range(L)) / L


def replay_state_bytes_per_token(d: Dims) -> float:
    """Checkpoint/copy bytes only, window-averaged."""
    L = d.window
    S, R = state_bytes(d), copy_bytes(d)
    nonflush = S if R == 0 else R
    return ((L - 1) * nonflush + (S + S + R)) / L


def conv_bytes_per_token(d: Dims, state_fmt: str = "f32") -> int:
    """Conventional fused decode: state read + write plus the step's vectors."""
    st = fp32_state_bytes(d) if state_fmt == "f32" else copy_bytes(Dims(**{**d.__dict__, "read_copy": state_fmt}))
    return 2 * st + record_bytes(d) + q_bytes(d) + o_bytes(d)


def conv_state_bytes_per_token(d: Dims) -> int:
    return 2 * fp32_state_bytes(d)


def replay_verify_bytes(d: Dims, h: int, T: int) -> int:
    """One output-only verify of T drafts for one sequence with h committed
    records: checkpoint (or its read copy) read once for all T queries, h
    records read, T drafts read and appended, T queries read, T outputs
    written."""
    read = copy_bytes(d) or state_bytes(d)
    return read + h * record_bytes(d) + 2 * T * record_bytes(d) + q_bytes(d, T) + o_bytes(d, T)


def replay_fold_bytes(d: Dims, h: int) -> int:
    """A standalone fold of h records (commit/flush): checkpoint read + write,
    copy write, h records read."""
    return 2 * state_bytes(d) + copy_bytes(d) + h * record_bytes(d)


def snapshot_verify_bytes(d: Dims, T: int) -> int:
    """Snapshot verify: 1 state read, T snapshot writes, T drafts' vectors."""
    return (fp32_state_bytes(d) * (1 + T) + T * record_bytes(d) + q_bytes(d, T) + o_bytes(d, T))
