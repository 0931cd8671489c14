"""ctypes front of the plain C fp64 stepper (oracle/cpu/oracle_cpu.c) --
TEST INFRASTRUCTURE ONLY.

Same definition as ``recurrence.decode`` (eq.R, [ru] §01), for sizes where the
numpy stepper is slow, and the CPU baseline the benchmark times.
parity: pinned against recurrence.decode (tests/test_oracle_pins.py), which is
itself pinned by closed forms.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cpu", "oracle_cpu.c")
_LIB = os.path.join(_HERE, "cpu", "liboracle_cpu.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_eqR_decode.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, I]
        lib.oracle_eqR_decode.restype = I
        lib.oracle_split_read_bound.argtypes = [I, I, I, I, I, I, I, P, P, P, P, P, P, P, I]
        lib.oracle_split_read_bound.restype = I
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = I
        _lib = lib
    return _lib


def threads() -> int:
    return _load().oracle_threads()


def decode(S0, alpha, k, v, q, want_outputs: bool = True, nthreads: int = 0):
    """alpha [steps][B][Hv], k/q [steps][B][Hk][N], v [steps][B][Hv][P] (float32);
    S0 [B][Hv][P][N].  Returns (outputs [steps][B][Hv][P] f64 or None, final S f64)."""
    lib = _load()
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    steps, B, Hv = alpha.shape
    Hk, N = k.shape[2], k.shape[3]
    P = v.shape[3]
    S = np.array(S0, dtype=np.float64, copy=True, order="C")
    assert S.shape == (B, Hv, P, N)
    o = np.zeros((steps, B, Hv, P), dtype=np.float64) if want_outputs else None
    rc = lib.oracle_eqR_decode(B, Hv, Hk, P, N, steps,
                               alpha.ctypes.data, k.ctypes.data, v.ctypes.data, q.ctypes.data,
                               S.ctypes.data, o.ctypes.data if o is not None else None,
                               int(nthreads))
    if rc != 0:
        raise ValueError("oracle_eqR_decode: bad sizes")
    return o, S


def split_read_bound(S0, alpha, k, v, q, window: int, nthreads: int = 0):
    """Per-step, per-output-element sums (A, Z) bounding the read error of the
    split-precision path (see oracle_split_read_bound in oracle_cpu.c):
    |o - o_exact| <= u_rel * A + u_abs * Z elementwise; zero on flush steps."""
    lib = _load()
    alpha = np.ascontiguousarray(alpha, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    steps, B, Hv = alpha.shape
    Hk, N = k.shape[2], k.shape[3]
    P = v.shape[3]
    S0 = None if S0 is None else np.ascontiguousarray(S0, dtype=np.float64)
    A = np.zeros((steps, B, Hv, P))
    Z = np.zeros((steps, B, Hv, P))
    rc = lib.oracle_split_read_bound(B, Hv, Hk, P, N, steps, int(window), alpha.ctypes.data, k.ctypes.data,
                                     v.ctypes.data, q.ctypes.data,
                                     S0.ctypes.data if S0 is not None else None,
                                     A.ctypes.data, Z.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("oracle_split_read_bound: bad sizes")
    return A, Z
