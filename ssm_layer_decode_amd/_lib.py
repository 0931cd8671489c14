"""ctypes declarations of the C ABI in include/replayssm.h (libreplayssm.so)
and of the measurement probes in include/rssm_probes.h (librssm_probes.so).

Loading fails loudly if a library has not been built: there is no fallback
path of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libreplayssm.so")
PROBE_LIB_PATH = os.path.join(HERE, "librssm_probes.so")

RSSM_OK, RSSM_EINVAL, RSSM_EUNSUPPORTED, RSSM_ESTATE, RSSM_EHIP = range(5)
STATUS_NAMES = {0: "RSSM_OK", 1: "RSSM_EINVAL", 2: "RSSM_EUNSUPPORTED", 3: "RSSM_ESTATE", 4: "RSSM_EHIP"}
RSSM_F32, RSSM_BF16 = 0, 1
RSSM_READ_NONE, RSSM_READ_BF16, RSSM_READ_FP8_ROW, RSSM_READ_MXFP4 = 0, 1, 2, 3
RSSM_STATE_F32, RSSM_STATE_BF16, RSSM_STATE_FP8_ROW = 0, 1, 2
RSSM_CKPT_F32, RSSM_CKPT_F16_SR, RSSM_CKPT_FP8_SR = 0, 1, 2
RSSM_DEVERR_POINTER, RSSM_DEVERR_ACCEPT, RSSM_DEVERR_OVERFLOW = 1, 2, 4
RSSM_STATIC_COMMIT_MAX_TILES = 262144
(RSSM_BUF_CKPT, RSSM_BUF_READ_COPY, RSSM_BUF_ROW_SCALE, RSSM_BUF_KBUF, RSSM_BUF_VBUF,
 RSSM_BUF_ABUF, RSSM_BUF_COUNT, RSSM_BUF_ERR, RSSM_BUF_WORK, RSSM_BUF_FOLDS, RSSM_NUM_BUFS) = range(11)
BUFFER_NAMES = ("ckpt", "read_copy", "row_scale", "kbuf", "vbuf", "abuf", "count", "err", "work", "folds")

EXPORTED = [
    "replayssm_version", "replayssm_query_sizes", "replayssm_create", "replayssm_destroy",
    "replayssm_reset", "replayssm_refresh_read_copy", "replayssm_decode_step", "replayssm_flush",
    "replayssm_spec_verify", "replayssm_commit", "replayssm_commit_static", "replayssm_read_error",
    "replayssm_prefill",
    "convssm_decode_step", "convssm_spec_verify", "convssm_commit",
]
PROBE_EXPORTED = ["rssm_probe_copy", "rssm_probe_read", "rssm_probe_read_chunked"]


class RssmConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_vheads", "n_kheads", "dim_v", "dim_k", "window", "max_draft",
        "in_dtype", "read_copy", "heads_per_tile", "ckpt_fmt")] + [("sr_seed", ctypes.c_uint64)]


# the rssm_buffers / rssm_config layout this binding marshals (RSSM_ABI_VERSION)
ABI_VERSION = "0.4"


class RssmBuffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BUFFER_NAMES]


class RssmError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(RssmConfig)
    st = ctypes.c_int
    sig = {
        "replayssm_version": ([], ctypes.c_char_p),
        "replayssm_query_sizes": ([cfgp, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_int32)], st),
        "replayssm_create": ([cfgp, ctypes.POINTER(RssmBuffers), ctypes.POINTER(ctypes.c_void_p)], st),
        "replayssm_destroy": ([P], st),
        "replayssm_reset": ([P, P, I, P], st),
        "replayssm_refresh_read_copy": ([P, P], st),
        "replayssm_decode_step": ([P, P, P, P, P, P, P], st),
        "replayssm_flush": ([P, P], st),
        "replayssm_spec_verify": ([P, I, P, P, P, P, P, P], st),
        "replayssm_commit": ([P, P, P], st),
        "replayssm_commit_static": ([P, P, P], st),
        "replayssm_read_error": ([P, ctypes.POINTER(ctypes.c_int32), I, P], st),
        "replayssm_prefill": ([P, I, P, P, P, P, P, P], st),
        "convssm_decode_step": ([cfgp, P, P, I, P, P, P, P, P, P], st),
        "convssm_spec_verify": ([cfgp, P, P, I, P, P, P, P, P, P], st),
        "convssm_commit": ([cfgp, P, P, I, P, P], st),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    got = lib.replayssm_version().decode()
    if got != "replayssm-gfx950 " + ABI_VERSION:
        raise ImportError(f"{LIB_PATH} is {got!r}; this binding expects ABI {ABI_VERSION} (rebuild the library)")
    _lib = lib
    return lib


_probes = None


def load_probes() -> ctypes.CDLL:
    """Load the measurement library (raises if it is missing)."""
    global _probes
    if _probes is not None:
        return _probes
    if not os.path.exists(PROBE_LIB_PATH):
        raise ImportError(f"{PROBE_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    P, S, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sig = {
        "rssm_probe_copy": ([P, P, S, P], st),
        "rssm_probe_read": ([P, S, P, P], st),
        "rssm_probe_read_chunked": ([P, S, P, S, P, P], st),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _probes = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != RSSM_OK:
        raise RssmError(fn, status)
