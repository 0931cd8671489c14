"""Python binding of the ReplaySSM C ABI (argument marshalling only).

Every function here has the name of the C entry point it calls.  Each checks
the shapes, dtypes, devices and contiguity of its tensors against the layer's
configuration (the kernels trust those sizes), passes raw device pointers and
torch's current HIP stream, and raises ``RssmError`` on a non-OK status.  All
arithmetic happens in the HIP kernels.  PyTorch provides device memory and
streams only.

``ReplaySSM`` owns the caller-side buffers of one layer (torch tensors) and
the library handle.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import RssmBuffers, RssmConfig, check

_DT = {"f32": _lib.RSSM_F32, "bf16": _lib.RSSM_BF16}
_RC = {"none": _lib.RSSM_READ_NONE, "bf16": _lib.RSSM_READ_BF16, "fp8": _lib.RSSM_READ_FP8_ROW,
       "mxfp4": _lib.RSSM_READ_MXFP4}
_SF = {"f32": _lib.RSSM_STATE_F32, "bf16": _lib.RSSM_STATE_BF16, "fp8": _lib.RSSM_STATE_FP8_ROW}
_CK = {"f32": _lib.RSSM_CKPT_F32, "f16sr": _lib.RSSM_CKPT_F16_SR, "fp8sr": _lib.RSSM_CKPT_FP8_SR}
_TORCH_CK = {"f32": torch.float32, "f16sr": torch.float16, "fp8sr": torch.uint8}
_TORCH_IN = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class LayerConfig:
    batch: int
    n_vheads: int
    n_kheads: int
    dim_v: int
    dim_k: int
    window: int
    max_draft: int = 0
    in_dtype: str = "f32"
    read_copy: str = "none"
    heads_per_tile: int = 0
    ckpt: str = "f32"            # "f32" | "f16sr" | "fp8sr" (fp16 / row-scaled e4m3 rows of
                                 # N + 16 bytes, stochastic rounding at folds; fp8 needs a copy)
    sr_seed: int = 0

    @staticmethod
    def of(shape, **kw) -> "LayerConfig":
        d = dict(batch=shape.batch, n_vheads=shape.n_vheads, n_kheads=shape.n_kheads,
                 dim_v=shape.dim_v, dim_k=shape.dim_k, window=shape.window,
                 max_draft=shape.max_draft, in_dtype=shape.in_dtype,
                 read_copy=getattr(shape, "read_copy", "none"), ckpt=getattr(shape, "ckpt", "f32"))
        d.update(kw)
        return LayerConfig(**d)

    def c(self) -> RssmConfig:
        return RssmConfig(self.batch, self.n_vheads, self.n_kheads, self.dim_v, self.dim_k,
                          self.window, self.max_draft, _DT[self.in_dtype], _RC[self.read_copy],
                          self.heads_per_tile, _CK[self.ckpt], self.sr_seed)


# The raw handle of the current device's current stream (the one the kernels
# are launched on).  torch's private accessors return it without building a
# Stream object, which matters where a call is a few microseconds; the public
# route is the fallback.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_cur_device = getattr(torch._C, "_cuda_getDevice", None)


def _stream() -> int:
    if _raw_stream is not None and _cur_device is not None:
        return _raw_stream(_cur_device())
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    """Device address as an int (the C signatures take void*; None is NULL)."""
    return t.data_ptr() if t is not None else None


def _want(name, t, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


# --------------------------------------------------------------------------
# Thin wrappers with the C names
# --------------------------------------------------------------------------
def replayssm_version() -> str:
    return _lib.load().replayssm_version().decode()


def replayssm_query_sizes(cfg: LayerConfig):
    """(sizes in bytes per RSSM_BUF_* index, tiles per sequence)."""
    lib = _lib.load()
    sizes = (ctypes.c_size_t * _lib.RSSM_NUM_BUFS)()
    tiles = ctypes.c_int32(0)
    c = cfg.c()
    check("replayssm_query_sizes", lib.replayssm_query_sizes(ctypes.byref(c), sizes, ctypes.byref(tiles)))
    return list(sizes), tiles.value


def replayssm_create(cfg: LayerConfig, bufs: dict):
    lib = _lib.load()
    c = cfg.c()
    b = RssmBuffers(*[bufs[n].data_ptr() if bufs.get(n) is not None else None for n in _lib.BUFFER_NAMES])
    h = ctypes.c_void_p()
    check("replayssm_create", lib.replayssm_create(ctypes.byref(c), ctypes.byref(b), ctypes.byref(h)))
    return h


def replayssm_destroy(layer: "ReplaySSM") -> None:
    if layer.handle:
        check("replayssm_destroy", _lib.load().replayssm_destroy(layer.handle))
        layer.handle = None


def replayssm_reset(layer: "ReplaySSM", seq_ids: Optional[torch.Tensor] = None) -> None:
    n = 0
    if seq_ids is not None:
        _want("seq_ids", seq_ids, (seq_ids.numel(),), torch.int32, layer.device)
        n = seq_ids.numel()
        if n == 0:
            return
    check("replayssm_reset", _lib.load().replayssm_reset(layer.handle, _ptr(seq_ids), n, _stream()))


def replayssm_refresh_read_copy(layer: "ReplaySSM") -> None:
    check("replayssm_refresh_read_copy", _lib.load().replayssm_refresh_read_copy(layer.handle, _stream()))


_STEP_NAMES = ("alpha", "k", "v", "q", "o")


def _step_specs(c: LayerConfig, T=None):
    """(shape, dtype) of alpha, k, v, q, o for a step (T is None) or T tokens."""
    B, Hv, Hk, P, N = c.batch, c.n_vheads, c.n_kheads, c.dim_v, c.dim_k
    lead = (B,) if T is None else (B, T)
    tin = _TORCH_IN[c.in_dtype]
    return ((lead + (Hv,), torch.float32), (lead + (Hk, N), tin), (lead + (Hv, P), tin),
            (lead + (Hk, N), tin), (lead + (Hv, P), torch.float32))


def _check_step(layer, alpha, k, v, q, o, T=None):
    dev = layer.device
    specs = layer._step_specs if T is None else _step_specs(layer.cfg, T)
    for name, t, (shape, dtype) in zip(_STEP_NAMES, (alpha, k, v, q, o), specs):
        # one combined test on the common path; _want names what is wrong
        if not (isinstance(t, torch.Tensor) and t.shape == shape and t.dtype == dtype and t.device == dev
                and t.is_contiguous()):
            _want(name, t, shape, dtype, dev)


def replayssm_decode_step(layer: "ReplaySSM", alpha, k, v, q, o) -> None:
    _check_step(layer, alpha, k, v, q, o)
    check("replayssm_decode_step", _lib.load().replayssm_decode_step(
        layer.handle, _ptr(alpha), _ptr(k), _ptr(v), _ptr(q), _ptr(o), _stream()))


def replayssm_flush(layer: "ReplaySSM") -> None:
    check("replayssm_flush", _lib.load().replayssm_flush(layer.handle, _stream()))


def replayssm_spec_verify(layer: "ReplaySSM", T: int, alpha, k, v, q, o) -> None:
    _check_step(layer, alpha, k, v, q, o, T=T)
    check("replayssm_spec_verify", _lib.load().replayssm_spec_verify(
        layer.handle, int(T), _ptr(alpha), _ptr(k), _ptr(v), _ptr(q), _ptr(o), _stream()))


def replayssm_prefill(layer: "ReplaySSM", T: int, alpha, k, v, q, o) -> None:
    _check_step(layer, alpha, k, v, q, o, T=T)
    check("replayssm_prefill", _lib.load().replayssm_prefill(
        layer.handle, int(T), _ptr(alpha), _ptr(k), _ptr(v), _ptr(q), _ptr(o), _stream()))


def replayssm_commit(layer: "ReplaySSM", accepted: torch.Tensor) -> None:
    _want("accepted", accepted, (layer.cfg.batch,), torch.int32, layer.device)
    check("replayssm_commit", _lib.load().replayssm_commit(layer.handle, _ptr(accepted), _stream()))


def replayssm_commit_static(layer: "ReplaySSM", accepted: torch.Tensor) -> None:
    _want("accepted", accepted, (layer.cfg.batch,), torch.int32, layer.device)
    check("replayssm_commit_static", _lib.load().replayssm_commit_static(layer.handle, _ptr(accepted), _stream()))


def replayssm_read_error(layer: "ReplaySSM", clear: bool = False) -> int:
    e = ctypes.c_int32(0)
    check("replayssm_read_error", _lib.load().replayssm_read_error(layer.handle, ctypes.byref(e),
                                                                   int(clear), _stream()))
    return e.value


def _conv_cfg(cfg: LayerConfig, max_draft=None) -> RssmConfig:
    c = cfg.c()
    if max_draft is not None:
        c.max_draft = max_draft
    return c


def convssm_decode_step(cfg: LayerConfig, state, row_scale, state_fmt: str, alpha, k, v, q, o) -> None:
    dev = state.device
    B, Hv, Hk, P, N = cfg.batch, cfg.n_vheads, cfg.n_kheads, cfg.dim_v, cfg.dim_k
    sd = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[state_fmt]
    _want("state", state, (B, Hv, P, N), sd, dev)
    if state_fmt == "fp8":
        _want("row_scale", row_scale, (B, Hv, P), torch.float32, dev)
    tin = _TORCH_IN[cfg.in_dtype]
    _want("alpha", alpha, (B, Hv), torch.float32, dev)
    _want("k", k, (B, Hk, N), tin, dev)
    _want("v", v, (B, Hv, P), tin, dev)
    _want("q", q, (B, Hk, N), tin, dev)
    _want("o", o, (B, Hv, P), torch.float32, dev)
    c = _conv_cfg(cfg)
    check("convssm_decode_step", _lib.load().convssm_decode_step(
        ctypes.byref(c), _ptr(state), _ptr(row_scale), _SF[state_fmt], _ptr(alpha), _ptr(k), _ptr(v),
        _ptr(q), _ptr(o), _stream()))


def convssm_spec_verify(cfg: LayerConfig, states, cur, T: int, alpha, k, v, q, o) -> None:
    dev = states.device
    B, Hv, Hk, P, N = cfg.batch, cfg.n_vheads, cfg.n_kheads, cfg.dim_v, cfg.dim_k
    _want("states", states, (B, cfg.max_draft + 1, Hv, P, N), torch.float32, dev)
    _want("cur", cur, (B,), torch.int32, dev)
    tin = _TORCH_IN[cfg.in_dtype]
    _want("alpha", alpha, (B, T, Hv), torch.float32, dev)
    _want("k", k, (B, T, Hk, N), tin, dev)
    _want("v", v, (B, T, Hv, P), tin, dev)
    _want("q", q, (B, T, Hk, N), tin, dev)
    _want("o", o, (B, T, Hv, P), torch.float32, dev)
    c = _conv_cfg(cfg)
    check("convssm_spec_verify", _lib.load().convssm_spec_verify(
        ctypes.byref(c), _ptr(states), _ptr(cur), int(T), _ptr(alpha), _ptr(k), _ptr(v), _ptr(q), _ptr(o),
        _stream()))


def convssm_commit(cfg: LayerConfig, cur, accepted, T: int, err) -> None:
    dev = cur.device
    _want("cur", cur, (cfg.batch,), torch.int32, dev)
    _want("accepted", accepted, (cfg.batch,), torch.int32, dev)
    _want("err", err, (err.numel(),), torch.int32, dev)
    c = _conv_cfg(cfg)
    check("convssm_commit", _lib.load().convssm_commit(ctypes.byref(c), _ptr(cur), _ptr(accepted), int(T),
                                                       _ptr(err), _stream()))


# --------------------------------------------------------------------------
# Owning wrapper
# --------------------------------------------------------------------------
class ReplaySSM:
    """One SSM layer's ReplaySSM decode state on a GPU: fp32 checkpoint, optional
    read copy, record buffers, per-tile pointer copies and the error word, all
    allocated zero-filled as torch tensors (empty buffers, zero checkpoint).
    commit_work=False allocates no commit work area: the layer then commits
    only with commit_static (the library's own device array)."""

    def __init__(self, cfg: LayerConfig, device="cuda", commit_work: bool = True):
        self.cfg = cfg
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self._step_specs = _step_specs(cfg)
        sizes, self.tiles = replayssm_query_sizes(cfg)
        B, Hv, Hk, P, N = cfg.batch, cfg.n_vheads, cfg.n_kheads, cfg.dim_v, cfg.dim_k
        C = cfg.window + cfg.max_draft
        self.capacity = C
        tin = _TORCH_IN[cfg.in_dtype]
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=self.device)
        # fp8: each row is N e4m3 codes and a 16-byte trailer holding its fp32 scale
        self.ckpt = z((B, Hv, P, N + 16 if cfg.ckpt == "fp8sr" else N), _TORCH_CK[cfg.ckpt])
        self.read_copy = None
        self.row_scale = None
        if cfg.read_copy == "bf16":
            self.read_copy = z((B, Hv, P, N), torch.bfloat16)
        elif cfg.read_copy == "fp8":
            self.read_copy = z((B, Hv, P, N), torch.uint8)
            self.row_scale = torch.ones((B, Hv, P), dtype=torch.float32, device=self.device)
        elif cfg.read_copy == "mxfp4":
            # E2M1 code pairs and E8M0 block exponents (zero bytes: an all-zero block)
            self.read_copy = z((B, Hv, P, N // 2), torch.uint8)
            self.row_scale = z((B, Hv, P, N // 32), torch.uint8)
        self.kbuf = z((B, Hk, C, N), tin)
        self.vbuf = z((B, Hv, C, P), tin)
        self.abuf = z((B, Hv, C), torch.float32)
        self.count = z((B, self.tiles), torch.int32)
        self.err = z((4,), torch.int32)
        self.work = z((sizes[_lib.RSSM_BUF_WORK] // 4,), torch.int32) if commit_work else None
        # fp16 / fp8 checkpoint: per-tile fold epochs of the stochastic rounding
        self.folds = z((B, self.tiles), torch.int32) if cfg.ckpt != "f32" else None
        got = {"ckpt": self.ckpt, "read_copy": self.read_copy, "row_scale": self.row_scale,
               "kbuf": self.kbuf, "vbuf": self.vbuf, "abuf": self.abuf, "count": self.count,
               "err": self.err, "work": self.work, "folds": self.folds}
        for i, n in enumerate(_lib.BUFFER_NAMES):
            t = got[n]
            have = 0 if t is None else t.numel() * t.element_size()
            need = sizes[i]
            if n == "work" and t is None:
                continue
            if (n == "err" and have < need) or (n != "err" and have != need):
                raise RuntimeError(f"buffer {n}: {have} bytes, library expects {need}")
        self.handle = replayssm_create(cfg, got)

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                replayssm_destroy(self)
        except Exception:
            pass

    # the C entry points, as methods
    def reset(self, seq_ids=None):
        replayssm_reset(self, seq_ids)

    def refresh_read_copy(self):
        replayssm_refresh_read_copy(self)

    def decode_step(self, alpha, k, v, q, o=None):
        if o is None:
            o = torch.empty((self.cfg.batch, self.cfg.n_vheads, self.cfg.dim_v), dtype=torch.float32,
                            device=self.device)
        replayssm_decode_step(self, alpha, k, v, q, o)
        return o

    def flush(self):
        replayssm_flush(self)

    def spec_verify(self, alpha, k, v, q, o=None):
        T = alpha.shape[1]
        if o is None:
            o = torch.empty((self.cfg.batch, T, self.cfg.n_vheads, self.cfg.dim_v), dtype=torch.float32,
                            device=self.device)
        replayssm_spec_verify(self, T, alpha, k, v, q, o)
        return o

    def prefill(self, alpha, k, v, q, o=None):
        T = alpha.shape[1]
        if o is None:
            o = torch.empty((self.cfg.batch, T, self.cfg.n_vheads, self.cfg.dim_v), dtype=torch.float32,
                            device=self.device)
        replayssm_prefill(self, T, alpha, k, v, q, o)
        return o

    def commit(self, accepted):
        replayssm_commit(self, accepted)

    def commit_static(self, accepted):
        replayssm_commit_static(self, accepted)

    def fold_epochs(self):
        """Folds stored so far per sequence (fp16 checkpoint: the epoch of
        each sequence's next stochastic rounding; all tiles of a sequence
        fold together), as a host numpy array [B]."""
        return self.folds[:, 0].cpu().numpy().astype("int64")

    def read_error(self, clear=False) -> int:
        return replayssm_read_error(self, clear)
