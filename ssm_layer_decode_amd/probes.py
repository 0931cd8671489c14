"""Bindings of the HBM probes (include/rssm_probes.h, librssm_probes.so):
measurement tools for the device's practical ceilings and for calibrating the
memory counters, not part of the decode method.  Argument marshalling only."""
from __future__ import annotations

import torch

from . import _lib
from ._lib import check
from .replayssm import _ptr, _stream


def rssm_probe_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n or not (src.is_cuda and dst.is_cuda):
        raise ValueError("rssm_probe_copy: dst too small or not on the GPU")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("rssm_probe_copy: tensors must be contiguous")
    check("rssm_probe_copy", _lib.load_probes().rssm_probe_copy(_ptr(dst), _ptr(src), n - n % 16, _stream()))


def rssm_probe_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    n = src.numel() * src.element_size()
    if not (src.is_cuda and sink.is_cuda and src.is_contiguous()):
        raise ValueError("rssm_probe_read: tensors must be contiguous GPU tensors")
    check("rssm_probe_read", _lib.load_probes().rssm_probe_read(_ptr(src), n - n % 16, _ptr(sink), _stream()))


def rssm_probe_read_chunked(src: torch.Tensor, dst: torch.Tensor, write_bytes: int, sink: torch.Tensor) -> None:
    n = src.numel() * src.element_size()
    n -= n % 32768
    if not (src.is_cuda and dst.is_cuda and sink.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("rssm_probe_read_chunked: tensors must be contiguous GPU tensors")
    if dst.numel() * dst.element_size() < n // 32768 * write_bytes:
        raise ValueError("rssm_probe_read_chunked: dst too small")
    check("rssm_probe_read_chunked", _lib.load_probes().rssm_probe_read_chunked(
        _ptr(src), n, _ptr(dst), int(write_bytes), _ptr(sink), _stream()))
