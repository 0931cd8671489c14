"""ReplaySSM decode hot path for MI355X (gfx950).

The compute lives in the HIP library ``libreplayssm.so`` (C ABI in
``include/replayssm.h``); ``replayssm`` is its Python binding.  ``workloads``
draws seeded synthetic inputs and ``bytes_model`` counts the algorithmic HBM
bytes of each call.
"""
from . import bytes_model, workloads  # noqa: F401

__all__ = ["bytes_model", "workloads", "replayssm"]
