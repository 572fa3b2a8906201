"""Hybrid HiSparse sparse-MLA decode step for MI355X (gfx950).

The compute path is the HIP library ``libhisparse.so`` (C ABI in
``include/hisparse.h``); ``hisparse`` is its ctypes binding and ``accounting``
holds the byte/FLOP figures the benchmark prices rooflines with.
"""
from . import accounting  # noqa: F401

__all__ = ["accounting", "hisparse", "build"]


def build() -> str:
    from .build import build as _build
    return _build()
