"""paged_attention_slot_amd -- PagedAttention decode hot path on MI355X.

Python face of ``libpkv.so`` (C ABI in ``include/pkv.h``): slot-scatter KV
append, copy-on-write block copy, block-table-driven GQA decode attention with
split-KV, and the host block manager that produces tables and slots.  All
compute runs in the library's HIP kernels; torch only supplies device memory
and streams.
"""
from ._lib import LIB_PATH, PkvError, lib  # noqa: F401
from .block_manager import BlockManager, NoFreeBlocks  # noqa: F401

__all__ = ["BlockManager", "NoFreeBlocks", "PkvError", "lib", "LIB_PATH", "ops", "runtime"]


def __getattr__(name):
    # ``ops`` and ``runtime`` import torch; load them on first use.
    if name in ("ops", "runtime"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
