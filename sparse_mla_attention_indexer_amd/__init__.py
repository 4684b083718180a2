"""Sparse MLA with a lightning indexer on MI355X (gfx950): indexer scoring -> exact per-query
top-k -> sparse MLA over a shared FP8 latent cache, behind the C ABI of ``include/smla.h``.

``ops`` holds the torch-facing wrappers (device memory and streams from torch; all compute in
the library's HIP kernels). ``workload`` draws seeded synthetic inputs.
"""
import importlib

from ._lib import KV_BF16, KV_FP8_656, SmlaError, lib  # noqa: F401

__all__ = ["KV_BF16", "KV_FP8_656", "SmlaError", "lib", "ops", "workload"]


def __getattr__(name):
    if name in ("ops", "workload"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
