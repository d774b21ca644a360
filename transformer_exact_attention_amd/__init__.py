"""Exact grouped-query attention for AMD MI355X (gfx950): libgqa_attn + Python binding.

``import transformer_exact_attention_amd`` does not load the HIP library; the
first call through :mod:`.gqa_attn` does (and raises if it is not built).
"""
from importlib import import_module as _imp

__all__ = ["gqa_attn", "workloads", "build"]


def __getattr__(name):
    if name in __all__:
        return _imp(f".{name}", __name__)
    raise AttributeError(name)
