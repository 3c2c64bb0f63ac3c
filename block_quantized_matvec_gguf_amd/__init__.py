"""Block-quantized (GGUF Q4_0 / Q4_K / Q6_K, BF16, F16) matrix-vector product
y = x @ W on AMD Instinct MI355X (gfx950), through a C-ABI library.

The HIP library ``libqmv.so`` is loaded lazily on first use; there is no CPU
fallback: if the library is missing, every compute call raises.
"""
import importlib

from .synth import FORMAT_IDS, FORMAT_NAMES, F16, BF16, Q4_0, Q4_K, Q6_K  # noqa: F401

_SUBMODULES = ("binding", "build", "synth")


def __getattr__(name):
    # Submodules import on demand, and the binding's names are re-exported
    # lazily so that input generation works without the HIP library.
    if name in _SUBMODULES:
        return importlib.import_module("." + name, __name__)
    binding = importlib.import_module(".binding", __name__)
    if hasattr(binding, name):
        return getattr(binding, name)
    raise AttributeError(name)
