"""MI355X-native DoRA module hot path: factored row norm, fused compose,
forward and norm-detached backward, as hand-written HIP kernels for gfx950
behind a C-ABI library (libdora.so).

The binding in ``dora_adapter_amd.dora`` marshals torch device tensors into
that library; submodules are imported on first use so that
``dora_adapter_amd.synth`` (seeded inputs) loads on hosts without the library.
"""
import importlib

__all__ = ["dora", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
