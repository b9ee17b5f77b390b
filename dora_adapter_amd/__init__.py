"""MI355X-native DoRA module hot path: factored row norm, fused compose,
forward and norm-detached backward, as hand-written HIP kernels for gfx950
behind a C-ABI library (libdora.so).

The binding in ``dora_adapter_amd.dora`` marshals torch device tensors into
that library; it is loaded lazily so that ``dora_adapter_amd.synth`` (seeded
inputs) can be imported on hosts without the library.
"""

__all__ = ["dora", "synth"]


def __getattr__(name):
    if name == "dora":
        from . import dora as _d
        return _d
    if name == "synth":
        from . import synth as _s
        return _s
    raise AttributeError(name)
