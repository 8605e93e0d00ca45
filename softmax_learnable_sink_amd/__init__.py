"""Sink attention for AMD MI355X (gfx950): hand-written HIP kernels behind a C ABI.

The compute entry points live in ``softmax_learnable_sink_amd.binding`` and load
the in-tree ``libattn_sink.so`` when first used; the input generators in
``softmax_learnable_sink_amd.synth`` need no GPU.
"""

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name in ("binding", "synth"):
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
