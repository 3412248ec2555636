"""MI355X-native (gfx950) MX block-scaled linear layer.

``mx_block_scaled_amd.mxfp8`` is the binding of the HIP library ``libmxfp8.so`` (C ABI in
``include/mxfp8.h``); ``mx_block_scaled_amd.synth`` draws the seeded synthetic inputs.  The
binding is imported lazily so that ``synth`` stays importable without torch.
"""
import importlib

__all__ = ["mxfp8", "synth"]


def __getattr__(name):
    if name in ("mxfp8", "synth"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
