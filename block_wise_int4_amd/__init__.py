"""block_wise_int4_amd -- block-wise int4 weight-only matmul (ONNX MatMulNBits
layout) for AMD MI355X (gfx950), behind the C-ABI library ``libmnb.so``.

The binding (``block_wise_int4_amd.mnb``) is imported on first use so that
``synth`` can be used without loading the HIP library.
"""
import importlib

__all__ = ["mnb", "synth"]


def __getattr__(name):
    if name in ("mnb", "synth"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
