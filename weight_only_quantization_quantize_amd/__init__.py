"""Group-wise weight-only 3/4-bit quantization and fused dequantize-GEMV/GEMM for MI355X (gfx950).

The compute path is the HIP library ``libwoq.so`` (C ABI in ``include/woq.h``);
``ops`` wraps it for PyTorch tensors, ``synth`` draws the seeded synthetic
inputs.  Importing the package does not load the library; the first call does,
and fails loudly if it has not been built.
"""
from . import _lib  # noqa: F401

__all__ = ["ops", "synth", "build"]


def __getattr__(name):
    if name in ("ops", "synth", "build"):
        import importlib

        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
