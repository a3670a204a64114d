"""Lossless byte-split BF16 weights with fused decode-GEMV/GEMM on MI355X (gfx950).

The compute path lives in ``liblbf.so`` (HIP kernels behind a C ABI declared in
``include/lbf.h``); :mod:`decode_byte_split_amd.lbf` is its thin ctypes binding.
:mod:`decode_byte_split_amd.synth` holds the seeded synthetic input generators.
Submodules are imported on demand so that input generation never loads the GPU
library.
"""

__all__ = ["lbf", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib

        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
