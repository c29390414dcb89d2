"""LoLA chunkwise hybrid attention layer on AMD MI355X (gfx950).

The compute lives in liblola.so (hand-written HIP kernels behind the C ABI of
include/lola.h).  `sparse_attention_chunkwise_amd.lola` is a thin ctypes
binding with the same call names; torch supplies device memory and streams
only.  Submodules are imported on first use, so the input generator can be
used without the library.
"""
import importlib

__all__ = ["lola", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
