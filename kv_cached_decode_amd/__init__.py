"""kv_cached_decode_amd: KV-cached decoder step for AMD MI355X (gfx950).

The hot path lives in a C-ABI shared library built from ``csrc/`` (HIP
kernels for gfx950); ``binding`` is a thin ctypes layer over it that takes
torch tensors on the ROCm device. Importing the package loads nothing; the
library is opened on first use of ``binding``.
"""
__all__ = ["binding", "inputs"]
