"""Deterministic, batch- and split-invariant grouped-query attention for MI355X (gfx950).

The compute path is the HIP C-ABI library ``librla_attn.so`` (sources in
``csrc/``, declarations in ``include/rla_attn.h``).  The Python layer here only
marshals torch tensors into that ABI: every step of the attention runs in the
library's kernels, and the calls raise if the library is missing.

The library is loaded lazily, so ``inputs`` (the seeded generator) can be used
on hosts without a GPU.
"""

__all__ = ["api", "inputs"]
