"""SparseLoCo pseudo-gradient compressor and aggregator for MI355X (gfx950).

The compute path is the HIP library libsparseloco.so (C-ABI in
include/sparseloco.h); the functions re-exported here marshal torch tensors
into that library and do no arithmetic of their own.
"""
from . import datagen  # noqa: F401  (distributions only)

__all__ = ["datagen"]
