"""MI355X (gfx950) Soft-DTW: C-ABI HIP library (libsdtw.so) + PyTorch layer.

The library is loaded on first use; a missing build raises instead of
falling back to anything else.
"""
from .softdtw import (EarlyStopping, SoftDTW, alignment, choose_fused, choose_mode,
                      soft_dtw, softdtw_barycenter, sqeuclidean)

__all__ = ["SoftDTW", "soft_dtw", "softdtw_barycenter", "sqeuclidean", "alignment",
           "choose_fused", "choose_mode", "EarlyStopping"]
