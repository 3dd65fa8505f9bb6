"""Re-ttention static block-sparse attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library librettn.so (C ABI in include/rettn.h);
this package is its thin Python binding.
"""
from .rettn import (BlockIndex, RettnError, calibrate, calibrate_workspace_bytes, dynamic_index,
                    dynamic_index_noalloc, dynamic_workspace_bytes, index_build, lib, mask_build, sparse,
                    sparse_workspace_bytes,
                    MASK_BAND, MASK_COGVIDEO3D, MASK_DIAG, MASK_FULL, RETTN_BF16, RETTN_F32, EXPORTED)

__all__ = ["BlockIndex", "RettnError", "calibrate", "calibrate_workspace_bytes", "dynamic_index",
           "dynamic_index_noalloc", "dynamic_workspace_bytes", "index_build", "lib", "mask_build", "sparse",
           "sparse_workspace_bytes",
           "MASK_BAND", "MASK_COGVIDEO3D", "MASK_DIAG", "MASK_FULL", "RETTN_BF16", "RETTN_F32", "EXPORTED"]
