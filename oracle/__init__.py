"""CPU oracle for Re-ttention's static block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  It shares no code with the HIP
library and never imports it; the product path does not fall back to it.

Every function here is plain and slow on purpose: float64 NumPy, one query
row block or one (batch, head) at a time, so a reader can check it against
the pages by eye.
"""
from .masks import diag_mask, band_mask, cogvideo3d_mask, full_mask, build_mask, csr_from_mask, mask_density
from .dynamic import block_means, block_scores, dynamic_mask
from .rettn import (tau, ramp, key_keep, slice_mask, calibrate, sparse_step, full_attention, window_attention,
                    ditfastattn_residual, ditfastattn_step, post_softmax_masked, textbook_attention)

__all__ = [
    "diag_mask", "band_mask", "cogvideo3d_mask", "full_mask", "build_mask", "csr_from_mask", "mask_density",
    "block_means", "block_scores", "dynamic_mask",
    "tau", "ramp", "key_keep", "slice_mask", "calibrate", "sparse_step", "full_attention", "window_attention",
    "ditfastattn_residual", "ditfastattn_step", "post_softmax_masked", "textbook_attention",
]
