"""Static block masks and their compacted (CSR) block index -- oracle side.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The mask is static: one fixed pattern used at every denoising step, which is
what lets the method cache statistics across steps (Re-ttention summary page,
"Limitations"; review thread, authors' answer to W2 of the first review: a
static mask adds no overhead during inference).  The pages fix no geometry;
the generators below are the readings used throughout:

  DIAG(nb)            query block qb keeps key block qb only.
  BAND(nb, w)         keeps w consecutive key blocks starting at
                      clamp(qb - floor((w-1)/2), 0, nb - w): always exactly w.
                      A window of 1/8 of the sequence is 87.5% sparsity and
                      1/32 is 96.875% (review thread, reply to W1 of the third
                      review).
  COGVIDEO3D(nb,t,s)  keeps the t text blocks 0..t-1 plus the blocks
                      {qb-1, qb, qb+1, qb-s, qb+s} that fall inside [0, nb):
                      a spatio-temporal neighbourhood plus the text column of
                      joint text+video self-attention (review thread, answer
                      to Q5 of the first review: text tokens share the
                      self-attention with video tokens).
  FULL(nb)            every key block (0% sparsity).

Mask entries are 0/1 bytes, shape [nqb, nkb]; a nonzero entry means "kept".
"""
import numpy as np

DIAG, BAND, COGVIDEO3D, FULL = 0, 1, 2, 3


def diag_mask(nb):
    m = np.zeros((nb, nb), dtype=np.uint8)
    for qb in range(nb):
        m[qb, qb] = 1
    return m


def band_mask(nb, w):
    if not (1 <= w <= nb):
        raise ValueError("band width must be in [1, nb]")
    m = np.zeros((nb, nb), dtype=np.uint8)
    for qb in range(nb):
        start = qb - (w - 1) // 2
        start = max(0, min(start, nb - w))
        for kb in range(start, start + w):
            m[qb, kb] = 1
    return m


def cogvideo3d_mask(nb, text_blocks, tshift):
    m = np.zeros((nb, nb), dtype=np.uint8)
    for qb in range(nb):
        for kb in range(min(text_blocks, nb)):
            m[qb, kb] = 1
        for kb in (qb - 1, qb, qb + 1, qb - tshift, qb + tshift):
            if 0 <= kb < nb:
                m[qb, kb] = 1
    return m


def full_mask(nb):
    return np.ones((nb, nb), dtype=np.uint8)


def build_mask(kind, nb, w=0, text_blocks=0, tshift=0):
    if kind == DIAG:
        return diag_mask(nb)
    if kind == BAND:
        return band_mask(nb, w)
    if kind == COGVIDEO3D:
        return cogvideo3d_mask(nb, text_blocks, tshift)
    if kind == FULL:
        return full_mask(nb)
    raise ValueError(f"unknown mask kind {kind}")


def csr_from_mask(mask):
    """Kept key blocks of each query block in ascending order: (row_ptr, col_idx), int32."""
    mask = np.asarray(mask)
    nqb, nkb = mask.shape
    row_ptr = [0]
    col_idx = []
    for qb in range(nqb):
        for kb in range(nkb):
            if mask[qb, kb] != 0:
                col_idx.append(kb)
        row_ptr.append(len(col_idx))
    return np.array(row_ptr, dtype=np.int32), np.array(col_idx, dtype=np.int32)


def mask_density(mask, L=None, block=None):
    """Fraction of kept (query, key) pairs; at token level when L and block are given."""
    mask = np.asarray(mask) != 0
    if L is None:
        return mask.sum() / mask.size
    nb = mask.shape[0]
    sizes = np.array([min(block, L - i * block) for i in range(nb)], dtype=np.int64)
    kept = 0
    for qb in range(nb):
        kept += sizes[qb] * sizes[mask[qb]].sum()
    return kept / (L * L)
