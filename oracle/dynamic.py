"""Dynamic block masks -- oracle side.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Re-ttention is built on a static mask.  The authors also tried it, briefly,
with masks computed afresh at every step (review thread, answers to W2 and Q1
of the first review): the denominator ratio rho stays predictable, but the
cached residual no longer matches the tokens that the current mask leaves out.
The pages do not say how those masks were computed.  The reading used here is
the plainest block-level rule that needs no training:

  * each block of queries and of keys is summarised by the mean of its tokens
    (the last block averages only the tokens < L);
  * block a scores block b by the dot product of the two means (the softmax
    scale is a positive constant and cannot change a ranking, so it is left out);
  * query block a keeps its own block a, then the keep - 1 other key blocks with
    the highest scores (keep >= nkb keeps every block).  Equal scores go to the
    lower block index, and a score that is not a number ranks below every other.

One mask per (batch, head) slice, in the order b*H + h.
"""
import numpy as np


def block_means(x, block):
    """Mean of each block's tokens, float64 [nb, d]; the last block averages the tokens < L only."""
    x = np.asarray(x, dtype=np.float64)
    L = x.shape[0]
    nb = -(-L // block)
    out = np.zeros((nb, x.shape[1]))
    for i in range(nb):
        toks = x[i * block:min(L, (i + 1) * block)]
        out[i] = toks.sum(axis=0) / len(toks)
    return out


def block_scores(q, k, block):
    """Scores of every (query block, key block) pair of one slice: <mean q_a, mean k_b>."""
    return block_means(q, block) @ block_means(k, block).T


def top_blocks(scores, a, keep):
    """Key blocks kept by query block a: a itself, then the best keep - 1 others (ties: lower index)."""
    s = np.array(scores, dtype=np.float64)
    nkb = s.shape[0]
    s[np.isnan(s)] = -np.inf
    chosen = [a]
    # stable sort on the negated score: highest first, equal scores in ascending block order
    for b in np.argsort(-s, kind="stable"):
        if len(chosen) >= min(keep, nkb):
            break
        if b != a:
            chosen.append(int(b))
    return sorted(chosen)


def dynamic_mask(q, k, block, keep):
    """uint8 [B*H, nb, nb]: per slice, every query block's kept key blocks under the rule above."""
    if keep < 1:
        raise ValueError("keep must be at least 1")
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, L, _ = q.shape
    nb = -(-L // block)
    out = np.zeros((B * H, nb, nb), dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            sc = block_scores(q[b, h], k[b, h], block)
            for a in range(nb):
                out[b * H + h, a, top_blocks(sc[a], a, keep)] = 1
    return out
