"""Pins of the oracle's dynamic block mask (no GPU).

The rule (mean-pooled block scores; the query block's own key block, then the
best keep - 1 others, ties to the lower index) is checked against constructed
inputs whose answer is known by hand, against a brute-force search over every
subset of blocks, and against its structural invariants.  Each check computes
its expectation without the oracle's helpers.
"""
import itertools

import numpy as np
import pytest

from oracle import dynamic as od
from oracle import masks as om


def _const_blocks(vals, u, block, L):
    """[L, d] tokens: every token of block i equals vals[i] * u."""
    x = np.zeros((L, len(u)))
    for i in range(L):
        x[i] = vals[i // block] * np.asarray(u)
    return x


def _rows(mask):
    return [sorted(np.nonzero(r)[0].tolist()) for r in mask]


def test_constructed_ranking():
    # key block j is c_j * u, every query block is u: block j scores c_j |u|^2
    block, c = 4, [0.3, 2.0, -1.0, 5.0, 1.1, 0.2]
    L = block * len(c)
    u = [1.0, -2.0, 0.5]
    q = _const_blocks([1.0] * len(c), u, block, L)[None, None]
    k = _const_blocks(c, u, block, L)[None, None]
    got = _rows(od.dynamic_mask(q, k, block, keep=3)[0])
    # by hand: order of the others by c is 3 (5.0), 1 (2.0), 4 (1.1), 0 (0.3), 5 (0.2), 2 (-1.0)
    assert got == [[0, 1, 3], [1, 3, 4], [1, 2, 3], [1, 3, 4], [1, 3, 4], [1, 3, 5]]


def test_tail_block_is_averaged_over_its_own_tokens():
    # block 8, L = 17: blocks 0 and 1 are full, block 2 holds one token
    block, L, u = 8, 17, [1.0, 0.0]
    q = np.tile(np.array(u), (L, 1))[None, None]
    k = _const_blocks([0.5, 0.2, 0.9], u, block, L)[None, None]
    # means 0.5, 0.2, 0.9: query block 0 keeps itself and block 2.  (A sum would rank block 1
    # first (1.6 > 0.9), and dividing block 2 by the full block size would give 0.11 < 0.2.)
    m = od.dynamic_mask(q, k, block, keep=2)[0]
    assert _rows(m)[0] == [0, 2]
    np.testing.assert_allclose(od.block_means(k[0, 0], block)[:, 0], [0.5, 0.2, 0.9])


def test_ties_go_to_the_lower_block():
    q = np.zeros((1, 1, 10, 2))            # every score is 0
    k = np.random.Generator(np.random.PCG64(3)).standard_normal((1, 1, 10, 2))
    got = _rows(od.dynamic_mask(q, k, 2, keep=3)[0])
    assert got == [[0, 1, 2], [0, 1, 2], [0, 1, 2], [0, 1, 3], [0, 1, 4]]


def test_not_a_number_ranks_last():
    block, L, u = 2, 8, [1.0, 1.0]
    q = np.tile(np.array(u), (L, 1))[None, None]
    k = _const_blocks([1.0, 4.0, 3.0, 2.0], u, block, L)[None, None]
    k[0, 0, 2, 0] = np.nan                 # block 1 (the best) now scores NaN
    got = _rows(od.dynamic_mask(q, k, block, keep=2)[0])
    assert got == [[0, 2], [1, 2], [2, 3], [2, 3]]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_best_subset_brute_force(seed):
    """Without ties, the kept set is the subset of keep - 1 other blocks with the largest total score."""
    g = np.random.Generator(np.random.PCG64(seed))
    B, H, L, d, block, keep = 1, 2, 23, 5, 4, 3
    q, k = g.standard_normal((B, H, L, d)), g.standard_normal((B, H, L, d))
    nb = -(-L // block)
    m = od.dynamic_mask(q, k, block, keep)
    for h in range(H):
        # means and scores with explicit loops
        qm, km = np.zeros((nb, d)), np.zeros((nb, d))
        for i in range(nb):
            n = 0
            for t in range(i * block, min(L, (i + 1) * block)):
                qm[i] += q[0, h, t]
                km[i] += k[0, h, t]
                n += 1
            qm[i] /= n
            km[i] /= n
        for a in range(nb):
            sc = [sum(qm[a, c] * km[b, c] for c in range(d)) for b in range(nb)]
            others = [b for b in range(nb) if b != a]
            best = max(itertools.combinations(others, keep - 1), key=lambda sub: sum(sc[b] for b in sub))
            assert _rows(m[h])[a] == sorted([a, *best])


def test_structure_and_degenerate_keeps():
    g = np.random.Generator(np.random.PCG64(7))
    B, H, L, d, block = 2, 3, 37, 4, 8
    q, k = g.standard_normal((B, H, L, d)), g.standard_normal((B, H, L, d))
    nb = 5
    for keep in (1, 2, 4, 5, 9):
        m = od.dynamic_mask(q, k, block, keep)
        assert m.shape == (B * H, nb, nb) and m.dtype == np.uint8
        assert np.all(m.sum(-1) == min(keep, nb))
        assert np.all(m[:, np.arange(nb), np.arange(nb)] == 1)
    np.testing.assert_array_equal(od.dynamic_mask(q, k, block, 1), np.broadcast_to(om.diag_mask(nb), (B * H, nb, nb)))
    np.testing.assert_array_equal(od.dynamic_mask(q, k, block, nb), np.ones((B * H, nb, nb), np.uint8))
    with pytest.raises(ValueError):
        od.dynamic_mask(q, k, block, 0)


def test_slices_in_batch_head_order():
    """Slice b*H + h is the mask of (b, h) computed alone."""
    g = np.random.Generator(np.random.PCG64(9))
    B, H, L, d, block = 2, 3, 30, 4, 6
    q, k = g.standard_normal((B, H, L, d)), g.standard_normal((B, H, L, d))
    m = od.dynamic_mask(q, k, block, 3)
    for b in range(B):
        for h in range(H):
            alone = od.dynamic_mask(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], block, 3)[0]
            np.testing.assert_array_equal(m[b * H + h], alone)
    assert len({m[i].tobytes() for i in range(B * H)}) == B * H   # the slices do differ


def test_permuting_key_blocks_permutes_columns():
    """Relabelling key blocks (queries fixed) relabels the chosen blocks, diagonal aside:
    compare the off-diagonal choice on rows whose diagonal block is a fixed point."""
    g = np.random.Generator(np.random.PCG64(11))
    L, d, block, keep = 24, 3, 4, 3
    q, k = g.standard_normal((1, 1, L, d)), g.standard_normal((1, 1, L, d))
    perm = [0, 1, 5, 3, 2, 4]                # swaps blocks 2 and 5 and moves 4; 0, 1, 3 fixed
    kp = np.concatenate([k[0, 0, p * block:(p + 1) * block] for p in perm])[None, None]
    m, mp = od.dynamic_mask(q, k, block, keep)[0], od.dynamic_mask(q, kp, block, keep)[0]
    for a in (0, 1, 3):
        assert sorted(perm[j] for j in np.nonzero(mp[a])[0]) == _rows(m)[a]


# ------------------------------------------------------------ planted mistakes
MUTATIONS = [
    ("own block not forced", "chosen = [a]", "chosen = []"),
    ("lowest scores kept", 'np.argsort(-s, kind="stable")', 'np.argsort(s, kind="stable")'),
    ("ties to the higher index", 'np.argsort(-s, kind="stable")', 'len(s) - 1 - np.argsort(-s[::-1], kind="stable")'),
    ("sum instead of mean", "out[i] = toks.sum(axis=0) / len(toks)", "out[i] = toks.sum(axis=0)"),
    ("tail divided by the block size", "out[i] = toks.sum(axis=0) / len(toks)", "out[i] = toks.sum(axis=0) / block"),
    ("not-a-number ranks first", "s[np.isnan(s)] = -np.inf", "s[np.isnan(s)] = np.inf"),
    ("scores transposed", "block_means(q, block) @ block_means(k, block).T",
     "block_means(k, block) @ block_means(q, block).T"),
    ("slices head-major", "out[b * H + h, a, ", "out[h * B + b, a, "),
    ("one block too many", "if len(chosen) >= min(keep, nkb):", "if len(chosen) > min(keep, nkb):"),
]


def _pins():
    return [test_constructed_ranking, test_tail_block_is_averaged_over_its_own_tokens, test_ties_go_to_the_lower_block,
            test_not_a_number_ranks_last, lambda: test_best_subset_brute_force(0), test_structure_and_degenerate_keeps,
            test_slices_in_batch_head_order, test_permuting_key_blocks_permutes_columns]


def _failures_with(module):
    global od
    saved, od = od, module
    failures = 0
    try:
        for pin in _pins():
            try:
                with np.errstate(all="ignore"):
                    pin()
            except Exception:
                failures += 1
    finally:
        od = saved
    return failures


def _mutant(old, new):
    import os
    import types
    src = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "dynamic.py")).read()
    assert old in src, f"mutation anchor not found: {old}"
    mod = types.ModuleType("dynamic_mutant")
    exec(compile(src.replace(old, new, 1), "dynamic_mutant", "exec"), mod.__dict__)
    return mod


def test_unmutated_copy_passes_every_pin():
    assert _failures_with(_mutant("import numpy as np", "import numpy as np")) == 0


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, old, new):
    assert _failures_with(_mutant(old, new)) >= 1, f"no pin caught: {name}"
