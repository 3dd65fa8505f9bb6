"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: the pages' worked
example (tests/golden/worked_example.txt), a textbook softmax attention
written with explicit loops, closed forms and invariants of the method, and
brute force over every mask of a 3x3 block grid.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import masks as om


# ---------------------------------------------------------------- worked example
def _example_inputs(probs, d=4):
    """One query row whose full attention over 4 one-hot keys is `probs`.

    K = V = I (block size 1), q = sqrt(d) ln p, so tau <q, k_j> = ln p_j and the
    attention output equals the probability row itself.  Four identical query
    rows are used so every query block has the same window.
    """
    L = len(probs)
    k = np.eye(L, d)[None, None]
    v = np.eye(L, d)[None, None]
    q = np.tile(math.sqrt(d) * np.log(np.asarray(probs, dtype=np.float64)), (L, 1))
    q = np.pad(q, ((0, 0), (0, d - L)))[None, None]
    return q, k, v


def _example_mask(window):
    w = np.asarray(window, dtype=np.uint8)
    return np.tile(w, (len(w), 1))


def test_worked_example_calibration(golden):
    g = golden("worked_example.txt")
    q, k, v = _example_inputs(g["full_probs"])
    mask = _example_mask(g["window"])
    o, rho, r = oracle.calibrate(q, k, v, mask, block=1)
    for i in range(4):
        np.testing.assert_allclose(o[0, 0, i], g["full_probs"], atol=1e-12)
        np.testing.assert_allclose(rho[0, 0, i], g["rho"][0], atol=1e-12)
        np.testing.assert_allclose(r[0, 0, i], g["residual"], atol=1e-12)
    # rescaled window probabilities: rho * softmax over the window
    win = oracle.window_attention(q, k, v, mask, 1)
    np.testing.assert_allclose(rho[0, 0, 0] * win[0, 0, 0], g["reshaped_window"], atol=1e-12)
    # DiTFastAttn comparator at the calibration step
    np.testing.assert_allclose(win[0, 0, 0], g["dfa_window"], atol=1e-12)
    np.testing.assert_allclose(oracle.ditfastattn_residual(o, win)[0, 0, 0], g["dfa_residual"], atol=1e-12)


def test_worked_example_drift(golden):
    g = golden("worked_example.txt")
    q, k, v = _example_inputs(g["full_probs"])
    mask = _example_mask(g["window"])
    o, rho, r = oracle.calibrate(q, k, v, mask, block=1)
    q2, _, _ = _example_inputs(g["drift_full_probs"])
    win2 = oracle.window_attention(q2, k, v, mask, 1)
    np.testing.assert_allclose(win2[0, 0, 0], g["drift_window"], atol=1e-12)
    np.testing.assert_allclose(rho[0, 0, 0] * win2[0, 0, 0], g["drift_reshaped"], atol=1e-12)
    # lambda = 0 pins the reshape and the residual add exactly
    out = oracle.sparse_step(q2, k, v, mask, 1, rho, r, lam=0.0, step=1)
    np.testing.assert_allclose(out[0, 0, 0], g["drift_rebuilt"], atol=1e-12)
    # and equals the drifted full attention (the reconstruction the authors claim)
    np.testing.assert_allclose(out[0, 0, 0], oracle.full_attention(q2, k, v)[0, 0, 0], atol=1e-12)
    r_dfa = oracle.ditfastattn_residual(o, oracle.window_attention(q, k, v, mask, 1))
    dfa = oracle.ditfastattn_step(q2, k, v, mask, 1, r_dfa)
    np.testing.assert_allclose(dfa[0, 0, 0], g["dfa_drift_rebuilt"], atol=1e-12)


# ---------------------------------------------------------------- textbook / brute force
def _rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


@pytest.mark.parametrize("B,H,L,d,block", [(1, 1, 5, 3, 2), (2, 2, 7, 4, 3), (1, 2, 8, 8, 4)])
def test_calibration_is_textbook_attention(B, H, L, d, block):
    q, k, v = (_rand((B, H, L, d), s) for s in (1, 2, 3))
    nb = -(-L // block)
    mask = (np.random.Generator(np.random.PCG64(9)).random((nb, nb)) < 0.5).astype(np.uint8)
    o, rho, r = oracle.calibrate(q, k, v, mask, block)
    ref = oracle.textbook_attention(q, k, v)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.full_attention(q, k, v), ref, rtol=1e-12, atol=1e-12)


def _scores(q, k):
    d = q.shape[-1]
    return np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(d)


def test_all_masks_3x3_brute_force():
    """Every one of the 512 masks of a 3x3 block grid, with a ragged tail block (L=5, block=2)."""
    B, H, L, d, block = 1, 2, 5, 3, 2
    q, k, v = (_rand((B, H, L, d), s) for s in (11, 12, 13))
    p = softmax(_scores(q, k), axis=-1)          # full attention probabilities (library softmax)
    full = p @ v
    blocks = np.arange(L) // block
    for bits in range(512):
        mask = np.array([(bits >> i) & 1 for i in range(9)], dtype=np.uint8).reshape(3, 3)
        keep = mask[blocks][:, blocks] != 0       # [L query, L key] token-level window
        o, rho, r = oracle.calibrate(q, k, v, mask, block)
        np.testing.assert_allclose(o, full, atol=1e-12)
        np.testing.assert_allclose(rho, (p * keep).sum(-1), atol=1e-12)
        np.testing.assert_allclose(r, (p * ~keep) @ v, atol=1e-12)
        # lambda = 0 sparse step on the calibration inputs rebuilds full attention
        out = oracle.sparse_step(q, k, v, mask, block, rho, r, lam=0.0, step=1)
        np.testing.assert_allclose(out, full, atol=1e-12)


def test_per_slice_masks_brute_force():
    """One mask per head ([H, nb, nb]) and one per (batch, head) ([B*H, nb, nb], order b*H + h):
    each slice's rho and R follow its own mask, by the token-level definitions; an empty row in
    one slice gives O' = R in that slice only."""
    B, H, L, d, block = 2, 3, 5, 3, 2
    q, k, v = (_rand((B, H, L, d), s) for s in (21, 22, 23))
    p = softmax(_scores(q, k), axis=-1)
    blocks = np.arange(L) // block
    g = np.random.Generator(np.random.PCG64(24))
    per_slice = (g.random((B * H, 3, 3)) < 0.5).astype(np.uint8)
    per_slice[4, 1] = 0                                  # slice (1, 1): query block 1 keeps nothing
    per_head = per_slice[:H].copy()
    for masks, pick in ((per_slice, lambda b, h: per_slice[b * H + h]), (per_head, lambda b, h: per_head[h])):
        o, rho, r = oracle.calibrate(q, k, v, masks, block)
        out = oracle.sparse_step(q, k, v, masks, block, rho, r, lam=0.0, step=1)
        for b in range(B):
            for h in range(H):
                keep = pick(b, h)[blocks][:, blocks] != 0
                np.testing.assert_allclose(rho[b, h], (p[b, h] * keep).sum(-1), atol=1e-12)
                np.testing.assert_allclose(r[b, h], (p[b, h] * ~keep) @ v[b, h], atol=1e-12)
                np.testing.assert_allclose(out[b, h], p[b, h] @ v[b, h], atol=1e-12)
    # the empty row of slice (1, 1) alone: the ramp cannot touch it, O' = R exactly
    o, rho, r = oracle.calibrate(q, k, v, per_slice, block)
    out = oracle.sparse_step(q, k, v, per_slice, block, rho, r, lam=0.5, step=3)
    np.testing.assert_array_equal(out[1, 1, 2:4], r[1, 1, 2:4])
    assert np.all(rho[1, 1, 2:4] == 0.0)
    with pytest.raises(ValueError):
        oracle.calibrate(q, k, v, per_slice[:4], block)


# ---------------------------------------------------------------- invariants
def _small_case(seed=0, B=2, H=2, L=40, d=8, block=8, density=0.4):
    q, k, v = (_rand((B, H, L, d), seed + s) for s in range(3))
    nb = -(-L // block)
    mask = (np.random.Generator(np.random.PCG64(seed + 5)).random((nb, nb)) < density).astype(np.uint8)
    mask[np.arange(nb), np.arange(nb)] = 1
    return q, k, v, mask, block


def test_sum_to_one():
    """Rescaled window probabilities plus residual weights sum to 1 at the calibration step:
    with V[..., 0] = 1, R[..., 0] = 1 - rho and rho * O_window[..., 0] + R[..., 0] = 1."""
    q, k, v, mask, block = _small_case(1)
    v = v.copy()
    v[..., 0] = 1.0
    o, rho, r = oracle.calibrate(q, k, v, mask, block)
    win = oracle.window_attention(q, k, v, mask, block)
    np.testing.assert_allclose(r[..., 0], 1.0 - rho, atol=1e-12)
    np.testing.assert_allclose(rho * win[..., 0] + r[..., 0], 1.0, atol=1e-12)
    np.testing.assert_allclose(o[..., 0], 1.0, atol=1e-12)
    assert np.all(rho > 0) and np.all(rho <= 1)


def test_zero_sparsity_is_dense_for_any_lambda():
    q, k, v, _, block = _small_case(2)
    nb = -(-q.shape[2] // block)
    mask = om.full_mask(nb)
    o, rho, r = oracle.calibrate(q, k, v, mask, block)
    np.testing.assert_allclose(rho, 1.0, atol=1e-12)
    np.testing.assert_allclose(r, 0.0, atol=1e-12)
    q2, k2, v2 = (x + 0.3 * _rand(x.shape, 50 + i) for i, x in enumerate((q, k, v)))
    dense2 = oracle.textbook_attention(q2[:1, :1], k2[:1, :1], v2[:1, :1])
    for lam, step in [(0.0, 1), (0.04, 3), (0.7, 4)]:
        out = oracle.sparse_step(q2, k2, v2, mask, block, rho, r, lam, step)
        np.testing.assert_allclose(out, oracle.full_attention(q2, k2, v2), atol=1e-12)
        np.testing.assert_allclose(out[:1, :1], dense2, atol=1e-12)


def test_reconstruction_on_calibration_inputs():
    q, k, v, mask, block = _small_case(3)
    o, rho, r = oracle.calibrate(q, k, v, mask, block)
    out = oracle.sparse_step(q, k, v, mask, block, rho, r, lam=0.0, step=1)
    np.testing.assert_allclose(out, o, atol=1e-12)


def test_rho_closed_form_and_monotone():
    q, k, v, mask, block = _small_case(4)
    L = q.shape[2]
    _, rho, _ = oracle.calibrate(q, k, v, mask, block)
    p = softmax(_scores(q, k), axis=-1)
    blocks = np.arange(L) // block
    keep = mask[blocks][:, blocks] != 0
    np.testing.assert_allclose(rho, (p * keep).sum(-1), atol=1e-12)
    bigger = mask.copy()
    bigger[0, :] = 1
    bigger[:, -1] = 1
    _, rho2, _ = oracle.calibrate(q, k, v, bigger, block)
    assert np.all(rho2 >= rho - 1e-15)
    assert np.any(rho2 > rho + 1e-6)


def test_post_softmax_masking_equals_rho_times_window():
    q, k, v, mask, block = _small_case(5)
    _, rho, _ = oracle.calibrate(q, k, v, mask, block)
    win = oracle.window_attention(q, k, v, mask, block)
    psm = oracle.post_softmax_masked(q, k, v, mask, block)
    np.testing.assert_allclose(psm, rho[..., None] * win, atol=1e-12)


def test_ramp_algebra():
    rho = np.linspace(0.0, 1.0, 11)
    np.testing.assert_allclose(oracle.ramp(rho, 0.0, 3), rho)
    for lam in (0.01, 0.04, 0.5):
        for step in (1, 2, 4):
            rt = oracle.ramp(rho, lam, step)
            assert np.all(rt <= 1.0) and np.all(rt >= rho)
    small = np.array([0.01, 0.2])
    np.testing.assert_allclose(oracle.ramp(small, 0.04, 3) - oracle.ramp(small, 0.04, 2),
                               oracle.ramp(small, 0.04, 2) - oracle.ramp(small, 0.04, 1))


def test_ramp_enters_sparse_step_linearly():
    q, k, v, mask, block = _small_case(6)
    o, rho, r = oracle.calibrate(q, k, v, mask, block)
    rho = rho * 0.5  # keep the clamp inactive
    win = oracle.window_attention(q, k, v, mask, block)
    out = oracle.sparse_step(q, k, v, mask, block, rho, r, lam=0.04, step=3)
    np.testing.assert_allclose(out, (rho * 1.12)[..., None] * win + r, atol=1e-12)


def test_empty_window_gives_residual():
    q, k, v, mask, block = _small_case(7)
    mask = mask.copy()
    mask[2, :] = 0
    o, rho, r = oracle.calibrate(q, k, v, mask, block)
    rows = np.arange(2 * block, 3 * block)
    np.testing.assert_allclose(rho[..., rows], 0.0, atol=1e-15)
    np.testing.assert_allclose(r[..., rows, :], o[..., rows, :], atol=1e-12)
    out = oracle.sparse_step(q, k, v, mask, block, rho, r, lam=0.04, step=2)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[..., rows, :], r[..., rows, :], atol=0)


def test_row_subset_matches_all_rows():
    q, k, v, mask, block = _small_case(8, L=37)
    rows = np.array([0, 5, 8, 17, 36])
    o, rho, r = oracle.calibrate(q, k, v, mask, block)
    os_, rhos, rs = oracle.calibrate(q, k, v, mask, block, rows=rows)
    np.testing.assert_allclose(os_, o[..., rows, :], atol=1e-14)
    np.testing.assert_allclose(rhos, rho[..., rows], atol=1e-14)
    np.testing.assert_allclose(rs, r[..., rows, :], atol=1e-14)
    out = oracle.sparse_step(q, k, v, mask, block, rho, r, 0.04, 2)
    outs = oracle.sparse_step(q, k, v, mask, block, rhos, rs, 0.04, 2, rows=rows)
    np.testing.assert_allclose(outs, out[..., rows, :], atol=1e-14)


def test_residual_cache_size_closed_form():
    """A residual of the attention output's shape for PixArt-Sigma at 1024x1024 (B=2 for CFG, 16 heads,
    64x64 tokens, head dim 72) in float32 is 36 MiB (review thread, answer to Q4 of the first review)."""
    r = np.zeros((2, 16, 4096, 72), dtype=np.float32)
    assert r.nbytes == 36 * 2 ** 20
