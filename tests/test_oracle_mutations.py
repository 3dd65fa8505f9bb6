"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's source (a
dropped term, a wrong sign or index, a transposed operand, a misplaced ramp)
and checks that at least one pin of tests/test_oracle.py then fails.  The
planted copy lives only in this test; the oracle itself is never changed.
"""
import os
import types

import numpy as np
import pytest

import tests.test_oracle as pins
from tests.conftest import read_golden

SRC = open(os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "rettn.py")).read()

MUTATIONS = [
    ("rho uses the window mass twice", "rho[b, h, pos] = D_in / D", "rho[b, h, pos] = D_in / D_in"),
    ("residual keeps window keys", "r[b, h, pos] = (e[:, ~keep] @ v[b, h][~keep])", "r[b, h, pos] = (e[:, keep] @ v[b, h][keep])"),
    ("residual uses the window denominator", "r[b, h, pos] = (e[:, ~keep] @ v[b, h][~keep]) / D[:, None]",
     "r[b, h, pos] = (e[:, ~keep] @ v[b, h][~keep]) / D_in[:, None]"),
    ("sign of the max shift", "e = np.exp(s - m)\n                D = e.sum", "e = np.exp(m - s)\n                D = e.sum"),
    ("scores transposed (k_i . q_j)", "s = t * (qi @ k[b, h].T)", "s = t * (k[b, h][rows[pos]] @ q[b, h].T)"),
    ("value operand transposed", "o[b, h, pos] = (e @ v[b, h])", "o[b, h, pos] = (e @ v[b, h][::-1])"),
    ("scale uses L instead of d", "t = tau(d)\n    groups = _rows_by_block(rows, block)\n    for b in range(B):\n        for h in range(H):\n            m_bh = slice_mask(mask, b, h, B, H)\n            for qb, pos in groups.items():\n                keep = key_keep(m_bh, block, L, qb)\n                qi",
     "t = tau(L)\n    groups = _rows_by_block(rows, block)\n    for b in range(B):\n        for h in range(H):\n            m_bh = slice_mask(mask, b, h, B, H)\n            for qb, pos in groups.items():\n                keep = key_keep(m_bh, block, L, qb)\n                qi"),
    ("per-head masks swapped between heads", "        return mask[h]\n", "        return mask[H - 1 - h]\n"),
    ("per-slice masks indexed head-major", "        return mask[b * H + h]\n", "        return mask[h * B + b]\n"),
    ("residual not added", "return scale[..., None] * o_sp + r", "return scale[..., None] * o_sp"),
    ("ramp applied to the residual", "return scale[..., None] * o_sp + r", "return scale[..., None] * (o_sp + r)"),
    ("ramp sign", "rho * (1.0 + float(lam) * float(step))", "rho * (1.0 - float(lam) * float(step))"),
    ("window uses the next block", "return np.asarray(mask)[qb, blocks] != 0", "return np.asarray(mask)[min(qb + 1, np.asarray(mask).shape[0] - 1), blocks] != 0"),
    ("key block index off by one", "blocks = np.arange(L) // block", "blocks = (np.arange(L) + 1) // block"),
    ("window softmax over all keys", "kk, vv = k[b, h][keep], v[b, h][keep]", "kk, vv = k[b, h], v[b, h]"),
]


def _mutant(old, new):
    assert old in SRC, f"mutation anchor not found: {old[:40]}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    # the mutant takes the same place as the oracle inside the pin functions
    ns = types.SimpleNamespace(**{k: getattr(mod, k) for k in dir(mod) if not k.startswith("__")})
    return ns


def _run_pins(m):
    """Run every pin against module-like `m`; return the number that fail."""
    import oracle as real
    failures = 0
    saved = pins.oracle
    pins.oracle = m
    try:
        checks = [
            lambda: pins.test_worked_example_calibration(read_golden),
            lambda: pins.test_worked_example_drift(read_golden),
            lambda: pins.test_calibration_is_textbook_attention(1, 2, 7, 4, 3),
            lambda: pins.test_all_masks_3x3_brute_force(),
            lambda: pins.test_per_slice_masks_brute_force(),
            lambda: pins.test_sum_to_one(),
            lambda: pins.test_reconstruction_on_calibration_inputs(),
            lambda: pins.test_ramp_algebra(),
            lambda: pins.test_ramp_enters_sparse_step_linearly(),
            lambda: pins.test_empty_window_gives_residual(),
        ]
        for c in checks:
            try:
                with np.errstate(all="ignore"):
                    c()
            except Exception:
                failures += 1
    finally:
        pins.oracle = saved
    return failures


def test_unmutated_copy_passes_every_pin():
    assert _run_pins(_mutant("def tau(d):", "def tau(d):")) == 0


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(name, old, new):
    assert _run_pins(_mutant(old, new)) >= 1, f"no pin caught: {name}"
