"""GPU parity of the comparators (window attention, post-softmax masking, DiTFastAttn).

Each comparator runs on the library's kernels and is checked element by
element against the oracle's definition of the same comparator, on the same
seeded inputs, to the bar of the main parity tests.  The cases cover the three
calibration kernels (64-token blocks with d <= 96 in bfloat16; the general
bfloat16 path at d = 128; float32), a ragged tail and a row with no kept block.
"""
import numpy as np
import pytest

import oracle
from oracle import masks as om
from tests.gpu_util import assert_parity, dev, host, log
from workloads import bf16_round, drift, make_qkv, random_mask

pytestmark = pytest.mark.gpu

CASES = [
    # name, dtype, B, H, L, d, block, mask maker
    ("bf16-b64-d64-band-tail", "bf16", 1, 2, 300, 64, 64, lambda nb: om.band_mask(nb, 2)),
    ("bf16-b64-d72-rand-emptyrow", "bf16", 2, 1, 260, 72, 64, lambda nb: random_mask(nb, nb, 0.5, 21, empty_rows=(1,))),
    ("bf16-b128-d128-band", "bf16", 1, 2, 300, 128, 128, lambda nb: om.band_mask(nb, 1)),
    ("f32-b32-d64-cog", "f32", 1, 2, 400, 64, 32, lambda nb: om.cogvideo3d_mask(nb, 2, 4)),
]


@pytest.fixture(scope="module")
def rt():
    import sparse_attention_diffusion_block_amd as rt_
    rt_.lib()
    return rt_


def _setup(rt, case, seed):
    name, dtype, B, H, L, d, block, make = case
    nb = -(-L // block)
    mask = make(nb).astype(np.uint8)
    scale = 1.0 if dtype == "bf16" else 0.125
    q, k, v = make_qkv(B, H, L, d, seed, scale=scale, dtype=dtype)
    idx = rt.index_build(mask, block)
    return dtype, block, mask, (q, k, v), idx, scale


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_difference_residual_and_unchanged_outputs(rt, case):
    import torch
    dtype, block, mask, (q, k, v), idx, _ = _setup(rt, case, 41)
    log(f"{case[0]}: difference residual")
    tq, tk, tv = (dev(x, dtype) for x in (q, k, v))
    o_m, rho_m, r_m = rt.calibrate(tq, tk, tv, idx)
    o_d, rho_d, r_d = rt.calibrate(tq, tk, tv, idx, residual="difference")
    torch.cuda.synchronize()
    # O and rho do not depend on the residual kind: identical bits
    assert torch.equal(o_m, o_d) and torch.equal(rho_m, rho_d)
    o_ref, _, _ = oracle.calibrate(q, k, v, mask, block)
    r_ref = oracle.ditfastattn_residual(o_ref, oracle.window_attention(q, k, v, mask, block))
    assert_parity(host(r_d), r_ref, dtype, "difference residual")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_attention(rt, case):
    import torch
    from sparse_attention_diffusion_block_amd.comparators import window_attention
    dtype, block, mask, (q, k, v), idx, _ = _setup(rt, case, 42)
    log(f"{case[0]}: window attention")
    g = window_attention(dev(q, dtype), dev(k, dtype), dev(v, dtype), idx)
    torch.cuda.synchronize()
    assert_parity(host(g), oracle.window_attention(q, k, v, mask, block), dtype, "window attention")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_post_softmax_masking_at_calibration(rt, case):
    """rho * window attention with the calibration's own rho is post-softmax masking exactly."""
    import torch
    from sparse_attention_diffusion_block_amd.comparators import post_softmax_step
    dtype, block, mask, (q, k, v), idx, _ = _setup(rt, case, 43)
    log(f"{case[0]}: post-softmax masking")
    _, rho_ref, _ = oracle.calibrate(q, k, v, mask, block)
    rho32 = rho_ref.astype(np.float32)
    g = post_softmax_step(dev(q, dtype), dev(k, dtype), dev(v, dtype), idx, torch.from_numpy(rho32).cuda(), 0.04, 0)
    torch.cuda.synchronize()
    # (rho rounded to float32 differs from the oracle's by < 2^-24 relative: far below the bar)
    assert_parity(host(g), oracle.post_softmax_masked(q, k, v, mask, block), dtype, "post-softmax masking")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ditfastattn_step(rt, case):
    """A later DiTFastAttn step on drifted inputs, both sides fed the oracle's residual in the I/O type."""
    import torch
    from sparse_attention_diffusion_block_amd.comparators import ditfastattn_step
    dtype, block, mask, (q, k, v), idx, scale = _setup(rt, case, 44)
    log(f"{case[0]}: DiTFastAttn step")
    o_ref, _, _ = oracle.calibrate(q, k, v, mask, block)
    r_dfa = oracle.ditfastattn_residual(o_ref, oracle.window_attention(q, k, v, mask, block))
    r_io = bf16_round(r_dfa.astype(np.float32)) if dtype == "bf16" else r_dfa.astype(np.float32)
    q2, k2, v2 = drift(q, k, v, 44, 1, scale=scale, dtype=dtype)
    g = ditfastattn_step(dev(q2, dtype), dev(k2, dtype), dev(v2, dtype), idx, dev(r_io, dtype))
    torch.cuda.synchronize()
    assert_parity(host(g), oracle.ditfastattn_step(q2, k2, v2, mask, block, r_io.astype(np.float64)), dtype,
                  "DiTFastAttn step")


def test_compare_chain_runs_and_ditfastattn_reconstructs(rt):
    """The comparison chain runs; on the calibration's own inputs DiTFastAttn's step (window
    attention plus the cached difference) gives back full attention."""
    import torch
    from sparse_attention_diffusion_block_amd.comparators import (METHODS, compare_chain, ditfastattn_calibrate,
                                                                  ditfastattn_step)
    from workloads import CONFIGS
    recs = compare_chain(config=2, T=3, steps=4)
    torch.cuda.synchronize()
    for rec in recs:
        log(str(rec))
        for m in METHODS:
            assert np.isfinite(rec[f"{m}_rel_l1"])
    assert recs[0]["rettention_rel_l1"] == 0.0 and recs[3]["rettention_rel_l1"] == 0.0
    cfg = CONFIGS[2]
    spec = cfg.masks[0]
    q, k, v = (dev(x, cfg.dtype) for x in make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, dtype=cfg.dtype))
    idx = rt.index_build(rt.mask_build(spec.kind, spec.nb, spec.w), cfg.block)
    full, r_dfa = ditfastattn_calibrate(q, k, v, idx)
    rec = ditfastattn_step(q, k, v, idx, r_dfa)
    torch.cuda.synchronize()
    diff = (rec.float() - full.float()).abs()
    # The difference residual is about minus the window output, several times larger than full
    # attention here, so its rounding to bfloat16 dominates the error: the bar is two roundings
    # relative to the residual's own magnitude (plus the full output's).
    scale = r_dfa.float().abs().sum() + full.float().abs().sum()
    assert float(diff.sum() / scale) <= 4e-3 and float(diff.max()) <= 2e-2


def test_library_loaded_before_any_torch_gpu_use():
    """Regression: loading the library first must still bind it to torch's HIP runtime
    (checked in a fresh process, where nothing has touched the GPU yet)."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, '.');"
            "import numpy as np;"
            "import sparse_attention_diffusion_block_amd as rt;"
            "rt.lib();"
            "idx = rt.index_build(np.eye(5, dtype=np.uint8), 64);"
            "assert idx.nnz == 5, idx.nnz;"
            "print('ok', flush=True)")
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=240)
    log(res.stdout + res.stderr[-2000:])
    assert res.returncode == 0 and "ok" in res.stdout
