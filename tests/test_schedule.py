"""The T-periodic schedule, the per-layer cache and chained drift runs.

CPU tests: the schedule's calibration steps and step counters, the cache
manager, and the refusal of a sparse step with nothing cached.  GPU tests: a
chained run through the C ABI step by step against the same chain run by the
oracle (whose cached R is stored in the I/O type, as the library stores it),
and the reconstruction invariant along a chain without drift (lambda = 0: every
sparse step reproduces full attention).
"""
import numpy as np
import pytest

import oracle
from oracle import masks as om
from sparse_attention_diffusion_block_amd.schedule import CacheManager, LayerCache, Rettention, Schedule
from workloads import bf16_round, drift, make_qkv

from tests.gpu_util import assert_parity, dev, host, log


def test_schedule_calibration_steps():
    s = Schedule(5)
    assert [t for t in range(16) if s.is_calibration(t)] == [0, 5, 10, 15]
    assert [s.k(t) for t in range(11)] == [0, 1, 2, 3, 4, 0, 1, 2, 3, 4, 0]
    assert all(Schedule(1).is_calibration(t) for t in range(6))
    s3, s7 = Schedule(3), Schedule(7)
    assert max(s3.k(t) for t in range(30)) == 2 and max(s7.k(t) for t in range(30)) == 6
    with pytest.raises(ValueError):
        Schedule(0)


def test_cache_manager_per_layer():
    cm = CacheManager()
    a, b = cm.get(0), cm.get(3)
    assert a is cm.get(0) and a is not b
    assert not a.valid and a.refreshed_at == -1
    assert cm.nbytes() == 0
    assert isinstance(a, LayerCache)


def test_sparse_step_without_calibration_is_refused():
    r = Rettention(index=None, schedule=Schedule(4), cache=CacheManager(), layer=2)
    with pytest.raises(RuntimeError, match="no calibration"):
        r(1, None, None, None)


def _oracle_chain(q, k, v, mask, block, T, steps, lam, sigma, dtype, seed):
    """The same chain on the CPU: calibrate every T steps, cache rho (float32) and R (I/O type)."""
    outs, rho_c, r_c = [], None, None
    for t in range(steps):
        if t > 0:
            q, k, v = drift(q, k, v, seed, t, sigma=sigma, dtype=dtype)
        if t % T == 0:
            o, rho, r = oracle.calibrate(q, k, v, mask, block)
            rho_c = rho.astype(np.float32).astype(np.float64)
            r_c = bf16_round(r.astype(np.float32)).astype(np.float64) if dtype == "bf16" else r
            outs.append(o)
        else:
            outs.append(oracle.sparse_step(q, k, v, mask, block, rho_c, r_c, lam, t % T))
    return outs


@pytest.mark.gpu
@pytest.mark.parametrize("T", [3, 5])
def test_chained_run_matches_oracle_chain(T):
    import torch
    import sparse_attention_diffusion_block_amd as rt
    B, H, L, d, block, lam, sigma, seed, steps = 1, 2, 300, 64, 64, 0.04, 0.05, 11, 7
    nb = -(-L // block)
    mask = om.band_mask(nb, 2)
    idx = rt.index_build(rt.mask_build(rt.MASK_BAND, nb, w=2), block)
    q, k, v = make_qkv(B, H, L, d, seed)
    ref = _oracle_chain(q, k, v, mask, block, T, steps, lam, sigma, "bf16", seed)
    run = Rettention(idx, Schedule(T), CacheManager(), layer=0, lam=lam)
    for t in range(steps):
        if t > 0:
            q, k, v = drift(q, k, v, seed, t, sigma=sigma)
        log(f"T={T} step {t}")
        o = run(t, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"))
        torch.cuda.synchronize()
        assert_parity(host(o), ref[t], "bf16", f"chained step {t} (T={T})")


@pytest.mark.gpu
def test_chain_without_drift_reconstructs_full_attention():
    import torch
    import sparse_attention_diffusion_block_amd as rt
    from sparse_attention_diffusion_block_amd.schedule import chained_drift_run
    recs = chained_drift_run(config=2, T=4, steps=5, sigma=0.0, lam=0.0)
    torch.cuda.synchronize()
    # Both sides are bfloat16 results of the library: the sparse output carries the rounding
    # of the cached R and its own, the calibration output its own, so the bar is twice the
    # single-rounding relative L1 bound.
    for rec in recs:
        log(str(rec))
        assert rec["rel_l1_vs_full"] <= 4e-3 and rec["maxabs_vs_full"] <= 2e-2, rec
    assert [r["kind"] for r in recs] == ["calibration", "sparse", "sparse", "sparse", "calibration"]


@pytest.mark.gpu
def test_dynamic_mask_run_invariants():
    """Calibration steps are exact; the static mask never moves; without drift the dynamic mask
    stays put and every sparse step rebuilds full attention (lambda = 0) for both mask kinds."""
    import torch
    from sparse_attention_diffusion_block_amd.schedule import dynamic_mask_run
    recs = dynamic_mask_run(config=2, T=3, steps=4, keep=3)
    torch.cuda.synchronize()
    for rec in recs:
        log(str(rec))
        if rec["k"] == 0:
            assert rec["rel_l1_vs_full"] == 0.0 and rec["rho_rel_err"] == 0.0 and rec["r_rel_err"] == 0.0
            assert rec["mask_moved"] == 0.0
        if rec["mask_kind"] == "static":
            assert rec["mask_moved"] == 0.0
    assert {r["mask_kind"] for r in recs} == {"static", "dynamic"}
    still = dynamic_mask_run(config=2, T=3, steps=3, keep=3, sigma=0.0, lam=0.0)
    torch.cuda.synchronize()
    for rec in still:
        log(str(rec))
        assert rec["mask_moved"] == 0.0
        assert rec["rel_l1_vs_full"] <= 4e-3 and rec["maxabs_vs_full"] <= 2e-2, rec


def test_cache_state_dict_round_trip_on_cpu(tmp_path):
    """The checkpoint format: host tensors keyed per layer, saved with torch.save and loaded back
    with weights_only=True (nothing in the file is executed); only calibrated layers are saved."""
    import torch
    cm = CacheManager()
    c = cm.get(4)
    c.rho = torch.rand(1, 2, 5)
    c.R = torch.randn(1, 2, 5, 8).to(torch.bfloat16)
    c.refreshed_at = 10
    cm.get(7)                                   # never calibrated: not saved
    path = tmp_path / "cache.pt"
    torch.save(cm.state_dict(), path)
    back = CacheManager()
    back.load_state_dict(torch.load(path, weights_only=True), device="cpu")
    assert sorted(back.layers) == [4]
    d = back.get(4)
    assert d.refreshed_at == 10 and d.valid
    assert torch.equal(d.rho.view(torch.int32), c.rho.view(torch.int32))
    assert torch.equal(d.R.view(torch.int16), c.R.view(torch.int16))


@pytest.mark.gpu
def test_checkpoint_resume_is_bit_identical(tmp_path):
    """The method's only cross-step state is the cache of rho and R (review thread, answer to Q4 of
    the first review: the residual cache).  Calibrate at step 0, checkpoint the cache to a file,
    reload it in a fresh cache manager and resume the schedule at step 3: every sparse step of the
    resumed run equals the uninterrupted run bit for bit."""
    import torch
    import sparse_attention_diffusion_block_amd as rt
    B, H, L, d, block, seed, T = 2, 3, 700, 64, 64, 21, 5
    nb = -(-L // block)
    idx = rt.index_build(rt.mask_build(rt.MASK_COGVIDEO3D, nb, text_blocks=1, tshift=3), block)
    sets = [make_qkv(B, H, L, d, seed)]
    for t in range(1, T):
        sets.append(drift(*sets[-1], seed, t))
    dsets = [tuple(dev(x, "bf16") for x in s) for s in sets]
    log("checkpoint: uninterrupted run")
    live = Rettention(idx, Schedule(T), CacheManager(), layer=2)
    want = [live(t, *dsets[t]).clone() for t in range(T)]
    torch.cuda.synchronize()
    # the same calibration, checkpointed after step 0
    first = Rettention(idx, Schedule(T), CacheManager(), layer=2)
    first(0, *dsets[0])
    torch.cuda.synchronize()
    path = tmp_path / "rettn_cache.pt"
    torch.save(first.cache.state_dict(), path)
    log(f"checkpoint: {path.stat().st_size} bytes written; resuming at step 3")
    cache = CacheManager()
    cache.load_state_dict(torch.load(path, weights_only=True), device="cuda")
    c0, c1 = first.cache.get(2), cache.get(2)
    assert torch.equal(c0.rho.view(torch.int32), c1.rho.view(torch.int32))
    assert torch.equal(c0.R.view(torch.int16), c1.R.view(torch.int16))
    resumed = Rettention(idx, Schedule(T), cache, layer=2)
    for t in range(3, T):
        got = resumed(t, *dsets[t])
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want[t].view(torch.int16)), f"step {t} differs after resuming"
