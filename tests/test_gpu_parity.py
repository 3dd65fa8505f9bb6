"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Each kernel is checked in isolation on identical inputs:
  * index build: bit-exact CSR;
  * calibration: the same (Q, K, V) -> O, rho, R;
  * sparse step: the same (Q', K', V') and the same cached rho / R bits.
Small cases (all rows, several tiles, ragged tails, padded head dims, empty
rows) run first; then every workload at its full size on sampled rows, in
the same launch configuration the bench times.
"""
import math
import zlib

import numpy as np
import pytest

import oracle
from oracle import masks as om
from tests.gpu_util import assert_parity, dev, host, log
from workloads import CONFIGS, SWEEP_C3, MaskSpec, bf16_round, drift, make_cache, make_qkv, random_mask, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_diffusion_block_amd as m
    m.lib()
    return m


# ------------------------------------------------------------------ index build
def _index_cases():
    cases = []
    for n, cfg in CONFIGS.items():
        for spec in cfg.masks:
            cases.append((f"cfg{n}-{spec.label()}", om.build_mask(spec.kind, spec.nb, spec.w, spec.text_blocks,
                                                                   spec.tshift)))
    cases.append(("1x1", np.ones((1, 1), np.uint8)))
    cases.append(("empty-3x5", np.zeros((3, 5), np.uint8)))
    cases.append(("tall-70x3", random_mask(70, 3, 0.5, 1)))
    cases.append(("wide-3x200", random_mask(3, 200, 0.3, 2, empty_rows=(1,))))
    cases.append(("random-1500x1500", random_mask(1500, 1500, 0.01, 3, empty_rows=(0, 777, 1499))))
    cases.append(("dense-129x129", random_mask(129, 129, 0.97, 4)))
    cases.append(("values-not-01", (random_mask(40, 40, 0.5, 5) * np.uint8(7))))
    return cases


@pytest.mark.parametrize("name,mask", _index_cases(), ids=[c[0] for c in _index_cases()])
def test_index_build_bit_exact(rt, name, mask):
    idx = rt.index_build(mask, block=64)
    row_ptr, col_idx = om.csr_from_mask(mask)
    assert idx.nnz == len(col_idx)
    assert np.array_equal(idx.row_ptr.cpu().numpy(), row_ptr)
    assert np.array_equal(idx.col_idx[: idx.nnz].cpu().numpy(), col_idx)


# ------------------------------------------------------------------ small cases, all rows
SMALL = [
    # name, dtype, B, H, L, d, block, mask maker
    ("f32-diag-L1024", "f32", 1, 2, 1024, 64, 32, lambda nb: om.diag_mask(nb)),
    ("bf16-band-L300-tail", "bf16", 1, 2, 300, 64, 64, lambda nb: om.band_mask(nb, 2)),
    ("bf16-rand-d72", "bf16", 2, 1, 200, 72, 64, lambda nb: random_mask(nb, nb, 0.5, 11)),
    ("bf16-band-d88-tail", "bf16", 1, 2, 333, 88, 64, lambda nb: om.band_mask(nb, 3)),
    ("bf16-block128-d128", "bf16", 1, 1, 260, 128, 128, lambda nb: om.band_mask(nb, 1)),
    ("bf16-block32-emptyrow", "bf16", 1, 2, 130, 32, 32, lambda nb: random_mask(nb, nb, 0.5, 12, empty_rows=(1,))),
    ("bf16-cog-d16", "bf16", 1, 1, 500, 16, 32, lambda nb: om.cogvideo3d_mask(nb, 2, 5)),
    ("bf16-full-L1", "bf16", 1, 1, 1, 64, 32, lambda nb: om.full_mask(nb)),
    ("bf16-full-d128", "bf16", 1, 2, 200, 128, 64, lambda nb: om.full_mask(nb)),
    ("bf16-b64-d48-emptyrow", "bf16", 2, 2, 450, 48, 64, lambda nb: random_mask(nb, nb, 0.4, 14, empty_rows=(3,))),
    ("bf16-b64-d32-full", "bf16", 1, 2, 200, 32, 64, lambda nb: om.full_mask(nb)),
    ("bf16-b64-d64-full", "bf16", 1, 1, 256, 64, 64, lambda nb: om.full_mask(nb)),
    ("bf16-b64-d64-cog-tail", "bf16", 2, 2, 1000, 64, 64, lambda nb: om.cogvideo3d_mask(nb, 2, 4)),
    ("f32-rand-L257", "f32", 1, 2, 257, 64, 64, lambda nb: random_mask(nb, nb, 0.4, 13, empty_rows=(2,))),
    ("f32-band-d96-block128", "f32", 2, 1, 190, 96, 128, lambda nb: om.band_mask(nb, 1)),
    ("f32-full-d8", "f32", 1, 1, 100, 8, 32, lambda nb: om.full_mask(nb)),
    ("f32-cog-block32-d128", "f32", 1, 1, 300, 128, 32, lambda nb: om.cogvideo3d_mask(nb, 1, 3)),
    # 128-token blocks at every padded head dimension (the sparse step's work-group kernel)
    ("bf16-b128-d32-tail", "bf16", 1, 2, 330, 32, 128, lambda nb: om.band_mask(nb, 2)),
    ("bf16-b128-d64-emptyrow", "bf16", 2, 1, 520, 64, 128, lambda nb: random_mask(nb, nb, 0.5, 15, empty_rows=(2,))),
    ("bf16-b128-d96-tail", "bf16", 1, 2, 400, 96, 128, lambda nb: om.cogvideo3d_mask(nb, 1, 2)),
    ("bf16-b128-d72-full", "bf16", 1, 1, 300, 72, 128, lambda nb: om.full_mask(nb)),
    # 64-token blocks above d = 64 (the single-slot 2-wave groups): an empty row, tails, padded d
    ("bf16-b64-d96-emptyrow-tail", "bf16", 2, 1, 300, 96, 64,
     lambda nb: random_mask(nb, nb, 0.5, 16, empty_rows=(1,))),
    ("bf16-b64-d112-band-tail", "bf16", 1, 2, 460, 112, 64, lambda nb: om.band_mask(nb, 3)),
]


def _run_small(rt, dtype, B, H, L, d, block, make_mask, seed, qk_scale=1.0):
    import torch
    scale = 1.0 / math.sqrt(d) if dtype == "f32" else 1.0
    q, k, v = make_qkv(B, H, L, d, seed, scale=scale, dtype=dtype)
    if qk_scale != 1.0:
        q, k = (bf16_round(x * np.float32(qk_scale)) if dtype == "bf16" else x * np.float32(qk_scale) for x in (q, k))
    nb = -(-L // block)
    mask = make_mask(nb)
    idx = rt.index_build(mask, block)
    o_g, rho_g, r_g = rt.calibrate(dev(q, dtype), dev(k, dtype), dev(v, dtype), idx)
    torch.cuda.synchronize()
    o_o, rho_o, r_o = oracle.calibrate(q, k, v, mask, block)
    assert_parity(host(o_g), o_o, dtype, "calibrate O")
    assert_parity(host(rho_g), rho_o, dtype, "calibrate rho")
    assert_parity(host(r_g), r_o, dtype, "calibrate R")
    # the sparse step consumes the oracle's cache, rounded to the I/O dtype, on both sides
    rho_in = rho_o.astype(np.float32)
    r_in = bf16_round(r_o.astype(np.float32)) if dtype == "bf16" else r_o.astype(np.float32)
    q2, k2, v2 = drift(q, k, v, 900 + seed, 1, scale=scale, dtype=dtype)
    for lam, step in [(0.04, 1), (0.04, 4), (0.0, 2)]:
        o2_g = rt.sparse(dev(q2, dtype), dev(k2, dtype), dev(v2, dtype), idx,
                         torch.from_numpy(rho_in).cuda(), dev(r_in, dtype), lam=lam, step=step)
        torch.cuda.synchronize()
        o2_o = oracle.sparse_step(q2, k2, v2, mask, block, rho_in, r_in, lam, step)
        assert_parity(host(o2_g), o2_o, dtype, f"sparse O' (lambda={lam}, step={step})")


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_case_all_rows(rt, case):
    name, dtype, B, H, L, d, block, make_mask = case
    log(f"case {name}: dtype={dtype} B={B} H={H} L={L} d={d} block={block}")
    _run_small(rt, dtype, B, H, L, d, block, make_mask, seed=zlib.crc32(name.encode()) % 1000)


def _random_case(seed):
    """A seeded draw of dtype, head dimension (any multiple of the 16-byte granule up to 128), block,
    ragged length, batch / heads, mask density and empty rows."""
    g = np.random.default_rng(1000 + seed)
    dtype = "f32" if g.random() < 0.25 else "bf16"
    gran = 4 if dtype == "f32" else 8
    d = int(gran * g.integers(1, 128 // gran + 1))
    block = int(g.choice([32, 64, 128]))
    L = int(g.integers(1, 640))
    B, H = int(g.integers(1, 3)), int(g.integers(1, 4))
    nb = -(-L // block)
    density = float(g.uniform(0.05, 1.0))
    empty = tuple(int(x) for x in g.choice(nb, size=min(nb, int(g.integers(0, 3))), replace=False))
    qk_scale = 2.5 if g.random() < 0.2 else 1.0
    return dtype, B, H, L, d, block, (lambda n: random_mask(n, n, density, 2000 + seed, empty_rows=empty)), qk_scale


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes_all_rows(rt, seed):
    """Seeded random shapes through every kernel family the dispatch can pick, on all rows."""
    dtype, B, H, L, d, block, make_mask, qk_scale = _random_case(seed)
    log(f"case random-{seed}: dtype={dtype} B={B} H={H} L={L} d={d} block={block} qk_scale={qk_scale}")
    _run_small(rt, dtype, B, H, L, d, block, make_mask, seed=3000 + seed, qk_scale=qk_scale)


@pytest.mark.parametrize("d,block", [(64, 64), (72, 64), (128, 128)])
def test_large_scores_rescale_path(rt, d, block):
    """Q and K scaled by 3 give scores of standard deviation ~9: later key blocks exceed the
    running reference by far, which forces the softmax to re-anchor and rescale."""
    log(f"case large-scores d={d} block={block}")
    _run_small(rt, "bf16", 1, 2, 640, d, block, lambda nb: om.band_mask(nb, 5), seed=77, qk_scale=3.0)


# ------------------------------------------------------------------ worked example, block-lifted
def _lifted(dtype):
    """L=128, block 32, d=64: key and value rows are the one-hot vector of their block, query
    rows are 8 ln p in the first four dims, so a query's full attention puts mass p_b on block b
    and its output's first four entries are p itself (worked example of the review thread)."""
    L, d, block = 128, 64, 32
    blk = np.arange(L) // block
    kv = np.zeros((1, 1, L, d), np.float32)
    kv[0, 0, np.arange(L), blk] = 1.0

    def qrows(p):
        q = np.zeros((1, 1, L, d), np.float32)
        q[0, 0, :, :4] = 8.0 * np.log(np.asarray(p, np.float64))
        return bf16_round(q) if dtype == "bf16" else q

    mask = np.zeros((4, 4), np.uint8)
    mask[:, 1:3] = 1
    return L, d, block, kv, qrows, mask


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_worked_example_lifted(rt, dtype, golden):
    import torch
    g = golden("worked_example.txt")
    L, d, block, kv, qrows, mask = _lifted(dtype)
    tol = 1e-5 if dtype == "f32" else 2e-2
    idx = rt.index_build(mask, block)
    q = qrows(g["full_probs"])
    o, rho, r = rt.calibrate(dev(q, dtype), dev(kv, dtype), dev(kv, dtype), idx)
    torch.cuda.synchronize()
    o, rho, r = host(o)[0, 0], host(rho)[0, 0], host(r)[0, 0]
    np.testing.assert_allclose(o[:, :4], np.tile(g["full_probs"], (L, 1)), atol=tol)
    np.testing.assert_allclose(rho, g["rho"][0], atol=tol)
    np.testing.assert_allclose(r[:, :4], np.tile(g["residual"], (L, 1)), atol=tol)
    q2 = qrows(g["drift_full_probs"])
    rho_t = torch.from_numpy(np.full((1, 1, L), g["rho"][0], np.float32)).cuda()
    r_in = np.zeros((1, 1, L, d), np.float32)
    r_in[0, 0, :, :4] = g["residual"]
    o2 = rt.sparse(dev(q2, dtype), dev(kv, dtype), dev(kv, dtype), idx, rho_t, dev(r_in, dtype), lam=0.0, step=1)
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(o2)[0, 0, :, :4], np.tile(g["drift_rebuilt"], (L, 1)), atol=tol)


# ------------------------------------------------------------------ determinism
@pytest.mark.parametrize("d", [64, 72])
def test_bitwise_deterministic(rt, d):
    import torch
    q, k, v = make_qkv(1, 4, 1000, d, 3)
    nb = -(-1000 // 64)
    mask = om.band_mask(nb, 2)
    idx = rt.index_build(mask, 64)
    args = [dev(x, "bf16") for x in (q, k, v)]
    o1, rho1, r1 = rt.calibrate(*args, idx)
    o2, rho2, r2 = rt.calibrate(*args, idx)
    s1 = rt.sparse(*args, idx, rho1, r1, 0.04, 2)
    s2 = rt.sparse(*args, idx, rho1, r1, 0.04, 2)
    torch.cuda.synchronize()
    for a, b in [(o1, o2), (rho1, rho2), (r1, r2), (s1, s2)]:
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


# ------------------------------------------------------------------ full-size workloads, sampled rows
def _full_config(rt, n, nrows):
    import torch
    cfg = CONFIGS[n]
    log(f"config {n} ({cfg.name}): B={cfg.B} H={cfg.H} L={cfg.L} d={cfg.d} block={cfg.block} {cfg.dtype}")
    q, k, v = make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, scale=cfg.input_scale, dtype=cfg.dtype)
    q2, k2, v2 = drift(q, k, v, n, 1, sigma=cfg.drift_sigma, scale=cfg.input_scale, dtype=cfg.dtype)
    rows = sample_rows(cfg.L, cfg.block, nrows, seed=n)
    rho_c, r_c = make_cache(cfg.B, cfg.H, cfg.L, cfg.d, seed=n, dtype=cfg.dtype)
    tq, tk, tv = (dev(x, cfg.dtype) for x in (q, k, v))
    tq2, tk2, tv2 = (dev(x, cfg.dtype) for x in (q2, k2, v2))
    trho, tr = torch.from_numpy(rho_c).cuda(), dev(r_c, cfg.dtype)
    for spec in cfg.masks:
        log(f" mask {spec.label()}")
        mask = om.build_mask(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
        idx = rt.index_build(rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift), cfg.block)
        # calibration
        o_g, rho_g, r_g = rt.calibrate(tq, tk, tv, idx)
        torch.cuda.synchronize()
        o_o, rho_o, r_o = oracle.calibrate(q, k, v, mask, cfg.block, rows=rows)
        assert_parity(host(o_g[:, :, rows]), o_o, cfg.dtype, "calibrate O")
        assert_parity(host(rho_g[:, :, rows]), rho_o, cfg.dtype, "calibrate rho")
        assert_parity(host(r_g[:, :, rows]), r_o, cfg.dtype, "calibrate R")
        del o_g, rho_g, r_g
        # sparse step on the synthetic cache, steps 1 and T-1
        for step in sorted({1, cfg.sparse_steps}):
            o2_g = rt.sparse(tq2, tk2, tv2, idx, trho, tr, lam=cfg.lam, step=step)
            torch.cuda.synchronize()
            o2_o = oracle.sparse_step(q2, k2, v2, mask, cfg.block, rho_c[:, :, rows], r_c[:, :, rows],
                                      cfg.lam, step, rows=rows)
            assert_parity(host(o2_g[:, :, rows]), o2_o, cfg.dtype, f"sparse O' step {step}")
            del o2_g


@pytest.mark.timeout(900)
@pytest.mark.parametrize("n,nrows", [(1, 1024), (2, 96), (3, 48), (4, 96), (5, 12)])
def test_full_size_config(rt, n, nrows):
    _full_config(rt, n, nrows)


# ------------------------------------------------------------------ density sweep on the video workload's shapes
@pytest.mark.timeout(900)
def test_sparsity_sweep_c3_shapes(rt):
    """Band windows of 75 / 87.5 / 93.8 / 96.9% block sparsity at B=2, H=30, L=17776, d=64 (sampled rows)."""
    import torch
    cfg = CONFIGS[3]
    q, k, v = make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, dtype=cfg.dtype)
    q2, k2, v2 = drift(q, k, v, cfg.number, 1, sigma=cfg.drift_sigma, dtype=cfg.dtype)
    rows = sample_rows(cfg.L, cfg.block, 24, seed=33)
    rho_c, r_c = make_cache(cfg.B, cfg.H, cfg.L, cfg.d, seed=33, dtype=cfg.dtype)
    tq, tk, tv = (dev(x, cfg.dtype) for x in (q, k, v))
    tq2, tk2, tv2 = (dev(x, cfg.dtype) for x in (q2, k2, v2))
    trho, tr = torch.from_numpy(rho_c).cuda(), dev(r_c, cfg.dtype)
    for spec in SWEEP_C3:
        log(f" mask {spec.label()}")
        mask = om.build_mask(spec.kind, spec.nb, spec.w)
        assert int(mask.sum(axis=1).min()) == int(mask.sum(axis=1).max()) == spec.w
        idx = rt.index_build(rt.mask_build(spec.kind, spec.nb, spec.w), cfg.block)
        o_g, rho_g, r_g = rt.calibrate(tq, tk, tv, idx)
        torch.cuda.synchronize()
        o_o, rho_o, r_o = oracle.calibrate(q, k, v, mask, cfg.block, rows=rows)
        assert_parity(host(o_g[:, :, rows]), o_o, cfg.dtype, "calibrate O")
        assert_parity(host(rho_g[:, :, rows]), rho_o, cfg.dtype, "calibrate rho")
        assert_parity(host(r_g[:, :, rows]), r_o, cfg.dtype, "calibrate R")
        del o_g, rho_g, r_g
        o2_g = rt.sparse(tq2, tk2, tv2, idx, trho, tr, lam=cfg.lam, step=2)
        torch.cuda.synchronize()
        o2_o = oracle.sparse_step(q2, k2, v2, mask, cfg.block, rho_c[:, :, rows], r_c[:, :, rows], cfg.lam, 2,
                                  rows=rows)
        assert_parity(host(o2_g[:, :, rows]), o2_o, cfg.dtype, "sparse O'")
        del o2_g


def test_binding_rejects_mismatched_outputs(rt):
    """Caller-supplied outputs and rho are checked against Q's layout before anything is launched:
    the kernels write them with Q's strides, so a smaller or differently laid-out tensor would be
    overrun."""
    import torch
    B, H, L, d, block = 1, 2, 256, 64, 64
    log("case binding output checks")
    q = dev(bf16_round(np.random.default_rng(5).standard_normal((B, H, L, d)).astype(np.float32)), "bf16")
    idx = rt.index_build(om.band_mask(L // block, 2), block)
    o, rho, r = rt.calibrate(q, q, q, idx)
    bad = [torch.zeros((B, H, L, d), dtype=torch.float32, device=q.device),                 # dtype
           torch.zeros((B, H, L // 2, d), dtype=torch.bfloat16, device=q.device),          # shape
           torch.zeros((B, H, d, L), dtype=torch.bfloat16, device=q.device).transpose(2, 3)]  # strides
    for t in bad:
        with pytest.raises(ValueError):
            rt.sparse(q, q, q, idx, rho, r, out=t)
        with pytest.raises(ValueError):
            rt.calibrate(q, q, q, idx, out=(t, rho, r))
        with pytest.raises(ValueError):
            rt.calibrate(q, q, q, idx, out=(o, rho, t))
    for bad_rho in (rho.double(), rho[:, :, : L // 2], rho.transpose(0, 1)):
        with pytest.raises(ValueError):
            rt.sparse(q, q, q, idx, bad_rho, r)
        with pytest.raises(ValueError):
            rt.calibrate(q, q, q, idx, out=(o, bad_rho, r))
    # matching outputs are accepted and written in place
    o2 = rt.sparse(q, q, q, idx, rho, r, out=o)
    torch.cuda.synchronize()
    assert o2.data_ptr() == o.data_ptr() and torch.isfinite(o2.float()).all()


@pytest.mark.timeout(600)
def test_slice_beyond_32bit_offsets(rt):
    """One (batch, head) slice larger than 2 GiB (a padded row stride of 16384 elements): the fast
    kernels address a slice with 32-bit buffer offsets, so such a call must take the general
    kernels, which use 64-bit addresses.  Calibration and a sparse step on sampled rows, the last
    row included."""
    import torch
    B, H, L, d, block, sl = 1, 1, 65600, 64, 64, 16384
    assert (L - 1) * sl * 2 + d * 2 >= 1 << 31
    log(f"case slice over 2 GiB: L={L} d={d} row stride {sl} elements")
    q, k, v = make_qkv(B, H, L, d, 41, dtype="bf16")
    q2, k2, v2 = drift(q, k, v, 41, 1, dtype="bf16")
    nb = -(-L // block)
    mask = om.band_mask(nb, 3)
    idx = rt.index_build(mask, block)
    rows = np.array([0, 1, 63, 64, 32767, 32768, 65535, 65536, L - 1])

    def strided(x):
        buf = torch.zeros((B, H, L, sl), dtype=torch.bfloat16, device="cuda")
        view = buf[..., :d]
        view.copy_(torch.from_numpy(x).to("cuda").to(torch.bfloat16))
        return view

    tq, tk, tv = (strided(x) for x in (q, k, v))
    assert tq.stride() == (H * L * sl, L * sl, sl, 1)
    o_g, rho_g, r_g = rt.calibrate(tq, tk, tv, idx)
    torch.cuda.synchronize()
    o_o, rho_o, r_o = oracle.calibrate(q, k, v, mask, block, rows=rows)
    assert_parity(host(o_g[:, :, rows]), o_o, "bf16", "calibrate O")
    assert_parity(host(rho_g[:, :, rows]), rho_o, "bf16", "calibrate rho")
    assert_parity(host(r_g[:, :, rows]), r_o, "bf16", "calibrate R")
    del tq, tk, tv
    # the sparse step reads the GPU's own cache on the same strided layout
    tq2, tk2, tv2 = (strided(x) for x in (q2, k2, v2))
    o2_g = rt.sparse(tq2, tk2, tv2, idx, rho_g, r_g, lam=0.04, step=1)
    torch.cuda.synchronize()
    rho_h, r_h = host(rho_g).astype(np.float64), host(r_g).astype(np.float64)
    o2_o = oracle.sparse_step(q2, k2, v2, mask, block, rho_h[:, :, rows], r_h[:, :, rows], 0.04, 1, rows=rows)
    assert_parity(host(o2_g[:, :, rows]), o2_o, "bf16", "sparse O'")


def test_refresh_period_replays_from_a_hip_graph(rt):
    """One refresh period (a calibration and four sparse steps, outputs supplied by the caller)
    captured in a HIP graph: each entry point only launches kernels on the current stream, so the
    period replays without the host.  Three replays, with the outputs cleared eagerly in between,
    must each reproduce the eager run bit for bit (the kernels are deterministic)."""
    import torch
    B, H, L, d, block = 2, 4, 1000, 64, 64
    log("case HIP graph of one refresh period")
    nb = -(-L // block)
    idx = rt.index_build(om.cogvideo3d_mask(nb, 2, 4), block)
    sets = [make_qkv(B, H, L, d, 61, dtype="bf16")]
    for kstep in range(1, 5):
        sets.append(drift(*sets[-1], 61, kstep, dtype="bf16"))
    dsets = [tuple(dev(x, "bf16") for x in s) for s in sets]
    o_cal, r_cal = torch.empty_like(dsets[0][0]), torch.empty_like(dsets[0][0])
    rho = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    o_sp = [torch.empty_like(dsets[0][0]) for _ in range(4)]

    def period():
        rt.calibrate(*dsets[0], idx, out=(o_cal, rho, r_cal))
        for kstep in range(1, 5):
            rt.sparse(*dsets[kstep], idx, rho, r_cal, lam=0.04, step=kstep, out=o_sp[kstep - 1])

    period()
    torch.cuda.synchronize()
    want = [t.clone() for t in (o_cal, rho, r_cal, *o_sp)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        period()   # warm-up on the capture stream, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        period()
    for replay in range(3):
        for t in (o_cal, rho, r_cal, *o_sp):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("O", "rho", "R", "O'1", "O'2", "O'3", "O'4"), (o_cal, rho, r_cal, *o_sp), want):
            assert torch.equal(got, ref), f"replay {replay}: {name} differs from the eager run"
    # and the eager result itself against the oracle on the last sparse step
    mask = om.cogvideo3d_mask(nb, 2, 4)
    _, rho_o, r_o = oracle.calibrate(*sets[0], mask, block)
    rho_in = host(rho)
    r_in = host(r_cal)
    o4 = oracle.sparse_step(*sets[4], mask, block, rho_in, r_in, 0.04, 4)
    assert_parity(host(o_sp[3]), o4, "bf16", "sparse O' (step 4)")
    assert_parity(rho_in, rho_o, "bf16", "calibrate rho")
