"""GPU parity of per-head / per-slice block masks and of dynamic block masks.

Per-slice masks: the sliced CSR build is bit-exact against the oracle's
compaction of every slice, and calibration and sparse steps with one mask
per head (S = H) or per (batch, head) slice (S = B*H) match the oracle on every
kernel family (the 64-token sparse step, the 64/128-token calibration, the
general bfloat16 kernels, float32), with ragged tails and a row that keeps
nothing in one slice only.

Dynamic masks: the mask is an integer decision taken from float scores, and
the GPU scores in float32 where the oracle scores in float64, so a row may
legitimately differ where two blocks score within rounding of each other.
Every GPU row is therefore checked for validity against the oracle's exact
scores with a rounding bound derived from the inputs (every block the GPU kept
scores at least as high as every block it dropped, up to that bound); rows
with a clear margin can only pass by matching the oracle exactly, and the
count of rows that differ is logged.  The CSR that comes with the mask is
checked bit-exactly against the mask, and a sparse step on a dynamic index is
compared with the oracle on a case whose every row has a clear margin.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import dynamic as od
from oracle import masks as om
from tests.gpu_util import assert_parity, dev, host, log
from workloads import CONFIGS, bf16_round, drift, make_qkv, random_mask

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24   # float32 unit roundoff


@pytest.fixture(scope="module")
def rt():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_attention_diffusion_block_amd as m
    m.lib()
    return m


def _slice_masks(S, nb, seed, empty=None):
    """S different masks: random densities, one full, one diagonal, and (optionally) one empty row."""
    ms = np.stack([random_mask(nb, nb, 0.2 + 0.6 * ((i * 37) % 10) / 10, seed + i) for i in range(S)])
    ms[0] = om.full_mask(nb)
    if S > 1:
        ms[1] = om.diag_mask(nb)
    if empty is not None:
        s, row = empty
        ms[s, row] = 0
    return ms


# ------------------------------------------------------------------ sliced CSR
@pytest.mark.parametrize("S,nqb,nkb", [(6, 70, 70), (1, 5, 5), (3, 1, 200), (24, 130, 130)])
def test_sliced_index_build_bit_exact(rt, S, nqb, nkb):
    log(f"sliced index S={S} {nqb}x{nkb}")
    g = np.random.Generator(np.random.PCG64(S * 1000 + nqb))
    masks = (g.random((S, nqb, nkb)) < g.random((S, 1, 1))).astype(np.uint8)
    masks[0, 0] = 0
    idx = rt.index_build(masks, 64)
    rp = idx.row_ptr.cpu().numpy()
    ci = idx.col_idx.cpu().numpy()
    nnz_max = 0
    for s in range(S):
        row_ptr, col_idx = om.csr_from_mask(masks[s])
        assert np.array_equal(rp[s], row_ptr), s
        assert np.array_equal(ci[s * nqb * nkb: s * nqb * nkb + len(col_idx)], col_idx), s
        nnz_max = max(nnz_max, len(col_idx))
    assert idx.nnz == nnz_max and idx.slices == S and idx.col_stride == nqb * nkb


# ------------------------------------------------------------------ per-slice attention
SLICED = [
    # name, dtype, B, H, L, d, block, per ("head" | "slice")
    ("bf16-b64-d64-slice-tail", "bf16", 2, 3, 300, 64, 64, "slice"),
    ("bf16-b64-d64-head", "bf16", 2, 3, 450, 64, 64, "head"),
    ("bf16-b64-d72-slice", "bf16", 2, 2, 260, 72, 64, "slice"),
    ("bf16-b128-d128-head", "bf16", 2, 2, 300, 128, 128, "head"),
    ("bf16-b32-d64-slice", "bf16", 1, 3, 200, 64, 32, "slice"),
    ("f32-b32-d64-slice", "f32", 2, 2, 200, 64, 32, "slice"),
    ("f32-b64-d96-head", "f32", 2, 2, 190, 96, 64, "head"),
]


@pytest.mark.parametrize("case", SLICED, ids=[c[0] for c in SLICED])
def test_per_slice_calibrate_and_sparse(rt, case):
    import torch
    name, dtype, B, H, L, d, block, per = case
    log(f"case {name}")
    nb = -(-L // block)
    S = H if per == "head" else B * H
    masks = _slice_masks(S, nb, 500 + len(name), empty=(S - 1, nb // 2))
    scale = 1.0 / math.sqrt(d) if dtype == "f32" else 1.0
    q, k, v = make_qkv(B, H, L, d, 60 + len(name), scale=scale, dtype=dtype)
    idx = rt.index_build(masks, block)
    assert idx.slices == S
    o_g, rho_g, r_g = rt.calibrate(dev(q, dtype), dev(k, dtype), dev(v, dtype), idx)
    torch.cuda.synchronize()
    o_o, rho_o, r_o = oracle.calibrate(q, k, v, masks, block)
    assert_parity(host(o_g), o_o, dtype, "calibrate O")
    assert_parity(host(rho_g), rho_o, dtype, "calibrate rho")
    assert_parity(host(r_g), r_o, dtype, "calibrate R")
    rho_in = rho_o.astype(np.float32)
    r_in = bf16_round(r_o.astype(np.float32)) if dtype == "bf16" else r_o.astype(np.float32)
    q2, k2, v2 = drift(q, k, v, 70 + len(name), 1, scale=scale, dtype=dtype)
    o2_g = rt.sparse(dev(q2, dtype), dev(k2, dtype), dev(v2, dtype), idx, torch.from_numpy(rho_in).cuda(),
                     dev(r_in, dtype), lam=0.04, step=2)
    torch.cuda.synchronize()
    o2_o = oracle.sparse_step(q2, k2, v2, masks, block, rho_in, r_in, 0.04, 2)
    assert_parity(host(o2_g), o2_o, dtype, "sparse O'")


def test_per_head_index_differs_from_shared(rt):
    """Guard against a kernel that ignores the slice: per-head masks that differ must change the output."""
    import torch
    B, H, L, d, block = 1, 2, 256, 64, 64
    q, k, v = make_qkv(B, H, L, d, 5)
    nb = L // block
    shared = rt.index_build(om.diag_mask(nb), block)
    per_head = rt.index_build(np.stack([om.diag_mask(nb), om.full_mask(nb)]), block)
    _, rho_s, _ = rt.calibrate(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), shared)
    _, rho_h, _ = rt.calibrate(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), per_head)
    torch.cuda.synchronize()
    assert torch.equal(rho_s[0, 0], rho_h[0, 0])
    # head 1 keeps every block under its own mask: rho = D_in (1 / D), 1 up to that product's rounding
    assert float((rho_h[0, 1] - 1.0).abs().max()) <= 1e-6
    assert float(rho_s[0, 1].max()) < 0.99


# ------------------------------------------------------------------ dynamic masks
def _score_bounds(q, k, block):
    """Oracle scores and a bound on the float32 error of the GPU's scores, per slice [nb, nb]."""
    L, d = q.shape
    nb = -(-L // block)
    qm, km = od.block_means(q, block), od.block_means(k, block)
    dq, dk = np.zeros((nb, d)), np.zeros((nb, d))
    for i in range(nb):
        n = min(L, (i + 1) * block) - i * block
        # a float32 sum of n terms in any order, then one division: within 2 n u of the mean of |x|
        dq[i] = 2 * n * U32 * np.abs(q[i * block:i * block + n]).mean(0) + U32 * np.abs(qm[i])
        dk[i] = 2 * n * U32 * np.abs(k[i * block:i * block + n]).mean(0) + U32 * np.abs(km[i])
    aq, ak = np.abs(qm), np.abs(km)
    eps = aq @ dk.T + dq @ ak.T + dq @ dk.T + 2 * d * U32 * ((aq + dq) @ (ak + dk).T)
    return qm @ km.T, eps


def _check_dynamic(gmask, g_rp, g_ci, q, k, block, keep):
    """Validity of every GPU row against exact scores; CSR consistent with the mask.  Returns
    (rows, rows equal to the oracle's)."""
    B, H, L, _ = q.shape
    nb = -(-L // block)
    kk = min(keep, nb)
    ref = od.dynamic_mask(q, k, block, keep)
    assert gmask.shape == ref.shape
    assert np.all(gmask.sum(-1) == kk)
    assert np.all(gmask[:, np.arange(nb), np.arange(nb)] == 1)
    equal = 0
    for s in range(B * H):
        b, h = divmod(s, H)
        sc, eps = _score_bounds(q[b, h].astype(np.float64), k[b, h].astype(np.float64), block)
        row_ptr, col_idx = om.csr_from_mask(gmask[s])
        assert np.array_equal(g_rp[s], row_ptr)
        assert np.array_equal(g_ci[s * nb * kk:(s + 1) * nb * kk], col_idx)
        for a in range(nb):
            if np.array_equal(gmask[s, a], ref[s, a]):
                equal += 1
                continue
            kept = [j for j in range(nb) if gmask[s, a, j] and j != a]
            dropped = [j for j in range(nb) if not gmask[s, a, j]]
            lo = min(sc[a, j] + eps[a, j] for j in kept)
            hi = max(sc[a, j] - eps[a, j] for j in dropped)
            assert lo >= hi, f"slice {s} row {a}: kept {kept} not a top set within rounding"
    return B * H * nb, equal


DYN = [
    # name, dtype, B, H, L, d, block, keep
    ("bf16-b64-d64-nb79-tail", "bf16", 2, 3, 5000, 64, 64, 9),
    ("bf16-b64-d72", "bf16", 1, 2, 4173, 72, 64, 7),
    ("bf16-b128-d128", "bf16", 1, 2, 9000, 128, 128, 5),
    ("bf16-b32-d64-nb200", "bf16", 1, 2, 6400, 64, 32, 12),
    ("f32-b32-d64-nb94", "f32", 1, 2, 3000, 64, 32, 6),
    ("bf16-keep1", "bf16", 1, 1, 640, 64, 64, 1),
    ("bf16-keep-all", "bf16", 1, 1, 700, 64, 64, 50),
    ("bf16-one-block", "bf16", 1, 1, 40, 64, 64, 3),
    # every width of the per-lane score registers: 3, 7, 16 (more than 512 blocks) and 32 (the
    # largest supported count, 2048 blocks)
    ("bf16-b64-nb150-tail", "bf16", 1, 1, 150 * 64 - 17, 64, 64, 9),
    ("bf16-b32-d32-nb420", "bf16", 1, 1, 420 * 32, 32, 32, 9),
    ("bf16-b64-nb600", "bf16", 1, 1, 600 * 64, 64, 64, 9),
    ("bf16-b64-nb2048-max", "bf16", 1, 1, 2048 * 64, 64, 64, 9),
]


@pytest.mark.parametrize("case", DYN, ids=[c[0] for c in DYN])
def test_dynamic_index_against_oracle(rt, case):
    import torch
    name, dtype, B, H, L, d, block, keep = case
    log(f"dynamic {name}")
    scale = 1.0 / math.sqrt(d) if dtype == "f32" else 1.0
    q, k, _ = make_qkv(B, H, L, d, 300 + len(name), scale=scale, dtype=dtype)
    idx = rt.dynamic_index(dev(q, dtype), dev(k, dtype), keep, block)
    torch.cuda.synchronize()
    nb = -(-L // block)
    assert idx.slices == B * H and idx.col_stride == nb * min(keep, nb) and idx.nnz == idx.col_stride
    rows, equal = _check_dynamic(idx.mask.cpu().numpy(), idx.row_ptr.cpu().numpy(), idx.col_idx.cpu().numpy(),
                                 q, k, block, keep)
    log(f"  {equal} of {rows} rows equal to the oracle's; the rest are near-ties, valid within rounding")


def test_dynamic_index_full_size_video_workload(rt):
    """The full video workload (B 2, H 30, L 17776, d 64, block 64), keep 9: about its static mask's density."""
    import torch
    cfg = CONFIGS[3]
    log("dynamic full size")
    q, k, _ = make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, dtype=cfg.dtype)
    idx = rt.dynamic_index(dev(q, "bf16"), dev(k, "bf16"), 9, cfg.block)
    torch.cuda.synchronize()
    rows, equal = _check_dynamic(idx.mask.cpu().numpy(), idx.row_ptr.cpu().numpy(), idx.col_idx.cpu().numpy(),
                                 q, k, cfg.block, 9)
    log(f"  {equal} of {rows} rows equal to the oracle's")
    assert equal >= 0.95 * rows


def test_dynamic_index_reuses_buffers(rt):
    """A second call into the same buffers (another step's inputs) gives that step's mask."""
    import torch
    B, H, L, d, block, keep = 1, 2, 1300, 64, 64, 4
    q, k, v = make_qkv(B, H, L, d, 8)
    q2, k2, _ = drift(q, k, v, 8, 1, sigma=1.0)
    first = rt.dynamic_index(dev(q, "bf16"), dev(k, "bf16"), keep, block)
    m1 = first.mask.clone()
    again = rt.dynamic_index(dev(q2, "bf16"), dev(k2, "bf16"), keep, block, out=first)
    fresh = rt.dynamic_index(dev(q2, "bf16"), dev(k2, "bf16"), keep, block)
    torch.cuda.synchronize()
    assert again is first
    assert torch.equal(again.mask, fresh.mask) and torch.equal(again.col_idx, fresh.col_idx)
    assert not torch.equal(m1, fresh.mask)


def test_sparse_step_on_dynamic_index(rt):
    """Calibrate on one step's dynamic mask, then a sparse step on the next step's: both against
    the oracle's masks (every row of this case has a clear margin, so the masks are the oracle's)."""
    import torch
    B, H, L, d, block, keep = 2, 2, 1000, 64, 64, 4
    # seed 32: on both steps every row's gap between its last kept and first dropped block is more
    # than 1.8 times the float32 rounding bound, so the GPU's masks must be the oracle's
    q, k, v = make_qkv(B, H, L, d, 32)
    q2, k2, v2 = drift(q, k, v, 32, 1, sigma=0.5)
    m_cal, m_step = od.dynamic_mask(q, k, block, keep), od.dynamic_mask(q2, k2, block, keep)
    assert not np.array_equal(m_cal, m_step)
    i_cal = rt.dynamic_index(dev(q, "bf16"), dev(k, "bf16"), keep, block)
    i_step = rt.dynamic_index(dev(q2, "bf16"), dev(k2, "bf16"), keep, block)
    torch.cuda.synchronize()
    assert np.array_equal(i_cal.mask.cpu().numpy(), m_cal) and np.array_equal(i_step.mask.cpu().numpy(), m_step)
    o_g, rho_g, r_g = rt.calibrate(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), i_cal)
    torch.cuda.synchronize()
    o_o, rho_o, r_o = oracle.calibrate(q, k, v, m_cal, block)
    assert_parity(host(rho_g), rho_o, "bf16", "calibrate rho (dynamic mask)")
    assert_parity(host(r_g), r_o, "bf16", "calibrate R (dynamic mask)")
    rho_in, r_in = rho_o.astype(np.float32), bf16_round(r_o.astype(np.float32))
    o2_g = rt.sparse(dev(q2, "bf16"), dev(k2, "bf16"), dev(v2, "bf16"), i_step, torch.from_numpy(rho_in).cuda(),
                     dev(r_in, "bf16"), lam=0.04, step=1)
    torch.cuda.synchronize()
    assert_parity(host(o2_g), oracle.sparse_step(q2, k2, v2, m_step, block, rho_in, r_in, 0.04, 1), "bf16",
                  "sparse O' on the next step's dynamic mask")
