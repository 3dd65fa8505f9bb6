"""Oracle mask generators and CSR against definitions written out as sets (no GPU)."""
import numpy as np
import pytest

from oracle import masks as om
from workloads import CONFIGS


def _golden_counts():
    import os
    rows = []
    path = os.path.join(os.path.dirname(__file__), "golden", "mask_counts.txt")
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line or "=" in line:
                continue
            kind, nb, w, text, tshift, nnz = line.split()
            rows.append((kind, int(nb), int(w), int(text), int(tshift), int(nnz)))
    return rows


KINDS = {"diag": om.DIAG, "band": om.BAND, "cogvideo3d": om.COGVIDEO3D}


def _set_definition(kind, nb, w, text, tshift):
    """Kept key blocks per query block, from the definitions, as Python sets."""
    out = []
    for qb in range(nb):
        if kind == "diag":
            s = {qb}
        elif kind == "band":
            start = min(max(qb - (w - 1) // 2, 0), nb - w)
            s = set(range(start, start + w))
        else:
            s = set(range(min(text, nb))) | {x for x in (qb - 1, qb, qb + 1, qb - tshift, qb + tshift) if 0 <= x < nb}
        out.append(s)
    return out


@pytest.mark.parametrize("row", _golden_counts())
def test_generator_counts_and_sets(row):
    kind, nb, w, text, tshift, nnz = row
    m = om.build_mask(KINDS[kind], nb, w=w, text_blocks=text, tshift=tshift)
    sets = _set_definition(kind, nb, w, text, tshift)
    for qb in range(nb):
        assert set(np.nonzero(m[qb])[0].tolist()) == sets[qb]
    assert int(m.sum()) == nnz
    row_ptr, col_idx = om.csr_from_mask(m)
    assert row_ptr[0] == 0 and row_ptr[-1] == nnz and len(col_idx) == nnz
    for qb in range(nb):
        seg = col_idx[row_ptr[qb]:row_ptr[qb + 1]]
        assert list(seg) == sorted(sets[qb])


def test_band_always_w_per_row():
    for nb in (1, 2, 7, 64):
        for w in range(1, nb + 1):
            assert np.all(om.band_mask(nb, w).sum(1) == w)


def test_page_sparsity_fractions():
    import os
    from tests.conftest import read_golden
    g = read_golden("mask_counts.txt")
    # a window of 1/8 of the blocks keeps 1/8 of the pairs: 87.5 % sparsity
    assert 1 - om.mask_density(om.band_mask(64, 8)) == pytest.approx(g["one_eighth_window_sparsity"][0], abs=0)
    assert 1 - om.mask_density(om.band_mask(64, 2)) == pytest.approx(g["one_32nd_window_sparsity"][0], abs=0)
    assert 1 - om.mask_density(om.diag_mask(32)) == pytest.approx(g["one_32nd_window_sparsity"][0], abs=0)


def test_workload_sparsities():
    expected = {1: [0.96875], 2: [0.96875], 3: [1 - 2443 / 278 ** 2], 4: [1 - 2 / 66, 1 - 4 / 66],
                5: [0.75, 1 - 113 / 900, 1 - 56 / 900, 1 - 28 / 900]}
    for n, cfg in CONFIGS.items():
        for spec, exp in zip(cfg.masks, expected[n]):
            m = om.build_mask(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
            assert m.shape == (cfg.nb, cfg.nb)
            assert 1 - om.mask_density(m) == pytest.approx(exp, abs=1e-12)


def test_csr_random_masks_bruteforce():
    rng = np.random.Generator(np.random.PCG64(3))
    for trial in range(50):
        nq, nk = rng.integers(1, 40, size=2)
        m = (rng.random((nq, nk)) < rng.random()).astype(np.uint8)
        row_ptr, col_idx = om.csr_from_mask(m)
        assert len(row_ptr) == nq + 1
        flat = [(qb, kb) for qb in range(nq) for kb in range(nk) if m[qb, kb]]
        rebuilt = [(qb, int(col_idx[e])) for qb in range(nq) for e in range(row_ptr[qb], row_ptr[qb + 1])]
        assert rebuilt == flat
