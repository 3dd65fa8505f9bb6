"""The work units behind every reported rate: effective flops of a sparse step, flops of a
calibration and algorithmic bytes per launch (bench.py and measure.py), pinned to the values the
hot-path scope table lists for each workload, and the attainable-roofline arithmetic."""
import numpy as np
import pytest

import bench
from oracle import masks as om
from sparse_attention_diffusion_block_amd import measure
from workloads import CONFIGS

# per workload and mask: (effective sparse flops, calibration flops, algorithmic bytes per launch),
# as listed (to the digits shown there) in the scope table's measurement section
TABLE = {
    (1, 0): (1.68e7, 5.37e8, 2.6e6),
    (2, 0): (4.83e9, 1.55e11, 94.9e6),
    (3, 0): (1.5355e11, 4.85e12, 686.9e6),
    (4, 0): (5.97e9, 1.96e11, 118.0e6),
    (4, 1): (1.20e10, 1.96e11, 118.0e6),
    (5, 0): (4.08e13, 1.63e14, 3.55e9),
    (5, 1): (2.05e13, 1.63e14, 3.55e9),
    (5, 2): (1.01e13, 1.63e14, 3.55e9),
    (5, 3): (5.07e12, 1.63e14, 3.55e9),
}


def _mask(cfg, spec):
    return om.build_mask(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)


def _digits(x):
    """Relative tolerance of a value printed with its leading digits only."""
    s = f"{x:.3e}".split("e")[0].rstrip("0").rstrip(".")
    decimals = len(s.split(".")[1]) if "." in s else 0
    return 0.5 * 10.0 ** (-decimals) / float(s)


@pytest.mark.parametrize("key", sorted(TABLE))
def test_counts_match_scope_table(key):
    n, m = key
    cfg = CONFIGS[n]
    spec = cfg.masks[m]
    f_sp, f_cal, nbytes, pairs = bench.workload_counts(cfg, _mask(cfg, spec))
    for got, want in zip((f_sp, f_cal, nbytes), TABLE[key]):
        assert got == pytest.approx(want, rel=_digits(want) + 1e-12), (key, got, want)


@pytest.mark.parametrize("key", sorted(TABLE))
def test_bench_and_measure_count_alike(key):
    n, m = key
    cfg = CONFIGS[n]
    mask = _mask(cfg, cfg.masks[m])
    assert bench.workload_counts(cfg, mask) == measure._counts(cfg, mask)


def test_effective_flops_by_brute_force_on_a_small_case():
    """4 d per kept (query, key) token pair, with the last block's true size."""
    class C:   # a small workload: L = 150 with block 64 leaves a 22-token tail block
        B, H, L, d, block, dtype = 1, 2, 150, 32, 64, "bf16"
    mask = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], dtype=np.uint8)
    tok = np.arange(C.L) // C.block
    pairs = sum(int(mask[tok[i], tok[j]]) for i in range(C.L) for j in range(C.L))
    f_sp, f_cal, nbytes, p = bench.workload_counts(C, mask)
    assert p == pairs
    assert f_sp == 4 * C.d * pairs * C.B * C.H
    assert f_cal == 4 * C.d * C.L * C.L * C.B * C.H
    assert nbytes == C.B * C.H * C.L * (5 * C.d * 2 + 4)


def test_roofline_bound_and_fraction():
    peak_flops, hbm = measure.MFMA_PEAK_TFLOPS * 1e12, measure.HBM_PEAK_GBS * 1e9
    ridge = peak_flops / hbm
    # below the ridge: HBM-bound, attainable = AI x bandwidth
    r = measure._roofline(1.5355e11, 686.9e6, 0.2076e-3)
    ai = 1.5355e11 / 686.9e6
    assert ai < ridge and r["bound"] == "hbm"
    assert r["attainable_tflops"] == pytest.approx(ai * hbm / 1e12, abs=0.05)
    assert r["roofline_frac"] == pytest.approx(1.5355e11 / 0.2076e-3 / (ai * hbm), abs=1e-4)
    # above the ridge: MFMA-bound, attainable = the matrix peak
    r = measure._roofline(4.08e13, 3.55e9, 42.4e-3)
    assert r["bound"] == "mfma" and r["attainable_tflops"] == pytest.approx(measure.MFMA_PEAK_TFLOPS, abs=0.05)
    assert r["roofline_frac"] == pytest.approx(4.08e13 / 42.4e-3 / peak_flops, abs=1e-4)


def test_stream_floor_scales_the_probe_to_the_step(monkeypatch, tmp_path):
    """The floor is the probe's best time scaled to the step's algorithmic bytes; a probe that is
    missing or prints nothing usable is reported in the line, not raised."""
    import json
    import subprocess
    exe = tmp_path / "sparse_attention_diffusion_block_amd" / "probe_stream"
    exe.parent.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert "error" in bench.stream_floor(0.2, 686_864_640)             # not built
    exe.write_text("")
    rec = {"pattern": "mix 4R+1W", "policy": "nt", "bytes": 682598400, "best_us": 120.0, "mean_us": 122.0}

    class Done:
        stdout = "warm-up line\n" + json.dumps(rec) + "\n"
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Done())
    out = bench.stream_floor(0.24, 686_864_640)
    floor = 0.120 * 686_864_640 / 682598400
    assert out["floor_ms"] == pytest.approx(floor, abs=1e-4)
    assert out["sparse_frac_of_floor"] == pytest.approx(floor / 0.24, abs=1e-4)
    assert out["probe"]["policy"] == "nt"

    class Garbled:
        stdout = "not json\n"
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Garbled())
    assert "error" in bench.stream_floor(0.24, 686_864_640)
