"""Measurements beyond the one-line bench: a density sweep, per-workload timings, peaks.

    python -m sparse_attention_diffusion_block_amd.measure sweep    [--runs 50]
    python -m sparse_attention_diffusion_block_amd.measure configs  [--runs 50]
    python -m sparse_attention_diffusion_block_amd.measure peaks
    python -m sparse_attention_diffusion_block_amd.measure dynamic  [--runs 50] [--keep 9] [--cache both]
    python -m sparse_attention_diffusion_block_amd.measure graph    [--runs 50]
    python -m sparse_attention_diffusion_block_amd.measure kernels  --config N [--runs 3] [--mask I]

sweep    the sparse step on the shapes of the CogVideoX-2B-like workload (B=2, H=30,
         L=17776, d=64, block 64) under band windows of 75 / 87.5 / 93.8 / 96.9% block
         sparsity and under its own 3D window + text column mask.  The pages claim that
         96.9% sparsity runs more than 2x faster than 87.5%; the sweep reports that ratio.
configs  calibration and sparse-step times of every workload and mask; the two image
         workloads, whose working sets fit in the 256 MB last-level cache, are also
         timed cold (after writing a 512 MiB buffer before each run).
dynamic  on the CogVideoX-2B-like shapes: the dynamic block-mask index (block means of Q
         and K, then a per-row top-keep; one read of Q and K, so HBM-bound; warm and cold), and the sparse
         step on that per-(batch, head) index beside the static mask shared by all heads
         and the same static mask given once per head.
graph    wall time of one refresh period (a calibration and the sparse steps until the next
         one, outputs preallocated) on the image and video workloads, launched eagerly from
         Python and replayed from a HIP graph: what the host's launch path costs per period.
kernels  the calibration and the sparse step of one workload (every mask, or the one `--mask`
         selects), `--runs` calls each, nothing timed: the program a counter-collecting
         profiler runs.
peaks    a measured matrix peak (a large bfloat16 GEMM through the vendor library) and
         a measured copy bandwidth, beside the datasheet figures.

Timing: HIP events on the current stream around 5 library calls queued back to back
(behind one more call, so the GPU is busy before the first event and the host's launch
time stays out of the sample), 10 warm-up calls, then `--runs` samples; median, p10 and
p90 of the per-call time.  Cold timings flush the cache before every single call.
Inputs are the seeded synthetic workloads; every call processes all (batch, head)
slices.  Output: one JSON object per measurement on stdout.
"""
import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0


def _time(fn, runs, warm=10, before=None, reps=5):
    """Per-call milliseconds: `runs` samples, each `reps` calls back to back between two events
    (queued behind each other, so the host's own launch time stays out of the sample once the
    first call is running).  With `before` (a cache flush) every call is its own sample, queued
    behind the flush, which keeps the GPU busy while it is launched."""
    import torch
    for _ in range(warm):
        if before:
            before()
        fn()
    reps = 1 if before else reps
    ts = []
    for _ in range(runs):
        if before:
            before()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        if not before:
            fn()                  # keeps the queue busy while the samples are being launched
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1) / reps)
    ts = np.array(ts)
    return {"median_ms": round(float(np.median(ts)), 4), "p10_ms": round(float(np.percentile(ts, 10)), 4),
            "p90_ms": round(float(np.percentile(ts, 90)), 4)}


def _counts(cfg, mask):
    """(effective flops of a sparse step, flops of a calibration, algorithmic bytes, kept token pairs)."""
    L, d, bl = cfg.L, cfg.d, cfg.block
    nb = mask.shape[0]
    sizes = np.array([min(bl, L - i * bl) for i in range(nb)], dtype=np.int64)
    pairs = int(sum(sizes[qb] * sizes[mask[qb] != 0].sum() for qb in range(nb)))
    bh = cfg.B * cfg.H
    esize = 2 if cfg.dtype == "bf16" else 4
    return 4.0 * d * pairs * bh, 4.0 * d * L * L * bh, bh * L * (5 * d * esize + 4), pairs


def _inputs(cfg):
    import torch
    from workloads import drift, make_cache, make_qkv
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, scale=cfg.input_scale, dtype=cfg.dtype)
    q2, k2, v2 = drift(q, k, v, cfg.number, 1, sigma=cfg.drift_sigma, dtype=cfg.dtype)
    rho, r = make_cache(cfg.B, cfg.H, cfg.L, cfg.d, seed=cfg.number, dtype=cfg.dtype)
    on = lambda x: torch.from_numpy(x).to("cuda").to(dt)
    return (on(q), on(k), on(v)), (on(q2), on(k2), on(v2)), torch.from_numpy(rho).to("cuda"), on(r)


def _sparse_record(cfg, spec, base, drifted, rho, r, runs, label, before=None):
    import torch
    from . import rettn as rt
    m = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
    idx = rt.index_build(m, cfg.block)
    f_sp, f_cal, nbytes, pairs = _counts(cfg, m)
    q, k, v = drifted
    out = torch.empty_like(q)
    t = _time(lambda: rt.sparse(q, k, v, idx, rho, r, lam=cfg.lam, step=1, out=out), runs, before=before)
    s = t["median_ms"] * 1e-3
    return {"what": "sparse_step", "workload": cfg.name, "mask": spec.label(), "timing": label,
            "block_sparsity": round(1.0 - float(m.sum()) / m.size, 6),
            "token_sparsity": round(1.0 - pairs / (cfg.L * cfg.L), 6), **t,
            "effective_tflops": round(f_sp / s / 1e12, 2), "mfma_frac": round(f_sp / s / 1e12 / MFMA_PEAK_TFLOPS, 4),
            "algorithmic_gbs": round(nbytes / s / 1e9, 1), "hbm_frac": round(nbytes / s / 1e9 / HBM_PEAK_GBS, 4),
            **_roofline(f_sp, nbytes, s)}


def _roofline(flops, nbytes, s):
    """Attainable rate at the kernel's arithmetic intensity, min(MFMA peak, AI x HBM peak), and the share
    of it reached."""
    ai = flops / nbytes
    attainable = min(MFMA_PEAK_TFLOPS * 1e12, ai * HBM_PEAK_GBS * 1e9)
    return {"flop_per_byte": round(ai, 2), "bound": "hbm" if attainable < MFMA_PEAK_TFLOPS * 1e12 else "mfma",
            "attainable_tflops": round(attainable / 1e12, 1), "roofline_frac": round(flops / s / attainable, 4)}


def cmd_sweep(args):
    from workloads import CONFIGS, SWEEP_C3
    cfg = CONFIGS[3]
    base, drifted, rho, r = _inputs(cfg)
    recs = []
    for spec in SWEEP_C3 + cfg.masks:
        rec = _sparse_record(cfg, spec, base, drifted, rho, r, args.runs, "warm")
        recs.append(rec)
        print(json.dumps(rec), flush=True)
    by_w = {rec["mask"]: rec for rec in recs}
    t875 = by_w[SWEEP_C3[1].label()]["median_ms"]
    t969 = by_w[SWEEP_C3[3].label()]["median_ms"]
    print(json.dumps({"what": "sweep_ratio", "workload": cfg.name,
                      "speedup_96.9_over_87.5": round(t875 / t969, 3),
                      "note": "the pages report more than 2x for this pair"}), flush=True)


def cmd_configs(args):
    import torch
    from workloads import CONFIGS
    from . import rettn as rt
    flush = None
    for n, cfg in CONFIGS.items():
        base, drifted, rho, r = _inputs(cfg)
        cold_too = n in (2, 4)
        if cold_too and flush is None:
            flush = torch.empty(512 << 18, dtype=torch.float32, device="cuda")   # 512 MiB
        runs = args.runs if n != 5 else max(3, args.runs // 10)
        for spec in cfg.masks:
            m = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
            idx = rt.index_build(m, cfg.block)
            f_sp, f_cal, nbytes, pairs = _counts(cfg, m)
            q, k, v = base
            o, rh, rr = torch.empty_like(q), torch.empty_like(rho), torch.empty_like(q)
            for label, before in [("warm", None)] + ([("cold", lambda: flush.zero_())] if cold_too else []):
                t = _time(lambda: rt.calibrate(q, k, v, idx, out=(o, rh, rr)), runs, warm=3 if n == 5 else 10,
                          before=before)
                s = t["median_ms"] * 1e-3
                print(json.dumps({"what": "calibrate", "workload": cfg.name, "mask": spec.label(), "timing": label,
                                  **t, "tflops": round(f_cal / s / 1e12, 2),
                                  "mfma_frac": round(f_cal / s / 1e12 / MFMA_PEAK_TFLOPS, 4),
                                  **_roofline(f_cal, nbytes, s)}), flush=True)
                print(json.dumps(_sparse_record(cfg, spec, base, drifted, rho, r, runs, label, before)), flush=True)
        del base, drifted, rho, r
        torch.cuda.empty_cache()


def cmd_dynamic(args):
    import torch
    from workloads import CONFIGS
    from . import rettn as rt
    cfg = CONFIGS[3]
    spec = cfg.masks[0]
    base, drifted, rho, r = _inputs(cfg)
    q, k, v = drifted
    nb = -(-cfg.L // cfg.block)
    ws = torch.empty(rt.dynamic_workspace_bytes(q, cfg.block), dtype=torch.uint8, device="cuda")
    dyn = rt.dynamic_index(q, k, args.keep, cfg.block, workspace=ws)
    nbytes = 2 * cfg.B * cfg.H * cfg.L * cfg.d * 2     # one read of Q and K
    # warm: back to back on one input (Q and K, 273 MB, partly stay in the 256 MB last-level cache);
    # cold: a 512 MiB write before every call, so Q and K come from HBM
    flush = torch.empty(512 << 18, dtype=torch.float32, device="cuda")
    for label, before in (("warm", None), ("cold", lambda: flush.zero_())):
        if args.cache not in (label, "both"):
            continue
        t = _time(lambda: rt.dynamic_index(q, k, args.keep, cfg.block, workspace=ws, out=dyn), args.runs,
                  before=before)
        s_ = t["median_ms"] * 1e-3
        print(json.dumps({"what": "dynamic_index", "workload": cfg.name, "keep": args.keep, "cache": label, **t,
                          "algorithmic_gbs": round(nbytes / s_ / 1e9, 1),
                          "hbm_frac": round(nbytes / s_ / 1e9 / HBM_PEAK_GBS, 4)}), flush=True)
    del flush
    static = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
    per_head = rt.index_build(np.broadcast_to(static, (cfg.H, nb, nb)).copy(), cfg.block)
    masks = {"static (shared)": (rt.index_build(static, cfg.block), static[None]),
             "static (one per head)": (per_head, static[None]),
             f"dynamic keep {args.keep} (one per slice)": (dyn, dyn.mask.cpu().numpy())}
    out = torch.empty_like(q)
    for label, (idx, m) in masks.items():
        pairs = sum(_counts(cfg, m[i])[3] for i in range(m.shape[0])) / m.shape[0]
        f_sp = 4.0 * cfg.d * pairs * cfg.B * cfg.H
        t = _time(lambda: rt.sparse(q, k, v, idx, rho, r, lam=cfg.lam, step=1, out=out), args.runs)
        s_ = t["median_ms"] * 1e-3
        print(json.dumps({"what": "sparse_step", "workload": cfg.name, "index": label,
                          "token_sparsity": round(1.0 - pairs / (cfg.L * cfg.L), 6), **t,
                          "effective_tflops": round(f_sp / s_ / 1e12, 2)}), flush=True)


def cmd_graph(args):
    import time
    import torch
    from workloads import CONFIGS, drift, make_qkv
    from . import rettn as rt
    for n in (2, 3, 4):
        cfg = CONFIGS[n]
        spec = cfg.masks[0]
        T = cfg.sparse_steps
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        sets = [make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, scale=cfg.input_scale, dtype=cfg.dtype)]
        for kstep in range(1, T + 1):
            sets.append(drift(*sets[-1], cfg.number, kstep, sigma=cfg.drift_sigma,
                              dtype=cfg.dtype))
        dev = [tuple(torch.from_numpy(x).to("cuda").to(dt) for x in st) for st in sets]
        del sets
        idx = rt.index_build(rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift), cfg.block)
        o_cal, r_cal = torch.empty_like(dev[0][0]), torch.empty_like(dev[0][0])
        rho = torch.empty(dev[0][0].shape[:3], dtype=torch.float32, device="cuda")
        o_sp = [torch.empty_like(dev[0][0]) for _ in range(T)]

        def period():
            rt.calibrate(*dev[0], idx, out=(o_cal, rho, r_cal))
            for kstep in range(1, T + 1):
                rt.sparse(*dev[kstep], idx, rho, r_cal, lam=cfg.lam, step=kstep, out=o_sp[kstep - 1])

        def wall(fn):
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.runs):
                fn()
            torch.cuda.synchronize()
            return (time.perf_counter() - t0) * 1e3 / args.runs

        eager = wall(period)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            period()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            period()
        replay = wall(g.replay)
        print(json.dumps({"what": "refresh_period", "workload": cfg.name, "mask": spec.label(),
                          "calls": 1 + T, "eager_ms": round(eager, 4), "graph_ms": round(replay, 4),
                          "graph_speedup": round(eager / replay, 3)}), flush=True)
        del dev, o_cal, r_cal, rho, o_sp, g
        torch.cuda.empty_cache()


def cmd_kernels(args):
    import torch
    from workloads import CONFIGS
    from . import rettn as rt
    cfg = CONFIGS[args.config]
    base, drifted, rho, r = _inputs(cfg)
    q, k, v = base
    o, rh, rr, o2 = torch.empty_like(q), torch.empty_like(rho), torch.empty_like(q), torch.empty_like(q)
    masks = cfg.masks if args.mask is None else (cfg.masks[args.mask],)
    for spec in masks:
        idx = rt.index_build(rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift), cfg.block)
        for _ in range(args.runs):
            rt.calibrate(q, k, v, idx, out=(o, rh, rr))
        for _ in range(args.runs):
            rt.sparse(*drifted, idx, rho, r, lam=cfg.lam, step=1, out=o2)
        torch.cuda.synchronize()
        print(json.dumps({"what": "kernels", "workload": cfg.name, "mask": spec.label(), "calls": args.runs}),
              flush=True)


def cmd_peaks(args):
    import torch
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(n, n, dtype=torch.bfloat16, device="cuda")
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda")
    t = _time(lambda: torch.matmul(a, b, out=c), args.runs)
    print(json.dumps({"what": "matrix_peak", "kernel": f"bf16 GEMM {n}^3 (vendor library)", **t,
                      "tflops": round(2.0 * n ** 3 / (t["median_ms"] * 1e-3) / 1e12, 1),
                      "datasheet_tflops": MFMA_PEAK_TFLOPS}), flush=True)
    nbytes = 1 << 30
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    t = _time(lambda: y.copy_(x), args.runs)
    print(json.dumps({"what": "copy_bandwidth", "bytes_each_way": nbytes, **t,
                      "gbs_read_plus_write": round(2.0 * nbytes / (t["median_ms"] * 1e-3) / 1e9, 1),
                      "datasheet_gbs": HBM_PEAK_GBS}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    for name in ("sweep", "configs", "peaks", "dynamic", "graph", "kernels"):
        sp = sub.add_parser(name)
        sp.add_argument("--runs", type=int, default=3 if name == "kernels" else 50)
        if name == "kernels":
            sp.add_argument("--config", type=int, required=True)
            sp.add_argument("--mask", type=int, default=None, help="only this mask of the workload (0-based)")
        if name == "dynamic":
            sp.add_argument("--keep", type=int, default=9)
            sp.add_argument("--cache", choices=("warm", "cold", "both"), default="both",
                            help="time the index back to back (warm), after a cache flush (cold), or both")
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    from . import rettn
    rettn.lib()
    return {"sweep": cmd_sweep, "configs": cmd_configs, "peaks": cmd_peaks, "dynamic": cmd_dynamic,
            "graph": cmd_graph, "kernels": cmd_kernels}[args.cmd](args) or 0


if __name__ == "__main__":
    sys.exit(main())
