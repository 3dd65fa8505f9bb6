#!/usr/bin/env python3
"""Benchmark of the Re-ttention hot path on one MI355X.

One step is one full refresh period of the method on the CogVideoX-2B-like
workload (B=2, H=30, L=17776 = 226 text + 13 x 30 x 45 video tokens, d=64,
bfloat16, block 64, 3D window + text column at 96.84% sparsity):
    static mask build (host) -> block-index build (GPU, one sync)
    -> calibration (full attention, rho, R) on step-0 inputs
    -> 4 sparse steps on drifted inputs (random walk, sigma = 0.05), lambda = 0.04.
Inputs sit in HBM before the timed region starts.

The headline value is the sparse step's effective throughput: the flops of
the kept blocks only (4 d per kept (query, key) pair) divided by the mean
duration of the sparse-step kernel, measured with HIP events on the stream the
library launches on, over the timed steps.  ms_per_step is the wall time of
the whole period.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix peak, TFLOP/s


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def workload_counts(cfg, mask):
    """Effective flops of one sparse step, flops of a calibration, algorithmic bytes of either kernel."""
    L, d, bl = cfg.L, cfg.d, cfg.block
    nb = mask.shape[0]
    sizes = np.array([min(bl, L - i * bl) for i in range(nb)], dtype=np.int64)
    pairs = int(sum(sizes[qb] * sizes[mask[qb] != 0].sum() for qb in range(nb)))
    bh = cfg.B * cfg.H
    f_sparse = 4.0 * d * pairs * bh
    f_calib = 4.0 * d * L * L * bh
    esize = 2 if cfg.dtype == "bf16" else 4
    # read Q, K, V, one of R (sparse reads it, calibration writes it), write O; rho is 4 bytes per row
    bytes_alg = bh * L * (5 * d * esize + 4)
    return f_sparse, f_calib, bytes_alg, pairs


def cpu_baseline(cfg, spec, inputs_host, lam, budget_s=20.0):
    """The CPU oracle's sparse step, timed on whole (batch, head) slices of the same workload."""
    import oracle
    from oracle import masks as om
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    mask = om.build_mask(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
    (q, k, v), rho, r = inputs_host
    heads_done, t_total = 0, 0.0
    bh_total = cfg.B * cfg.H
    while heads_done < bh_total and t_total < budget_s:
        b, h = divmod(heads_done, cfg.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        t0 = time.perf_counter()
        oracle.sparse_step(q[sl], k[sl], v[sl], mask, cfg.block, rho[sl], r[sl], lam, 1)
        t_total += time.perf_counter() - t0
        heads_done += 1
    f_head, _, _, _ = workload_counts(cfg, mask)
    f_head /= bh_total
    return {"value": f_head * heads_done / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle sparse step on {heads_done} of {bh_total} (batch, head) slices "
                      f"(all {cfg.L} rows each), {t_total:.1f} s; effective flops of the kept blocks / time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter scale reference) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the path needs no collective (every (batch, head) is "
              f"independent); --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b_ = torch.empty_like(a)
        for _ in range(3):
            b_.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_each_way": n * 4, "launches": 3}))
        return 0

    import sparse_attention_diffusion_block_amd as rt
    from workloads import CONFIGS, drift, make_qkv

    cfg = CONFIGS[args.config]
    spec = cfg.masks[0]
    T = cfg.sparse_steps
    lam = cfg.lam
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    rt.lib()

    log(f"generating inputs for {cfg.name} (B={cfg.B}, H={cfg.H}, L={cfg.L}, d={cfg.d})")
    host_sets = [make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, scale=cfg.input_scale, dtype=cfg.dtype)]
    for kstep in range(1, T + 1):
        host_sets.append(drift(*host_sets[-1], cfg.number, kstep, sigma=cfg.drift_sigma, scale=cfg.input_scale,
                               dtype=cfg.dtype))
    dev_sets = [tuple(torch.from_numpy(x).to("cuda").to(dt) for x in s) for s in host_sets]
    host_keep = host_sets[:2] if not args.no_cpu_baseline else None
    del host_sets

    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    o_cal = torch.empty((B, H, L, d), dtype=dt, device="cuda")
    r_cal = torch.empty_like(o_cal)
    rho = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    o_sp = torch.empty_like(o_cal)

    mask_np = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
    f_sparse, f_calib, bytes_alg, pairs = workload_counts(cfg, mask_np)

    ev = {"calibrate": [], "sparse": [], "index": []}

    def step(record):
        m = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record()
        idx = rt.index_build(m, cfg.block)
        if record:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record()
            ev["index"].append((e0, e1))
        q, k, v = dev_sets[0]
        if record:
            c0 = torch.cuda.Event(enable_timing=True)
            c0.record()
        rt.calibrate(q, k, v, idx, out=(o_cal, rho, r_cal))
        if record:
            c1 = torch.cuda.Event(enable_timing=True)
            c1.record()
            ev["calibrate"].append((c0, c1))
        for kstep in range(1, T + 1):
            q, k, v = dev_sets[kstep]
            if record:
                s0 = torch.cuda.Event(enable_timing=True)
                s0.record()
            rt.sparse(q, k, v, idx, rho, r_cal, lam=lam, step=kstep, out=o_sp)
            if record:
                s1 = torch.cuda.Event(enable_timing=True)
                s1.record()
                ev["sparse"].append((s0, s1))

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / max(args.steps, 1)

    def mean_ms(pairs_):
        return float(np.mean([a.elapsed_time(b) for a, b in pairs_])) if pairs_ else float("nan")

    sp_each = [a.elapsed_time(b) for a, b in ev["sparse"]]
    t_sp = mean_ms(ev["sparse"]) * 1e-3
    t_cal = mean_ms(ev["calibrate"]) * 1e-3
    t_idx = mean_ms(ev["index"]) * 1e-3
    sparse_tflops = f_sparse / t_sp / 1e12
    calib_tflops = f_calib / t_cal / 1e12
    sparse_gbs = bytes_alg / t_sp / 1e9
    calib_gbs = bytes_alg / t_cal / 1e9
    ai_sparse = f_sparse / bytes_alg
    ridge = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)

    from sparse_attention_diffusion_block_amd.profiling import kernel_source_hash, read_traffic
    traffic = read_traffic(os.path.join(ROOT, "profiles", f"hbm_traffic_{cfg.name}.txt"))

    def traffic_of(kernel):
        """Counter-measured HBM bytes per launch, if taken on the current source of the kernel."""
        sha, nbytes = traffic.get(kernel, (None, None))
        return nbytes if sha is not None and sha == kernel_source_hash(kernel) else None

    k_sparse, k_cal = "sparse64_kernel<64>", "calib_kernel<64, 64>"
    roof_sparse = {"bound": "hbm" if ai_sparse < ridge else "mfma",
                   "kernel": k_sparse,
                   "achieved": round(sparse_gbs, 1) if ai_sparse < ridge else round(sparse_tflops, 1),
                   "peak": HBM_PEAK_GBS if ai_sparse < ridge else MFMA_PEAK_TFLOPS,
                   "unit": "GB/s" if ai_sparse < ridge else "TFLOP/s",
                   "traffic": traffic_of(k_sparse),
                   "mfma_frac": round(sparse_tflops / MFMA_PEAK_TFLOPS, 4),
                   "ms": round(t_sp * 1e3, 4)}
    roof_sparse["frac"] = round(roof_sparse["achieved"] / roof_sparse["peak"], 4)
    roof_cal = {"bound": "mfma", "kernel": k_cal,
                "achieved": round(calib_tflops, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(calib_tflops / MFMA_PEAK_TFLOPS, 4), "traffic": traffic_of(k_cal),
                "ms": round(t_cal * 1e3, 4)}
    # the dominant kernel of a step is the one with the larger share of its time
    dominant_is_cal = t_cal > T * t_sp
    out = {
        "metric": "sparse-step ms + effective TFLOP/s at 96.9% sparsity, L=17776, H=30, d=64",
        "value": round(sparse_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic: Q,K,V ~ N(0,1) seeded, random-walk drift sigma 0.05",
        "config": {"workload": f"{cfg.name}: B={B} H={H} L={L} d={d} block={cfg.block}, "
                               f"mask {spec.label()} ({1 - pairs / (L * L):.4%} sparsity), "
                               f"1 calibration + {T} sparse steps per step, lambda={lam}",
                   "global_batch": B, "seq_len": L, "parallelism": "none (1 GPU)"},
        "sparse_step_ms": round(t_sp * 1e3, 4),
        "sparse_step_ms_p10_p50_p90": [round(float(np.percentile(sp_each, q)), 4) for q in (10, 50, 90)],
        # mean per launch by steps since the calibration (k = 1 runs right after the calibration)
        "sparse_step_ms_by_k": [round(float(np.mean(sp_each[j::T])), 4) for j in range(T)],
        "calibrate_ms": round(t_cal * 1e3, 4),
        "index_build_ms": round(t_idx * 1e3, 4),
        "sparse_effective_flops": f_sparse,
        "calibrate_flops": f_calib,
        "algorithmic_bytes_per_launch": bytes_alg,
        "roofline": roof_cal if dominant_is_cal else roof_sparse,
        "roofline_sparse": roof_sparse,
        "roofline_calibrate": roof_cal,
    }
    if not args.no_cpu_baseline:
        from workloads import make_cache
        rho_c, r_c = make_cache(B, H, L, d, seed=cfg.number, dtype=cfg.dtype)
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, spec, (host_keep[1], rho_c, r_c), lam)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
