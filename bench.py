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
the whole period.  `roofline` describes that sparse-step kernel (HBM-bound at
its arithmetic intensity); `roofline_calibrate` the calibration kernel.

After the timed steps (outside the timed region) the line also carries:
  sweep_c3        the sparse step on the same shapes under band masks of 75 /
                  87.5 / 93.8 / 96.9% block sparsity and the video mask, and
                  the 87.5% -> 96.9% speedup (the pages claim more than 2x);
  workloads       calibration and sparse-step times of the other workloads
                  (the image workloads warm and after a 512 MiB cache flush;
                  the long-video workload at its four windows);
  stream_floor    the time in which a plain streaming kernel (the in-tree probe
                  `probe_stream`, non-temporal loads and stores, last-level cache
                  evicted) moves the sparse step's traffic on the same device,
                  and the sparse step's fraction of that rate;
  cpu_baseline    the CPU oracle's sparse step on the same workload, timed on
                  the host cores (float32 and float64 modes, a process pool over
                  (batch, head) slices with one BLAS thread per process).

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extras]
"""
import argparse
import json
import os
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix peak, TFLOP/s
POOL_MAX = 16                  # worker processes for the CPU baseline (the host share of one GPU)


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


# ------------------------------------------------------------------ CPU baseline (the oracle)
_SHARED = {}


def _cpu_worker_init(names, meta):
    """Attach the workload's arrays from shared memory (no copy) and pin BLAS to one thread."""
    from multiprocessing import shared_memory
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    for key, name in names.items():
        shape, dtype = meta[key]
        shm = shared_memory.SharedMemory(name=name)
        _SHARED[key] = (shm, np.ndarray(shape, dtype=dtype, buffer=shm.buf))


def _cpu_worker(task):
    """The oracle's sparse step on one (batch, head) slice; returns its compute seconds."""
    import oracle
    b, h, block, lam, dtype = task
    a = {key: val[1] for key, val in _SHARED.items()}
    sl = (slice(b, b + 1), slice(h, h + 1))
    t0 = time.perf_counter()
    oracle.sparse_step(a["q"][sl], a["k"][sl], a["v"][sl], a["mask"], block, a["rho"][sl], a["r"][sl], lam, 1,
                       dtype=np.dtype(dtype))
    return time.perf_counter() - t0


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, spec, q, k, v, rho, r, lam):
    """The CPU oracle's sparse step on every (batch, head) slice of the workload, timed in float32 (the
    baseline) and float64 (the parity mode): a spawned process pool over the slices, one BLAS thread
    per process, inputs shared with the workers through shared memory; whole-workload wall time,
    median of 3 runs (1 if one run exceeds 60 s)."""
    import multiprocessing as mp
    from multiprocessing import shared_memory
    from oracle import masks as om
    mask = om.build_mask(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, POOL_MAX))
    f_sparse, _, _, _ = workload_counts(cfg, mask)
    out = {"unit": "TFLOP/s", "cores": workers, "kind": "oracle", "cpu_model": _cpu_model(),
           "host_threads_available": affinity}
    arrays = {"q": q, "k": k, "v": v, "rho": rho, "r": r, "mask": mask}
    shms, names, meta = [], {}, {}
    saved_env = {key: os.environ.get(key) for key in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    try:
        for key, arr in arrays.items():
            arr = np.ascontiguousarray(arr)
            shm = shared_memory.SharedMemory(create=True, size=max(arr.nbytes, 1))
            shms.append(shm)
            np.ndarray(arr.shape, dtype=arr.dtype, buffer=shm.buf)[...] = arr
            names[key], meta[key] = shm.name, (arr.shape, arr.dtype.str)
        for key in saved_env:
            os.environ[key] = "1"                     # the spawned workers start with one BLAS thread
        ctx = mp.get_context("spawn")
        with ctx.Pool(workers, initializer=_cpu_worker_init, initargs=(names, meta)) as pool:
            for dtype in ("float32", "float64"):
                tasks = [(b, h, cfg.block, lam, dtype) for b in range(cfg.B) for h in range(cfg.H)]
                pool.map(_cpu_worker, tasks[:workers], chunksize=1)          # warm the workers (imports)
                walls = []
                for _ in range(3):
                    t0 = time.perf_counter()
                    pool.map(_cpu_worker, tasks, chunksize=1)
                    walls.append(time.perf_counter() - t0)
                    if walls[-1] > 60.0:
                        break
                wall = float(np.median(walls))
                out[dtype] = {"value": round(f_sparse / wall / 1e12, 6), "seconds": round(wall, 3),
                              "runs": len(walls)}
    finally:
        for key, val in saved_env.items():
            if val is None:
                os.environ.pop(key, None)
            else:
                os.environ[key] = val
        for shm in shms:
            shm.close()
            shm.unlink()
    out["value"] = out["float32"]["value"]
    out["sample"] = (f"the oracle's sparse step (float32 mode; float64 beside it) on all {cfg.B * cfg.H} (batch, head) "
                     f"slices, all {cfg.L} rows each, of the timed workload; {workers} spawned processes with one BLAS "
                     f"thread each; whole-workload wall time, median of {out['float32']['runs']}; effective flops of "
                     f"the kept blocks / time")
    return out


# ------------------------------------------------------------------ timed extras (outside the timed region)
def _gpu_inputs(cfg, seed):
    """Seeded N(0,1) Q, K, V drawn on the device (timing only: the workload's shapes and distribution)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    shape = (cfg.B, cfg.H, cfg.L, cfg.d)
    return tuple((torch.randn(shape, generator=g, device="cuda", dtype=torch.float32) * cfg.input_scale).to(dt)
                 for _ in range(3))


def _sparse_rec(rt, timer, cfg, spec, qkv, rho, r, runs, before=None):
    from sparse_attention_diffusion_block_amd.measure import _counts
    import torch
    m = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
    idx = rt.index_build(m, cfg.block)
    f_sp, _, nbytes, pairs = _counts(cfg, m)
    out = torch.empty_like(qkv[0])
    t = timer(lambda: rt.sparse(*qkv, idx, rho, r, lam=cfg.lam, step=1, out=out), runs, before=before)
    s = t["median_ms"] * 1e-3
    return {"mask": spec.label(), "token_sparsity": round(1.0 - pairs / (cfg.L * cfg.L), 5), "ms": t["median_ms"],
            "p10_p90_ms": [t["p10_ms"], t["p90_ms"]], "effective_tflops": round(f_sp / s / 1e12, 1),
            "algorithmic_gbs": round(nbytes / s / 1e9, 1)}


def _calib_rec(rt, timer, cfg, spec, qkv, runs, before=None):
    from sparse_attention_diffusion_block_amd.measure import _counts
    import torch
    m = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
    idx = rt.index_build(m, cfg.block)
    _, f_cal, _, _ = _counts(cfg, m)
    q = qkv[0]
    o, rr = torch.empty_like(q), torch.empty_like(q)
    rho = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    t = timer(lambda: rt.calibrate(*qkv, idx, out=(o, rho, rr)), runs, warm=2 if cfg.number == 5 else 10,
              before=before)
    s = t["median_ms"] * 1e-3
    return {"mask": spec.label(), "ms": t["median_ms"], "tflops": round(f_cal / s / 1e12, 1),
            "mfma_frac": round(f_cal / s / 1e12 / MFMA_PEAK_TFLOPS, 4)}


def extras(rt, c3_sets, rho_c3, r_c3):
    """Per-workload timings and the density sweep (HIP events, median of batched calls)."""
    import torch
    from sparse_attention_diffusion_block_amd.measure import _time
    from workloads import CONFIGS, SWEEP_C3
    out = {}
    cfg3 = CONFIGS[3]
    log("extras: density sweep on the video workload's shapes")
    recs = [_sparse_rec(rt, _time, cfg3, spec, c3_sets[1], rho_c3, r_c3, 20) for spec in SWEEP_C3 + cfg3.masks]
    t875 = recs[1]["ms"]
    t969 = recs[3]["ms"]
    out["sweep_c3"] = {"records": recs, "speedup_96.9_over_87.5": round(t875 / t969, 3),
                       "note": "band windows of 70 / 35 / 17 / 9 of 278 blocks, then the 3D window + text mask; "
                               "the pages report more than 2x for 87.5% -> 96.9%"}
    flush = torch.empty(512 << 18, dtype=torch.float32, device="cuda")          # 512 MiB
    wl = {}
    for n in (1, 2, 4, 5):
        cfg = CONFIGS[n]
        log(f"extras: workload {n} ({cfg.name})")
        qkv = _gpu_inputs(cfg, 100 + n)
        qkv2 = _gpu_inputs(cfg, 200 + n)
        g = torch.Generator(device="cuda")
        g.manual_seed(300 + n)
        rho = torch.rand(qkv[0].shape[:3], generator=g, device="cuda") * 0.98 + 0.01
        r = (torch.randn(qkv[0].shape, generator=g, device="cuda") * 0.05).to(qkv[0].dtype)
        timings = [("warm", None)] + ([("cold", lambda: flush.zero_())] if n in (2, 4) else [])
        runs = 5 if n == 5 else 20
        rec = {"shape": f"B={cfg.B} H={cfg.H} L={cfg.L} d={cfg.d} block={cfg.block} {cfg.dtype}", "masks": []}
        for spec in cfg.masks:
            m = {"mask": spec.label()}
            for label, before in timings:
                if n != 5 or spec is cfg.masks[0]:
                    m[f"calibrate_{label}"] = _calib_rec(rt, _time, cfg, spec, qkv, 3 if n == 5 else runs, before)
                m[f"sparse_{label}"] = _sparse_rec(rt, _time, cfg, spec, qkv2, rho, r, runs, before)
            rec["masks"].append(m)
        wl[cfg.name] = rec
        del qkv, qkv2, rho, r
        torch.cuda.empty_cache()
    out["workloads"] = wl
    out["extras_note"] = ("HIP events around 5 back-to-back calls (one more queued in front), median of the samples; "
                          "cold: a 512 MiB buffer is written before every single call; inputs drawn on the device "
                          "with the workloads' shapes and N(0,1) values")
    return out


def stream_floor(sparse_ms, bytes_alg):
    """The streaming probe's four-read/one-write mix (the sparse step's traffic, one 136.5 MB tensor per
    stream), run as a child process after the timed region; its best time scaled to the step's
    algorithmic bytes is the floor for moving them.  A missing or failing probe is reported, not fatal."""
    exe = os.path.join(ROOT, "sparse_attention_diffusion_block_amd", "probe_stream")
    if not os.path.exists(exe):
        return {"error": "probe_stream is not built"}
    try:
        p = subprocess.run([exe, "--mix-json"], capture_output=True, text=True, timeout=120)
        rec = json.loads(p.stdout.strip().splitlines()[-1])
    except Exception as e:                      # noqa: BLE001 - reported in the line
        return {"error": f"probe_stream: {e}"[:200]}
    floor_ms = rec["best_us"] * 1e-3 * bytes_alg / rec["bytes"]
    return {"probe": rec, "floor_ms": round(floor_ms, 4), "sparse_step_ms": round(sparse_ms, 4),
            "sparse_frac_of_floor": round(floor_ms / sparse_ms, 4)}


def copy_bandwidth():
    """Measured read + write rate of a plain 1 GiB device copy (the streaming ceiling of this chip)."""
    import torch
    from sparse_attention_diffusion_block_amd.measure import _time
    x = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    t = _time(lambda: y.copy_(x), 10)
    return 2.0 * (1 << 30) / (t["median_ms"] * 1e-3) / 1e9


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
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
    from sparse_attention_diffusion_block_amd.profiling import dispatched_kernels, kernel_source_hash, read_traffic
    from workloads import CONFIGS, drift, make_cache, make_qkv

    cfg = CONFIGS[args.config]
    spec = cfg.masks[0]
    T = cfg.sparse_steps
    lam = cfg.lam
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    rt.lib()

    log(f"generating inputs for {cfg.name} (B={cfg.B}, H={cfg.H}, L={cfg.L}, d={cfg.d})")
    host_sets = [make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, scale=cfg.input_scale, dtype=cfg.dtype)]
    for kstep in range(1, T + 1):
        host_sets.append(drift(*host_sets[-1], cfg.number, kstep, sigma=cfg.drift_sigma,
                               dtype=cfg.dtype))
    dev_sets = [tuple(torch.from_numpy(x).to("cuda").to(dt) for x in s) for s in host_sets]
    host_keep = host_sets[1] if not args.no_cpu_baseline else None
    del host_sets

    B, H, L, d = cfg.B, cfg.H, cfg.L, cfg.d
    o_cal = torch.empty((B, H, L, d), dtype=dt, device="cuda")
    r_cal = torch.empty_like(o_cal)
    rho = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    o_sp = torch.empty_like(o_cal)
    # the calibration's device workspace (V in float16), allocated once like the outputs
    ws_cal = torch.empty(max(rt.calibrate_workspace_bytes(o_cal, cfg.block), 1), dtype=torch.uint8, device="cuda")

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
        rt.calibrate(q, k, v, idx, out=(o_cal, rho, r_cal), workspace=ws_cal)
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
    ai_sparse = f_sparse / bytes_alg
    ridge = MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    copy_gbs = copy_bandwidth()

    traffic = read_traffic(os.path.join(ROOT, "profiles", f"hbm_traffic_{cfg.name}.txt"))

    def traffic_of(kernel):
        """Counter-measured HBM bytes per launch, if taken on the current source of the kernel."""
        sha, nbytes = traffic.get(kernel, (None, None))
        return nbytes if sha is not None and sha == kernel_source_hash(kernel) else None

    k_cal, k_sparse = dispatched_kernels(cfg.dtype, cfg.block, cfg.d, cfg.L)
    hbm_bound = ai_sparse < ridge
    roof_sparse = {"bound": "hbm" if hbm_bound else "mfma",
                   "kernel": k_sparse,
                   "achieved": round(sparse_gbs, 1) if hbm_bound else round(sparse_tflops, 1),
                   "peak": HBM_PEAK_GBS if hbm_bound else MFMA_PEAK_TFLOPS,
                   "unit": "GB/s" if hbm_bound else "TFLOP/s",
                   "traffic": traffic_of(k_sparse),
                   "mfma_frac": round(sparse_tflops / MFMA_PEAK_TFLOPS, 4),
                   "measured_copy_gbs": round(copy_gbs, 1),
                   "frac_of_measured_copy": round(sparse_gbs / copy_gbs, 4),
                   "ms": round(t_sp * 1e3, 4)}
    roof_sparse["frac"] = round(roof_sparse["achieved"] / roof_sparse["peak"], 4)
    roof_cal = {"bound": "mfma", "kernel": k_cal,
                "note": "ms and achieved cover the whole call: one pass converting V to float16 into the "
                        "workspace (v16_kernel), then the calibration kernel" if "true>" in k_cal and "calib" in k_cal
                        else "ms and achieved cover the whole call",
                "achieved": round(calib_tflops, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(calib_tflops / MFMA_PEAK_TFLOPS, 4), "traffic": traffic_of(k_cal),
                "ms": round(t_cal * 1e3, 4)}
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
                   "precision": "bf16 I/O, bf16 QK^T, fp16 P*V, fp32 accumulation and softmax" if cfg.dtype == "bf16"
                                else "fp32 throughout",
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
        "roofline": roof_sparse,
        "roofline_calibrate": roof_cal,
    }
    if not args.no_extras and args.config == 3:
        out.update(extras(rt, dev_sets, rho, r_cal))
        log("extras: streaming floor (probe_stream)")
        out["stream_floor"] = stream_floor(t_sp * 1e3, bytes_alg)
    if not args.no_cpu_baseline:
        rho_c, r_c = make_cache(B, H, L, d, seed=cfg.number, dtype=cfg.dtype)
        log("timing the CPU oracle (float32 and float64 modes)")
        q1, k1, v1 = host_keep
        out["cpu_baseline"] = cpu_baseline(cfg, spec, q1, k1, v1, rho_c, r_c, lam)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
