"""T-periodic Re-ttention schedule and per-layer cache of the reshape statistics.

Re-ttention (summary page, "Approach"; review thread, replies on the refresh
period) runs full attention once every T denoising steps and sparse attention in
between: the full ("calibration") step refreshes, per layer and per (batch,
head, query token), the denominator ratio rho and the residual R of the masked
tokens; the next T - 1 steps reuse that cache, ramping rho by lambda per step
since the refresh.  Nothing of the cache is updated at sparse steps.

    Schedule(T)          which steps calibrate; k = steps since the last refresh
    LayerCache           rho / R / k of one attention layer (device tensors)
    CacheManager         every layer's cache; state_dict / load_state_dict
                         checkpoint it to host memory and resume from it
    Rettention           one layer: call it once per denoising step with that
                         step's Q, K, V; it calibrates or runs the sparse step
    chained_drift_run    a synthetic chain of denoising steps (random-walk drift
                         of Q, K, V) through the schedule, reporting each step's
                         error against true full attention on the same inputs
    dynamic_mask_run     the same chain with a block mask recomputed from every
                         step's own Q and K, beside the static mask: how well the
                         cached rho and R still describe the step's own window

All computation goes through the C ABI (rettn_calibrate / rettn_sparse); this
module only orders the calls and owns the cache buffers.

    python -m sparse_attention_diffusion_block_amd.schedule --config 3 --T 5 --steps 15
    python -m sparse_attention_diffusion_block_amd.schedule --dynamic --config 3 --T 5 --steps 10
"""
import argparse
import json
import os
import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


class Schedule:
    """Calibrate at steps 0, T, 2T, ...; step t otherwise is sparse step k = t mod T (1 <= k < T)."""

    def __init__(self, T: int):
        if T < 1:
            raise ValueError("the refresh period T must be at least 1")
        self.T = T

    def is_calibration(self, t: int) -> bool:
        return t % self.T == 0

    def k(self, t: int) -> int:
        """Sparse steps since the last refresh (0 at a calibration step)."""
        return t % self.T


@dataclass
class LayerCache:
    """Reshape statistics of one attention layer, as of its last calibration."""
    rho: object = None          # float32 [B, H, L]
    R: object = None            # I/O dtype [B, H, L, d]
    refreshed_at: int = -1      # denoising step of the last calibration (-1: never)

    @property
    def valid(self) -> bool:
        return self.refreshed_at >= 0


class CacheManager:
    """One LayerCache per attention layer, allocated on first use and reused across steps."""

    def __init__(self):
        self.layers: Dict[int, LayerCache] = {}

    def get(self, layer: int) -> LayerCache:
        return self.layers.setdefault(layer, LayerCache())

    def nbytes(self) -> int:
        total = 0
        for c in self.layers.values():
            for t in (c.rho, c.R):
                if t is not None:
                    total += t.numel() * t.element_size()
        return total

    def state_dict(self) -> dict:
        """Host copies of every calibrated layer's cache: the method's only state carried from one
        denoising step to the next (rho, R and the step of the refresh).  Plain tensors keyed
        "<layer>.rho", "<layer>.R", "<layer>.refreshed_at", so torch.save / safetensors can store
        it and a later process can resume the schedule mid-period."""
        import torch
        out = {}
        for layer, c in sorted(self.layers.items()):
            if c.valid:
                out[f"{layer}.rho"] = c.rho.detach().cpu().contiguous()
                out[f"{layer}.R"] = c.R.detach().cpu().contiguous()
                out[f"{layer}.refreshed_at"] = torch.tensor(c.refreshed_at, dtype=torch.int64)
        return out

    def load_state_dict(self, state: dict, device="cuda") -> None:
        """Restore caches saved by state_dict onto `device` (bit for bit)."""
        layers = sorted({int(key.split(".", 1)[0]) for key in state})
        for layer in layers:
            c = self.get(layer)
            c.rho = state[f"{layer}.rho"].to(device).contiguous()
            c.R = state[f"{layer}.R"].to(device).contiguous()
            c.refreshed_at = int(state[f"{layer}.refreshed_at"])


class Rettention:
    """Re-ttention for one attention layer under a static block mask.

    Call once per denoising step t (in order) with that step's Q, K, V
    ([B, H, L, d], d contiguous).  Steps with t mod T == 0 run the calibration
    (full attention; refreshes the layer's rho and R); the others run the
    sparse step with k = t mod T.  Returns O for the step."""

    def __init__(self, index, schedule: Schedule, cache: CacheManager, layer: int = 0, lam: float = 0.04):
        self.index, self.schedule, self.cache, self.layer, self.lam = index, schedule, cache, layer, lam

    def __call__(self, t: int, q, k, v, out=None):
        from . import rettn as rt
        import torch
        c = self.cache.get(self.layer)
        if self.schedule.is_calibration(t):
            B, H, L, d = q.shape
            if c.rho is None or tuple(c.R.shape) != tuple(q.shape) or c.R.dtype != q.dtype:
                c.rho = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
                c.R = torch.empty_like(q)
            o = out if out is not None else torch.empty_like(q)
            rt.calibrate(q, k, v, self.index, out=(o, c.rho, c.R))
            c.refreshed_at = t
            return o
        if not c.valid or t - c.refreshed_at != self.schedule.k(t):
            raise RuntimeError(f"layer {self.layer}: sparse step {t} has no calibration at step "
                               f"{t - self.schedule.k(t)} to reuse")
        return rt.sparse(q, k, v, self.index, c.rho, c.R, lam=self.lam, step=self.schedule.k(t), out=out)


def _errors(g, ref):
    d = (g.float() - ref.float()).abs()
    return float(d.max()), float(d.sum() / ref.float().abs().sum().clamp_min(1e-30))


def chained_drift_run(config: int = 3, T: int = 5, steps: int = 15, layers: int = 1, sigma: Optional[float] = None,
                      lam: Optional[float] = None, mask_index: int = 0, log=None) -> List[dict]:
    """Run `steps` denoising steps of a synthetic drift chain through the T-periodic schedule.

    Step t's inputs are the workload's seeded Q, K, V after t random-walk drift steps (layer j
    uses seed offset 100 j).  At every step the true full attention on the same inputs is
    computed too (the calibration kernel is exact full attention), and the error of the
    step's output against it is reported."""
    import torch
    from workloads import CONFIGS, drift, make_qkv
    from . import rettn as rt
    cfg = CONFIGS[config]
    spec = cfg.masks[mask_index]
    sigma = cfg.drift_sigma if sigma is None else sigma
    lam = cfg.lam if lam is None else lam
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    idx = rt.index_build(rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift), cfg.block)
    sched, cache = Schedule(T), CacheManager()
    runs = [Rettention(idx, sched, cache, layer=j, lam=lam) for j in range(layers)]
    host = [make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed + 100 * j, scale=cfg.input_scale, dtype=cfg.dtype)
            for j in range(layers)]
    full_o = torch.empty((cfg.B, cfg.H, cfg.L, cfg.d), dtype=dt, device="cuda")
    full_rho = torch.empty((cfg.B, cfg.H, cfg.L), dtype=torch.float32, device="cuda")
    full_r = torch.empty_like(full_o)
    records = []
    for t in range(steps):
        for j in range(layers):
            if t > 0:
                host[j] = drift(*host[j], cfg.number + 100 * j, t, sigma=sigma, dtype=cfg.dtype)
            q, k, v = (torch.from_numpy(x).to("cuda").to(dt) for x in host[j])
            o = runs[j](t, q, k, v)
            rt.calibrate(q, k, v, idx, out=(full_o, full_rho, full_r))
            maxabs, rel = _errors(o, full_o)
            rec = {"step": t, "layer": j, "kind": "calibration" if sched.is_calibration(t) else "sparse",
                   "k": sched.k(t), "T": T, "sigma": sigma, "lambda": lam, "workload": cfg.name,
                   "mask": spec.label(), "maxabs_vs_full": round(maxabs, 6), "rel_l1_vs_full": round(rel, 6)}
            records.append(rec)
            if log:
                log(rec)
    torch.cuda.synchronize()
    return records


def dynamic_mask_run(config: int = 3, T: int = 5, steps: int = 10, keep: Optional[int] = None,
                     sigma: Optional[float] = None, lam: Optional[float] = None, log=None) -> List[dict]:
    """Re-ttention with a dynamic mask beside the workload's static mask, on one drift chain.

    The authors' trial of dynamic masks (review thread, answers to W2 and Q1 of the first
    review) found the denominator ratio still predictable but the cached residual wrong once the
    mask moves.  Per step and per mask kind this reports
      rel_l1_vs_full   the step's output against true full attention;
      rho_rel_err      the cached, ramped rho against the rho of the step's own window
                       (sum |rho~ - rho_t| / sum rho_t);
      r_rel_err        the cached R against the residual of the step's own window;
      mask_moved       the share of the step's kept blocks that the calibration's mask dropped.
    `keep` (blocks per row of the dynamic mask) defaults to the static mask's mean row count.
    At each step a calibration on that step's window gives the true values (it is exact full
    attention with that window's split); it is a measurement, not part of the method."""
    import torch
    from workloads import CONFIGS, drift, make_qkv
    from . import rettn as rt
    cfg = CONFIGS[config]
    spec = cfg.masks[0]
    sigma = cfg.drift_sigma if sigma is None else sigma
    lam = cfg.lam if lam is None else lam
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    static_mask = rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift)
    static = rt.index_build(static_mask, cfg.block)
    keep = int(round(static_mask.sum() / static_mask.shape[0])) if keep is None else keep
    sched = Schedule(T)
    records = []
    for kind in ("static", "dynamic"):
        host = make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, scale=cfg.input_scale, dtype=cfg.dtype)
        rho_c = r_c = idx_c = None
        for t in range(steps):
            if t > 0:
                host = drift(*host, cfg.number, t, sigma=sigma, dtype=cfg.dtype)
            q, k, v = (torch.from_numpy(x).to("cuda").to(dt) for x in host)
            idx = static if kind == "static" else rt.dynamic_index(q, k, keep, cfg.block)
            full, rho_t, r_t = rt.calibrate(q, k, v, idx)
            kstep = sched.k(t)
            if sched.is_calibration(t):
                rho_c, r_c, idx_c = rho_t, r_t, idx
                out = full
            else:
                out = rt.sparse(q, k, v, idx, rho_c, r_c, lam=lam, step=kstep)
            ramped = torch.clamp(rho_c * (1.0 + lam * kstep), max=1.0) if kstep else rho_c
            m_now, m_cal = idx.mask.bool(), idx_c.mask.bool()
            moved = float((m_now & ~m_cal).sum()) / max(float(m_now.sum()), 1.0)
            maxabs, rel = _errors(out, full)
            rec = {"mask_kind": kind, "step": t, "k": kstep, "T": T, "keep": keep if kind == "dynamic" else None,
                   "sigma": sigma, "lambda": lam, "workload": cfg.name,
                   "rel_l1_vs_full": round(rel, 6), "maxabs_vs_full": round(maxabs, 6),
                   "rho_rel_err": round(float((ramped - rho_t).abs().sum() / rho_t.abs().sum().clamp_min(1e-30)), 6),
                   "r_rel_err": round(float((r_c.float() - r_t.float()).abs().sum()
                                            / r_t.float().abs().sum().clamp_min(1e-30)), 6),
                   "mask_moved": round(moved, 6)}
            records.append(rec)
            if log:
                log(rec)
    torch.cuda.synchronize()
    return records


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--T", type=int, nargs="+", default=[5, 3, 7])
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--layers", type=int, default=1)
    ap.add_argument("--sigma", type=float, default=None)
    ap.add_argument("--lam", type=float, default=None)
    ap.add_argument("--dynamic", action="store_true", help="dynamic mask beside the static one")
    ap.add_argument("--keep", type=int, default=None, help="blocks per row of the dynamic mask")
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.dynamic:
        for T in args.T:
            dynamic_mask_run(args.config, T, args.steps, args.keep, args.sigma, args.lam,
                             log=lambda r: print(json.dumps(r), flush=True))
        return 0
    for T in args.T:
        chained_drift_run(args.config, T, args.steps, args.layers, args.sigma, args.lam,
                          log=lambda r: print(json.dumps(r), flush=True))
    return 0


if __name__ == "__main__":
    sys.exit(main())
