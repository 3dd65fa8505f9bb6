"""Comparators of Re-ttention's statistical reshape, on the same GPU kernels.

The pages set Re-ttention against three ways of reusing attention across
denoising steps with a static sparse window (Re-ttention summary page,
"Approach" and "Surprising findings"; review thread, reply to W1 of the first
review on DiTFastAttn's residual):

    window         plain sparse attention: softmax over the kept keys only
    post_softmax   the kept keys' full-softmax probabilities, i.e. the window
                   output scaled by the denominator ratio rho, with no residual
                   (exact at a calibration step; at later steps rho is the
                   cached one, ramped like Re-ttention's)
    ditfastattn    window attention plus the difference (full minus window
                   attention) cached at the last full step

Each maps onto the library's two calls: window attention is rettn_sparse with
rho = 1, R = 0 and no ramp; post_softmax is rettn_sparse with R = 0;
DiTFastAttn's residual comes from rettn_calibrate_residual(DIFFERENCE) and its
step is rettn_sparse with rho = 1, R = that residual and no ramp.

    python -m sparse_attention_diffusion_block_amd.comparators --config 3 --T 5 --steps 10

runs one synthetic drift chain and reports, per step, every method's error
against true full attention on that step's inputs.
"""
import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METHODS = ("rettention", "window", "post_softmax", "ditfastattn")


def _ones_zeros(q):
    import torch
    B, H, L, d = q.shape
    return torch.ones((B, H, L), dtype=torch.float32, device=q.device), torch.zeros_like(q)


def window_attention(q, k, v, index, out=None):
    """softmax over the kept keys only (rows with no kept key give 0)."""
    from . import rettn as rt
    ones, zeros = _ones_zeros(q)
    return rt.sparse(q, k, v, index, ones, zeros, lam=0.0, step=1, out=out)


def post_softmax_step(q, k, v, index, rho, lam, step, out=None):
    """min(1, rho (1 + lam step)) * window attention, with no residual."""
    from . import rettn as rt
    _, zeros = _ones_zeros(q)
    return rt.sparse(q, k, v, index, rho, zeros, lam=lam, step=step, out=out)


def ditfastattn_calibrate(q, k, v, index):
    """Full step of DiTFastAttn: (O, residual = O - window attention)."""
    from . import rettn as rt
    o, _, r = rt.calibrate(q, k, v, index, residual="difference")
    return o, r


def ditfastattn_step(q, k, v, index, r_dfa, out=None):
    """Later step of DiTFastAttn: window attention + the cached difference."""
    from . import rettn as rt
    ones, _ = _ones_zeros(q)
    return rt.sparse(q, k, v, index, ones, r_dfa, lam=0.0, step=1, out=out)


def compare_chain(config=3, T=5, steps=10, sigma=None, lam=None, mask_index=0, log=None):
    """A synthetic drift chain through a T-periodic schedule, every method side by side.

    At calibration steps Re-ttention and post_softmax refresh rho (and Re-ttention R), and
    DiTFastAttn refreshes its difference residual; in between each reuses its cache.
    Every step's outputs are compared with true full attention on that step's inputs."""
    import torch
    from workloads import CONFIGS, drift, make_qkv
    from . import rettn as rt
    cfg = CONFIGS[config]
    spec = cfg.masks[mask_index]
    sigma = cfg.drift_sigma if sigma is None else sigma
    lam = cfg.lam if lam is None else lam
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    idx = rt.index_build(rt.mask_build(spec.kind, spec.nb, spec.w, spec.text_blocks, spec.tshift), cfg.block)
    host = make_qkv(cfg.B, cfg.H, cfg.L, cfg.d, cfg.seed, scale=cfg.input_scale, dtype=cfg.dtype)
    rho = r = r_dfa = None
    records = []
    for t in range(steps):
        if t > 0:
            host = drift(*host, cfg.number, t, sigma=sigma, dtype=cfg.dtype)
        q, k, v = (torch.from_numpy(x).to("cuda").to(dt) for x in host)
        full, rho_t, r_t = rt.calibrate(q, k, v, idx)
        kstep = t % T
        if kstep == 0:
            rho, r = rho_t, r_t
            _, r_dfa = ditfastattn_calibrate(q, k, v, idx)
            outs = {"rettention": full, "post_softmax": post_softmax_step(q, k, v, idx, rho, lam, 0),
                    "ditfastattn": full}
        else:
            outs = {"rettention": rt.sparse(q, k, v, idx, rho, r, lam=lam, step=kstep),
                    "post_softmax": post_softmax_step(q, k, v, idx, rho, lam, kstep),
                    "ditfastattn": ditfastattn_step(q, k, v, idx, r_dfa)}
        outs["window"] = window_attention(q, k, v, idx)
        fa = full.float()
        denom = fa.abs().sum().clamp_min(1e-30)
        rec = {"step": t, "k": kstep, "T": T, "sigma": sigma, "lambda": lam, "workload": cfg.name,
               "mask": spec.label()}
        for m in METHODS:
            dlt = (outs[m].float() - fa).abs()
            rec[f"{m}_rel_l1"] = round(float(dlt.sum() / denom), 6)
            rec[f"{m}_maxabs"] = round(float(dlt.max()), 6)
        records.append(rec)
        if log:
            log(rec)
    torch.cuda.synchronize()
    return records


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--T", type=int, default=5)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--sigma", type=float, default=None)
    ap.add_argument("--lam", type=float, default=None)
    args = ap.parse_args(argv)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    compare_chain(args.config, args.T, args.steps, args.sigma, args.lam,
                  log=lambda r: print(json.dumps(r), flush=True))
    return 0


if __name__ == "__main__":
    sys.exit(main())
