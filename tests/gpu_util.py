"""Helpers of the GPU parity tests: device transfer and the parity bar."""
import sys

import numpy as np

TOL_F32_MAXABS = 1e-4
TOL_BF16_MAXABS = 2e-2
TOL_BF16_REL_L1 = 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def dev(x, dtype):
    """Host float32 array (already representable in `dtype`) -> CUDA tensor of `dtype` (exact)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch_dtype(dtype))


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def errors(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    diff = np.abs(g - o)
    return float(diff.max()) if diff.size else 0.0, float(diff.sum() / max(np.abs(o).sum(), 1e-300))


def assert_parity(g, o, dtype, what, rel_l1=TOL_BF16_REL_L1):
    """fp32: max-abs <= 1e-4.  bf16: max-abs <= 2e-2 and relative L1 (sum|g-o| / sum|o|) <= 2e-3."""
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    maxabs, rel = errors(g, o)
    log(f"  {what}: max-abs {maxabs:.3e}  rel-L1 {rel:.3e}")
    if dtype == "f32":
        assert maxabs <= TOL_F32_MAXABS, f"{what}: max-abs {maxabs:.3e} > {TOL_F32_MAXABS}"
    else:
        assert maxabs <= TOL_BF16_MAXABS, f"{what}: max-abs {maxabs:.3e} > {TOL_BF16_MAXABS}"
        assert rel <= rel_l1, f"{what}: rel-L1 {rel:.3e} > {rel_l1}"
