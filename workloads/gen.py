"""Seeded input generation.

Q, K, V are drawn from numpy's PCG64 generator in the order Q, K, V, in
float32, then rounded to bfloat16 (round to nearest, ties to even) for
bfloat16 workloads, so the GPU and the oracle consume identical bits.
Drift between denoising steps is a random walk X_k = X_{k-1} + sigma * eps_k
with a fresh draw per tensor and step (seed 1000 * config + k).
"""
import numpy as np


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to the nearest bfloat16 (ties to even); returns a new float32 array."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    if not np.isfinite(x).all():
        raise ValueError("bf16_round expects finite values")
    u = x.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return x


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bfloat16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _draw(rng, shape, scale):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def make_qkv(B, H, L, d, seed, scale=1.0, dtype="bf16"):
    """Base Q, K, V (float32 arrays holding values representable in `dtype`)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, L, d)
    q, k, v = (_draw(rng, shape, scale) for _ in range(3))
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    return q, k, v


def drift(q, k, v, config_number, step, sigma=0.05, scale=1.0, dtype="bf16"):
    """One random-walk drift step applied to float32 Q, K, V (values of the previous step)."""
    rng = np.random.Generator(np.random.PCG64(1000 * config_number + step))
    out = []
    for x in (q, k, v):
        y = (x + _draw(rng, x.shape, sigma * scale)).astype(np.float32)
        out.append(bf16_round(y) if dtype == "bf16" else y)
    return tuple(out)


def sample_rows(L, block, n, seed):
    """Query rows to check at full size: the first and last rows, block edges and a seeded sample."""
    rng = np.random.Generator(np.random.PCG64(seed + 77))
    fixed = {0, 1, L - 1, L - 2, min(block, L - 1), min(block - 1, L - 1)}
    last_block_start = ((L - 1) // block) * block
    fixed.update({last_block_start, max(last_block_start - 1, 0)})
    rest = rng.choice(L, size=min(n, L), replace=False)
    return np.array(sorted(fixed.union(int(x) for x in rest)), dtype=np.int64)


def make_cache(B, H, L, d, seed, dtype="bf16"):
    """A synthetic (rho, R) cache: rho ~ U(0.01, 0.99) float32, R ~ N(0, 0.05^2) in `dtype`.

    Any rho in [0, 1] and any R are valid inputs of a sparse step, so the
    sparse step can be checked at full size without a full calibration.
    """
    rng = np.random.Generator(np.random.PCG64(seed + 5000))
    rho = rng.uniform(0.01, 0.99, size=(B, H, L)).astype(np.float32)
    r = _draw(rng, (B, H, L, d), 0.05)
    if dtype == "bf16":
        r = bf16_round(r)
    return rho, r


def random_mask(nqb, nkb, density, seed, empty_rows=()):
    """A seeded random 0/1 block mask (test input), optionally with rows forced empty."""
    rng = np.random.Generator(np.random.PCG64(seed + 9000))
    m = (rng.random((nqb, nkb)) < density).astype(np.uint8)
    for r in empty_rows:
        m[r, :] = 0
    return m
